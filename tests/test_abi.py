"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import gated_deltanet_recurrence_delta_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, INVALID, UNSUPPORTED, LAUNCH = 0, -1, -2, -3
# Non-null dummy host addresses: validation never dereferences them.
P = 0x1000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


def test_header_declares_entry_points():
    assert _declared_functions() == ["gdn_bwd", "gdn_bwd_noalloc", "gdn_bwd_saved", "gdn_bwd_workspace_size",
                                     "gdn_diag_fwd", "gdn_diag_fwd_recurrent", "gdn_fwd", "gdn_fwd_recurrent",
                                     "gdn_fwd_scan", "gdn_fwd_scan_workspace_size", "gdn_fwd_train",
                                     "gdn_strerror", "gdn_version"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gdn.lib_path())
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strerror():
    assert gdn.version() == 300
    for code in (OK, INVALID, UNSUPPORTED, LAUNCH, -4, 12345):
        assert isinstance(gdn.strerror(code), str) and gdn.strerror(code)


def _call(**kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, h0=0, cu_seqlens=0, out=P, hT=P,
             B=1, T=8, H=1, dk=32, dv=32, stream=None, dtype=1, chunk=64, flags=0)
    a.update(kw)
    return gdn.gdn_fwd(**a)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "out", "hT"])
def test_null_required_pointer(name):
    assert _call(**{name: 0}) == INVALID


@pytest.mark.parametrize("kw", [dict(B=-1), dict(T=-1), dict(H=0), dict(dk=0), dict(dv=-4),
                                dict(dtype=2), dict(dtype=-1), dict(chunk=48), dict(chunk=128),
                                dict(chunk=-64), dict(flags=2), dict(flags=-1), dict(flags=3)])
def test_invalid_sizes(kw):
    assert _call(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(dk=16), dict(dv=256), dict(dk=96), dict(dtype=1, chunk=16),
                                dict(dtype=0, chunk=64, dk=128), dict(dtype=0, chunk=64, dk=32)])
def test_unsupported(kw):
    assert _call(**kw) == UNSUPPORTED


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "out"])
def test_token_pointers_may_be_null_without_tokens(name):
    # No chains (B == 0) and no tokens: success without a launch.
    assert _call(**{name: 0, "T": 0, "B": 0, "hT": 0}) == OK


def test_state_pointer_required_with_chains():
    assert _call(hT=0, T=0) == INVALID


def test_empty_batch_is_a_no_op():
    # B == 0: nothing to launch, nothing touched, success.
    assert _call(B=0) == OK
    assert _call(B=0, cu_seqlens=P, T=0) == OK


def test_python_wrapper_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 1, 32)
    g = torch.zeros(1, 4, 1)
    with pytest.raises(ValueError):
        gdn.fwd(q, q, q, g, g)


# ------------------------------------------------------ chunk-map scan --

def _call_scan(**kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, h0=0, cu_seqlens=0, out=P, hT=P,
             B=1, T=4096, H=2, dk=128, dv=128, stream=None, dtype=1, chunk=64,
             workspace=P, workspace_bytes=1 << 40)
    a.update(kw)
    return gdn.gdn_fwd_scan(**a)


def test_scan_workspace_size():
    MAT = 128 * 128 * 4
    # a dense 4,096-token sequence is cut into 4 segments: 4 slots x H x (P, Q, S)
    assert gdn.gdn_fwd_scan_workspace_size(1, 4096, 2, 128, 128, 0, 1, 64) == 4 * 2 * 3 * MAT
    assert gdn.gdn_fwd_scan_workspace_size(3, 4096, 2, 128, 128, 0, 1, 0) == 3 * 4 * 2 * 3 * MAT
    # 17 chunks: 2 segments of 9 and 8 chunks
    assert gdn.gdn_fwd_scan_workspace_size(1, 1025, 1, 128, 128, 0, 1, 64) == 2 * 3 * MAT
    # packed: floor(T / 1024) + B slots
    assert gdn.gdn_fwd_scan_workspace_size(5, 5000, 1, 128, 128, 1, 1, 64) == (4 + 5) * 3 * MAT
    # nothing is cut at or below 16 chunks, and other shapes never use it
    assert gdn.gdn_fwd_scan_workspace_size(8, 1024, 16, 128, 128, 0, 1, 64) == 0
    assert gdn.gdn_fwd_scan_workspace_size(8, 1024, 16, 128, 128, 1, 1, 64) == 0
    assert gdn.gdn_fwd_scan_workspace_size(1, 4096, 2, 32, 32, 0, 1, 64) == 0
    assert gdn.gdn_fwd_scan_workspace_size(1, 4096, 2, 128, 128, 0, 1, 32) == 0
    assert gdn.gdn_fwd_scan_workspace_size(1, 4096, 2, 128, 128, 0, 0, 32) == 0
    assert gdn.gdn_fwd_scan_workspace_size(-1, 4096, 2, 128, 128, 0, 1, 64) == INVALID
    assert gdn.gdn_fwd_scan_workspace_size(1, 4096, 0, 128, 128, 0, 1, 64) == INVALID


@pytest.mark.parametrize("kw", [dict(workspace=0), dict(workspace_bytes=4 * 2 * 3 * 65536 - 1),
                                dict(workspace=P + 4), dict(workspace_bytes=-1)])
def test_scan_rejects_bad_workspace(kw):
    assert _call_scan(**kw) == INVALID


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "out", "hT"])
def test_scan_null_required_pointer(name):
    assert _call_scan(**{name: 0}) == INVALID


@pytest.mark.parametrize("kw", [dict(B=-1), dict(H=0), dict(dtype=2), dict(chunk=48)])
def test_scan_invalid_sizes(kw):
    assert _call_scan(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(dk=16), dict(dtype=0, chunk=64)])
def test_scan_unsupported(kw):
    assert _call_scan(**kw) == UNSUPPORTED


def test_scan_no_chains_is_a_no_op():
    assert _call_scan(B=0, workspace=0, workspace_bytes=0) == OK


# -------------------------------------------------- token-by-token entry --

def _call_rec(**kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, h0=0, cu_seqlens=0, out=P, hT=P,
             B=1, T=8, H=1, dk=32, dv=32, stream=None, dtype=1)
    a.update(kw)
    return gdn.gdn_fwd_recurrent(**a)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "out", "hT"])
def test_recurrent_null_required_pointer(name):
    assert _call_rec(**{name: 0}) == INVALID


@pytest.mark.parametrize("kw", [dict(B=-1), dict(T=-1), dict(H=0), dict(dk=0), dict(dv=-4),
                                dict(dtype=2), dict(dtype=-1)])
def test_recurrent_invalid_sizes(kw):
    assert _call_rec(**kw) == INVALID


def test_token_rows_fit_32_bits():
    assert _call(B=1 << 16, T=1 << 15) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(dk=16), dict(dv=256), dict(dk=96), dict(dv=48)])
def test_recurrent_unsupported(kw):
    assert _call_rec(**kw) == UNSUPPORTED


def test_recurrent_no_chains_is_a_no_op():
    assert _call_rec(B=0) == OK
    assert _call_rec(B=0, T=0, q=0, k=0, v=0, g=0, beta=0, out=0, hT=0) == OK
    assert _call_rec(hT=0, T=0) == INVALID


# ------------------------------------------- diagonal-decay additive form ---

def _diag_args(**kw):
    a = dict(v=P, b=P, c=P, g=P, A_log=P, Dskip=0, gate=0, h0=0, cu_seqlens=0, out=P, hT=P,
             B=2, T=64, H=3, S=32, D=32, stream=0, dtype=1)
    a.update(kw)
    return a


def _call_diag(chunk=0, **kw):
    return gdn.gdn_diag_fwd(**_diag_args(**kw), chunk=chunk)


def _call_diag_rec(**kw):
    return gdn.gdn_diag_fwd_recurrent(**_diag_args(**kw))


@pytest.mark.parametrize("call", [_call_diag, _call_diag_rec])
@pytest.mark.parametrize("name", ["v", "b", "c", "g", "A_log", "out", "hT"])
def test_diag_null_required_pointer(call, name):
    assert call(**{name: 0}) == INVALID


@pytest.mark.parametrize("call", [_call_diag, _call_diag_rec])
@pytest.mark.parametrize("kw", [dict(B=-1), dict(T=-1), dict(H=0), dict(S=0), dict(D=-4),
                                dict(dtype=2), dict(dtype=-1)])
def test_diag_invalid_sizes(call, kw):
    assert call(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(S=8), dict(D=256), dict(S=48), dict(D=96)])
def test_diag_recurrent_unsupported(kw):
    assert _call_diag_rec(**kw) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(dtype=0), dict(S=64), dict(D=16), dict(chunk=32),
                                dict(chunk=16), dict(T=1 << 20, H=64)])
def test_diag_chunked_unsupported(kw):
    assert _call_diag(**kw) == UNSUPPORTED


def test_diag_no_chains_is_a_no_op():
    for call in (_call_diag, _call_diag_rec):
        assert call(B=0) == OK
        assert call(B=0, T=0, v=0, b=0, c=0, g=0, A_log=0, out=0, hT=0) == OK
        assert call(hT=0, T=0) == INVALID


# ------------------------------------------------------------- backward ---

def _ws_floats(ttot, B, H, dk, dv):
    nslots = ttot // 32 + B + 1
    return H * nslots * (2 * 32 * 32 + 2 * dk * dv)


@pytest.mark.parametrize("B,T,H,dk,dv,packed", [(4, 4096, 16, 128, 128, 0), (1, 1, 1, 32, 32, 0),
                                                (3, 100, 2, 64, 32, 1), (2, 0, 3, 32, 64, 0)])
def test_bwd_workspace_size(B, T, H, dk, dv, packed):
    ttot = T if packed else B * T
    assert gdn.gdn_bwd_workspace_size(B, T, H, dk, dv, packed) == 4 * _ws_floats(ttot, B, H, dk, dv)


@pytest.mark.parametrize("kw,code", [(dict(B=-1), INVALID), (dict(H=0), INVALID),
                                     (dict(dk=48), UNSUPPORTED), (dict(dv=256), UNSUPPORTED),
                                     (dict(H=70000), UNSUPPORTED),
                                     (dict(B=70000, T=70000), INVALID)])
def test_bwd_workspace_size_rejects(kw, code):
    a = dict(B=1, T=8, H=1, dk=32, dv=32, packed=0)
    a.update(kw)
    assert gdn.gdn_bwd_workspace_size(**a) == code


def _bcall(**kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, h0=0, cu_seqlens=0, dout=P, dhT=0, dq=P, dk=P, dv=P,
             dg=P, dbeta=P, dh0=0, workspace=P, workspace_bytes=1 << 40, B=1, T=8, H=1, dk_=32,
             dv_=32, stream=None, dtype=1)
    a.update(kw)
    return gdn.gdn_bwd(**a)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "dout", "dq", "dk", "dv", "dg",
                                  "dbeta", "workspace"])
def test_bwd_null_required_pointer(name):
    assert _bcall(**{name: 0}) == INVALID


@pytest.mark.parametrize("kw,code", [(dict(B=-1), INVALID), (dict(T=-1), INVALID),
                                     (dict(H=0), INVALID), (dict(dtype=2), INVALID),
                                     (dict(dk_=16), UNSUPPORTED), (dict(dv_=96), UNSUPPORTED),
                                     (dict(H=70000), UNSUPPORTED),
                                     (dict(workspace_bytes=-1), INVALID),
                                     (dict(workspace=P + 2), INVALID),
                                     (dict(workspace_bytes=4 * _ws_floats(8, 1, 1, 32, 32) - 1),
                                      INVALID)])
def test_bwd_invalid(kw, code):
    assert _bcall(**kw) == code


def test_bwd_exact_workspace_accepted_without_launch():
    """The exact workspace size passes validation; B = 0 launches nothing."""
    need = gdn.gdn_bwd_workspace_size(0, 8, 1, 32, 32, 0)
    assert _bcall(B=0, workspace_bytes=need) == OK


# -------------------------------------------- training forward / saved bwd --

def _tcall(**kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, h0=0, cu_seqlens=0, out=P, hT=P, B=1, T=8, H=1, dk=128,
             dv=128, stream=None, dtype=1, chunk=0, workspace=P, workspace_bytes=1 << 40)
    a.update(kw)
    return gdn.gdn_fwd_train(**a)


def test_fwd_train_only_for_the_full_width_shapes():
    """Records exist for bf16 with dk = dv = 128 and 64-token chunks only;
    every other valid request is refused before anything is launched."""
    assert _tcall(dtype=0, chunk=16) == UNSUPPORTED
    assert _tcall(dk=64, dv=64) == UNSUPPORTED
    assert _tcall(chunk=32) == UNSUPPORTED
    assert _tcall(B=0) == OK


# (parameters hold no library calls: nothing may load libgdn.so while the
# tests are collected, before torch has brought up its HIP runtime)
@pytest.mark.parametrize("kw,code", [(dict(q=0), INVALID), (dict(hT=0), INVALID), (dict(B=-1), INVALID),
                                     (dict(workspace=0), INVALID), (dict(workspace=P + 8), INVALID),
                                     (dict(workspace_bytes="one short"), INVALID), (dict(chunk=48), INVALID)])
def test_fwd_train_rejects(kw, code):
    if kw.get("workspace_bytes") == "one short":
        kw = dict(kw, workspace_bytes=gdn.gdn_bwd_workspace_size(1, 8, 1, 128, 128, 0) - 1)
    assert _tcall(**kw) == code


def test_bwd_saved_only_for_the_full_width_shapes():
    a = dict(dk_=128, dv_=128, workspace_bytes=1 << 40)
    assert gdn.gdn_bwd_saved(**{**_bargs(), **a, "dtype": 0}) == UNSUPPORTED
    assert gdn.gdn_bwd_saved(**{**_bargs(), "dk_": 64, "dv_": 64}) == UNSUPPORTED
    assert gdn.gdn_bwd_saved(**{**_bargs(), **a, "workspace": P + 8}) == UNSUPPORTED
    assert gdn.gdn_bwd_saved(**{**_bargs(), **a, "workspace": 0}) == INVALID
    assert gdn.gdn_bwd_saved(**{**_bargs(), **a, "q": 0}) == INVALID
    assert gdn.gdn_bwd_saved(**{**_bargs(), **a, "B": 0}) == OK


def _bargs():
    return dict(q=P, k=P, v=P, g=P, beta=P, h0=0, cu_seqlens=0, dout=P, dhT=0, dq=P, dk=P, dv=P,
                dg=P, dbeta=P, dh0=0, workspace=P, workspace_bytes=1 << 40, B=1, T=8, H=1, dk_=32,
                dv_=32, stream=None, dtype=1)


# ---------------------------------------------------- no-allocation backward --

def _call_noalloc(**kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, h0=0, cu_seqlens=0, dout=P, dhT=0, dq=P, dk=P, dv=P,
             dg=P, dbeta=P, dh0=0, B=1, T=8, H=1, dk_=32, dv_=32, stream=None, dtype=1)
    a.update(kw)
    return gdn.gdn_bwd_noalloc(**a)


def test_noalloc_rejects_bad_args_before_any_device_call():
    assert _call_noalloc(q=0) == INVALID
    assert _call_noalloc(B=-1) == INVALID
    assert _call_noalloc(dk_=48) == UNSUPPORTED
    assert _call_noalloc(B=0) == OK  # nothing to do


def test_noalloc_rejects_problems_beyond_its_scratch():
    # 4 x 4096 tokens, 16 heads, d = 128 needs about 1.15 GB of workspace
    assert gdn.gdn_bwd_workspace_size(4, 4096, 16, 128, 128, 0) > gdn.NOALLOC_SCRATCH_BYTES
    assert _call_noalloc(B=4, T=4096, H=16, dk_=128, dv_=128) == -4
    assert "scratch" in gdn.strerror(-4)
