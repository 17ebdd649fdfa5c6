"""CPU checks of the comparison function every parity test relies on, of the
host-side offset check and of the binding's output-buffer checks."""
import numpy as np
import pytest

import oracle
import synth
from hip_case import per_chain_errors

import gated_deltanet_recurrence_delta_amd as gdn


# ------------------------------------------------------------ oracle.rel_err

def test_rel_err_hand_values():
    # max|x - ref| / max|ref|: the largest deviation over the largest reference value
    assert oracle.rel_err([1.0, 2.0, -4.0], [1.0, 2.0, -4.0]) == 0.0
    assert oracle.rel_err([1.5, 2.0, -4.0], [1.0, 2.0, -4.0]) == pytest.approx(0.5 / 4.0)
    assert oracle.rel_err([1.0, 2.0, -3.0], [1.0, 2.0, -4.0]) == pytest.approx(1.0 / 4.0)
    # the deviation and the scale may sit at different positions
    assert oracle.rel_err([0.0, 10.0], [0.1, 10.0]) == pytest.approx(0.01)
    # sign of the error does not matter, nor the sign of the reference's extreme
    assert oracle.rel_err([-2.0, 0.0], [-1.0, 0.0]) == pytest.approx(1.0)


def test_rel_err_degenerate_cases():
    assert oracle.rel_err(np.zeros(0), np.zeros(0)) == 0.0
    assert oracle.rel_err(np.zeros(3), np.zeros(3)) == 0.0
    assert oracle.rel_err([0.0, 1e-3], np.zeros(2)) == float("inf")


def test_rel_err_mistakes_are_caught():
    """A comparator that forgot the absolute value, or divided by the
    average instead of the maximum, would give other numbers here."""
    ref = np.array([3.0, -5.0, 1.0])
    x = ref + np.array([0.0, -1.0, 0.0])
    assert oracle.rel_err(x, ref) == pytest.approx(0.2)       # |-1| / 5
    assert oracle.rel_err(ref - (x - ref), ref) == pytest.approx(0.2)


def test_per_chain_errors_use_each_chains_scale():
    inp = synth.generate(synth.custom(name="pc", seed=1, B=2, T=3, H=2, dk=2, dv=2))
    o_ref = np.ones((2, 3, 2, 2))
    o_ref[1, :, 0] = 0.01           # chain (1, 0) is 100x smaller
    h_ref = np.ones((2, 2, 2, 2))
    o = o_ref.copy()
    o[1, 2, 0, 1] += 0.001          # 0.1 % of the tensor's scale, 10 % of the chain's
    e_o, e_h = per_chain_errors(inp, o, h_ref.copy(), o_ref, h_ref)
    assert e_o[1, 0] == pytest.approx(0.1)
    assert e_o[0, 0] == 0.0 and e_o[0, 1] == 0.0 and e_o[1, 1] == 0.0
    assert float(e_h.max()) == 0.0
    assert oracle.rel_err(o, o_ref) == pytest.approx(0.001)  # the whole-tensor view misses it


def test_per_chain_errors_packed_slices():
    inp = synth.generate(synth.custom(name="pcp", seed=2, H=1, dk=2, dv=2, seq_lens=[2, 0, 3]))
    o_ref = np.ones((5, 1, 2))
    h_ref = np.ones((3, 1, 2, 2))
    o = o_ref.copy()
    o[3, 0, 0] = 1.5                # token 3 belongs to sequence 2
    e_o, e_h = per_chain_errors(inp, o, h_ref, o_ref, h_ref)
    assert e_o[2, 0] == pytest.approx(0.5) and e_o[0, 0] == 0.0 and e_o[1, 0] == 0.0


# ------------------------------------------------------- cu_seqlens host check

def test_check_offsets_accepts_valid():
    gdn.check_offsets(np.array([0, 3, 3, 10], dtype=np.int32), 10)
    gdn.check_offsets(np.array([0], dtype=np.int32), 0)


@pytest.mark.parametrize("cu,T,msg", [([1, 3, 10], 10, "cu_seqlens\\[0\\]"),
                                      ([0, 5, 3, 10], 10, "non-decreasing"),
                                      ([0, 3, 9], 10, "packed length"),
                                      ([], 0, "at least one")])
def test_check_offsets_rejects(cu, T, msg):
    with pytest.raises(ValueError, match=msg):
        gdn.check_offsets(np.array(cu, dtype=np.int32), T)


# ---------------------------------------------- caller-supplied output buffers

def _cpu_inputs(B=1, T=4, H=2, dk=32, dv=32):
    torch = pytest.importorskip("torch")
    q = torch.zeros(B, T, H, dk, dtype=torch.bfloat16)
    v = torch.zeros(B, T, H, dv, dtype=torch.bfloat16)
    g = torch.zeros(B, T, H)
    return torch, q, v, g


@pytest.mark.parametrize("bad", ["out_dtype", "out_shape", "hT_dtype", "hT_shape"])
def test_fwd_rejects_mismatched_outputs(bad):
    """An undersized or wrongly typed out/hT is refused before anything
    reaches the device (these tensors are on the CPU: the shape check comes
    first)."""
    torch, q, v, g = _cpu_inputs()
    out = torch.empty_like(v)
    hT = torch.empty(1, 2, 32, 32)
    if bad == "out_dtype":
        out = torch.empty(v.shape, dtype=torch.float32)
    elif bad == "out_shape":
        out = torch.empty(1, 3, 2, 32, dtype=torch.bfloat16)
    elif bad == "hT_dtype":
        hT = torch.empty(1, 2, 32, 32, dtype=torch.bfloat16)
    else:
        hT = torch.empty(1, 2, 32, 16)
    name = bad.split("_")[0]
    for f in (gdn.fwd, gdn.fwd_recurrent):
        with pytest.raises(ValueError, match=name):
            f(q, q, v, g, g, out=out, hT=hT)


def test_diag_fwd_rejects_mismatched_outputs():
    torch = pytest.importorskip("torch")
    v = torch.zeros(1, 4, 2, 32, dtype=torch.bfloat16)
    b = torch.zeros(1, 4, 2, 32, dtype=torch.bfloat16)
    g = torch.zeros(1, 4, 2)
    A = torch.zeros(2, 32)
    with pytest.raises(ValueError, match="hT"):
        gdn.diag_fwd(v, b, b, g, A, hT=torch.empty(1, 2, 16, 32))
    with pytest.raises(ValueError, match="out"):
        gdn.diag_fwd(v, b, b, g, A, out=torch.empty(1, 4, 2, 16, dtype=torch.bfloat16))
