"""The FP64 oracle against facts the rule fixes (closed forms, invariants,
hand-worked examples) and against its two other independent forms."""
import numpy as np
import pytest

import oracle
import synth
from pins import ALL_PINS


def _seq(q, k, v, g, beta, h0=None, cu=None):
    return oracle.fwd_seq(q, k, v, g, beta, h0, cu, nthreads=2)


def _matrix(q, k, v, g, beta, h0=None, cu=None):
    return oracle.fwd_matrix(q, k, v, g, beta, h0, cu)


def _chunked(C):
    def f(q, k, v, g, beta, h0=None, cu=None):
        return oracle.fwd_chunked(q, k, v, g, beta, h0, cu, chunk=C)
    return f


IMPLS = {"seq_c": _seq, "matrix_numpy": _matrix, "chunked_C1": _chunked(1),
         "chunked_C4": _chunked(4), "chunked_C16": _chunked(16)}


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(impl, pin):
    pin(IMPLS[impl], np.random.default_rng(1234))


@pytest.mark.parametrize("C", [1, 3, 16, 64, 1000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_equals_sequential(C, dtype):
    """Brute-force chunked form == sequential rule, incl. a ragged last
    chunk, a chunk longer than the sequence and a non-zero h0."""
    wl = synth.custom(seed=11, B=2, T=70, H=2, dk=8, dv=6, dtype=dtype, h0_std=0.3)
    inp = synth.generate(wl)
    a = [inp.as_f64(n) for n in ("q", "k", "v", "g", "beta", "h0")]
    o1, h1 = oracle.fwd_seq(*a)
    o2, h2 = oracle.fwd_chunked(*a, chunk=C)
    assert oracle.rel_err(o2, o1) < 1e-12
    assert oracle.rel_err(h2, h1) < 1e-12


def test_three_forms_agree_packed():
    wl = synth.custom(seed=12, H=3, dk=16, dv=8, dtype="bf16", seq_lens=[33, 1, 0, 64, 65])
    inp = synth.generate(wl)
    a = [inp.as_f64(n) for n in ("q", "k", "v", "g", "beta", "h0")]
    o1, h1 = oracle.fwd_seq(*a, cu_seqlens=inp.cu_seqlens)
    o2, h2 = oracle.fwd_matrix(*a, cu_seqlens=inp.cu_seqlens)
    o3, h3 = oracle.fwd_chunked(*a, cu_seqlens=inp.cu_seqlens, chunk=16)
    for o, h in ((o2, h2), (o3, h3)):
        assert oracle.rel_err(o, o1) < 1e-12
        assert oracle.rel_err(h, h1) < 1e-12


def test_chain_subset():
    """Computing a subset of chains gives those chains' full-run values."""
    wl = synth.custom(seed=13, B=3, T=40, H=4, dk=8, dv=8, h0_std=0.1)
    inp = synth.generate(wl)
    a = [inp.as_f64(n) for n in ("q", "k", "v", "g", "beta", "h0")]
    o1, h1 = oracle.fwd_seq(*a)
    chains = [0, 5, 11]
    o2, h2 = oracle.fwd_seq(*a, chains=chains)
    for c in chains:
        b, h = divmod(c, 4)
        assert np.array_equal(o2[b, :, h], o1[b, :, h])
        assert np.array_equal(h2[b, h], h1[b, h])
    assert not o2[0, :, 1].any()


def test_seq_rejects_bad_args():
    z = np.zeros((1, 2, 1, 2))
    zg = np.zeros((1, 2, 1))
    with pytest.raises(ValueError):
        oracle.fwd_seq(z[0], z[0], z[0], zg[0], zg[0], cu_seqlens=np.array([0, 3], np.int32))
    with pytest.raises(ValueError):
        oracle.fwd_seq(z, z, z, zg, zg, chains=[7])
