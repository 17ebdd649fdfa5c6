"""The affine chunk map (oracle/scan.py) against closed forms of the token
transition and against the sequential oracle."""
import numpy as np
import pytest

import oracle
from oracle import scan


def _chain(rng, T, dk=5, dv=4):
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return (k, rng.standard_normal((T, dv)), -np.logaddexp(0.0, rng.standard_normal(T) - 1.0),
            1.0 / (1.0 + np.exp(-rng.standard_normal(T))))


def test_one_token_map_is_the_transition():
    """A one-token chunk: P = alpha (I - beta k k^T), Q = beta k v^T."""
    rng = np.random.default_rng(0)
    k, v, g, b = _chain(rng, 1)
    P, Q = scan.chunk_map(k, v, g, b)
    a = np.exp(g[0])
    assert np.allclose(P, a * (np.eye(5) - b[0] * np.outer(k[0], k[0])), atol=1e-14)
    assert np.allclose(Q, b[0] * np.outer(k[0], v[0]), atol=1e-14)


def test_no_write_map_is_pure_decay():
    """beta = 0: P = exp(sum g) I and Q = 0."""
    rng = np.random.default_rng(1)
    k, v, g, b = _chain(rng, 9)
    P, Q = scan.chunk_map(k, v, g, np.zeros_like(b))
    assert np.allclose(P, np.exp(g.sum()) * np.eye(5), atol=1e-14)
    assert np.allclose(Q, 0.0, atol=1e-14)


def test_chunk_map_composes_token_maps():
    """A chunk's map equals the composition of its tokens' one-token maps."""
    rng = np.random.default_rng(2)
    k, v, g, b = _chain(rng, 7)
    acc = None
    for t in range(7):
        m = scan.chunk_map(k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1])
        acc = m if acc is None else scan.compose(acc, m)
    P, Q = scan.chunk_map(k, v, g, b)
    assert np.allclose(P, acc[0], atol=1e-13) and np.allclose(Q, acc[1], atol=1e-13)


@pytest.mark.parametrize("chunk,seg", [(4, 3), (16, 2), (5, 1)])
def test_segment_scan_gives_exact_states(chunk, seg):
    """The scan over composed segment maps gives, at every segment boundary,
    the state the sequential oracle reaches there, and the final state."""
    rng = np.random.default_rng(3 + chunk)
    T = 61
    k, v, g, b = _chain(rng, T)
    q = rng.standard_normal(k.shape)
    h0 = rng.standard_normal((5, 4))
    states = scan.scan_entry_states(scan.segment_maps(k, v, g, b, chunk, seg), h0)
    bounds = list(range(0, T, chunk * seg)) + [T]
    for s, t in enumerate(bounds):
        if t == 0:
            ref = h0
        else:
            sel = lambda x: x[None, :t, None]
            _, hT = oracle.fwd_seq(sel(q), sel(k), sel(v), g[None, :t, None], b[None, :t, None],
                                   h0[None, None])
            ref = hT[0, 0]
        assert np.max(np.abs(states[s] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), (s, t)


def test_planted_mistakes_are_caught(monkeypatch):
    """Composition in the wrong order, and a chunk map without the chunk's
    decay on the carried state, each break the exact-state check."""
    rng = np.random.default_rng(9)
    T, chunk, seg = 40, 4, 2
    k, v, g, b = _chain(rng, T)
    q = rng.standard_normal(k.shape)
    h0 = rng.standard_normal((5, 4))
    _, hT = oracle.fwd_seq(q[None, :, None], k[None, :, None], v[None, :, None],
                           g[None, :, None], b[None, :, None], h0[None, None])
    good = scan.scan_entry_states(scan.segment_maps(k, v, g, b, chunk, seg), h0)[-1]
    assert np.allclose(good, hT[0, 0], atol=1e-12)

    def wrong_order(first, second):
        P1, Q1 = first
        P2, Q2 = second
        return P1 @ P2, P1 @ Q2 + Q1

    monkeypatch.setattr(scan, "compose", wrong_order)
    bad = scan.scan_entry_states(scan.segment_maps(k, v, g, b, chunk, seg), h0)[-1]
    assert not np.allclose(bad, hT[0, 0], atol=1e-6)
    monkeypatch.undo()

    real = scan.chunk_map

    def no_decay(k_, v_, g_, b_):
        P, Q = real(k_, v_, g_, b_)
        return P + (1.0 - np.exp(np.sum(g_))) * np.eye(P.shape[0]), Q

    monkeypatch.setattr(scan, "chunk_map", no_decay)
    bad = scan.scan_entry_states(scan.segment_maps(k, v, g, b, chunk, seg), h0)[-1]
    assert not np.allclose(bad, hT[0, 0], atol=1e-6)
