"""GPU parity of archead_logits_topk against the oracle's top-k (oracle.row_topk).

Two checks per case:
  - the selection alone: on the GPU's own fp32 logits (the forward run on the
    same 256-token chunks, so the logits are the same numbers) the indices
    and values equal the oracle's top-k of those logits exactly;
  - against the fp64 oracle logits: the i-th largest value differs from the
    oracle's i-th largest by at most 2e-3 * max|Y_ref| (an order statistic
    moves by at most the largest logit error), and each chosen index's exact
    logit is that close to the oracle's i-th value.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, ah_mod, device_H, log, torch_mod

pytestmark = pytest.mark.gpu

CHUNK = 256


def _own_logits(head, H):
    ah = ah_mod()
    parts = [ah.logits(H[t0:t0 + CHUNK], head) for t0 in range(0, H.shape[0], CHUNK)]
    torch_mod().cuda.synchronize()
    return np.concatenate([p.cpu().numpy() for p in parts], 0)


CASES = [
    # V, D, r_c, r_r, g, N, k: decode path chunks (N <= 16), tile chunks, a
    # ragged last chunk, k from 1 to 16
    (1000, 512, 16, 8, 64, 1, 1),
    (2048, 1024, 32, 32, 128, 5, 10),
    (777, 256, 8, 0, 32, 16, 16),
    (1000, 512, 16, 8, 64, 40, 5),
    (2048, 1024, 32, 32, 128, 300, 10),
    (530, 512, 40, 72, 256, 513, 4),
    # many 1024-logit spans per row, so the span-maximum threshold leaves
    # most spans out: k = 1, 5, 16, one and several chunks
    (30000, 256, 16, 8, 64, 9, 16),
    (30011, 512, 8, 8, 32, 70, 1),
    (65536, 256, 16, 16, 128, 300, 5),
]


@pytest.mark.parametrize("V,D,r_c,r_r,g,N,k", CASES)
def test_topk_matches_oracle(V, D, r_c, r_r, g, N, k):
    log(f"topk V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N} k={k}")
    inp = synth.make("tiny", seed=V + 3 * N + k, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
    ah = ah_mod()
    head = ah.PackedHead.from_components(inp.head)
    H = device_H(inp.H_bits)
    vals, idx = ah.archead_logits_topk(H, head, k)
    torch_mod().cuda.synchronize()
    vals, idx = vals.cpu().numpy(), idx.cpu().numpy()
    own = _own_logits(head, H)
    ov, oi = oracle.row_topk(own, k)
    assert np.array_equal(idx, oi), f"selection differs on own logits: {idx[:2]} vs {oi[:2]}"
    assert np.array_equal(vals.view(np.uint32), ov.astype(np.float32).view(np.uint32))
    Yr = oracle.logits(inp.H_bits, inp.head)
    rv, _ = oracle.row_topk(Yr, k)
    scale = np.abs(Yr).max()
    err = np.abs(vals.astype(np.float64) - rv).max()
    log(f"  top-k values vs oracle: {err / scale:.3e}")
    assert err <= TOL * scale
    assert np.abs(np.take_along_axis(Yr, idx.astype(np.int64), 1) - rv).max() <= 2 * TOL * scale


@pytest.mark.parametrize("V,k", [(600, 7), (20000, 16)])
def test_topk_ties(V, k):
    """A zero head gives Y = 0: every row's top-k is indices 0..k-1 with value
    0 (with V = 20000 every span's maximum equals the threshold)."""
    D, N = 256, 20
    inp = synth.make("tiny", seed=5, V=V, D=D, N=N, r_c=16, r_r=24, g=64)
    ah = ah_mod()
    head = ah.PackedHead.from_components(synth.zero_head(V, D, 16, 24, 64))
    vals, idx = ah.archead_logits_topk(device_H(inp.H_bits), head, k)
    torch_mod().cuda.synchronize()
    assert (idx.cpu().numpy() == np.arange(k)).all() and (vals.cpu().numpy() == 0).all()


def test_topk_planted_in_one_span():
    """One-hot rows pick one weight column: its largest stored value sits in
    sixteen rows of one span, and every other span's maximum is one step
    lower, so the threshold keeps many spans and the ties inside the best
    span decide by index."""
    V, D, N, k = 40000, 256, 4, 16
    inp = synth.make("tiny", seed=9, V=V, D=D, N=1, r_c=0, r_r=0, g=64)
    h = inp.head
    rng = np.random.default_rng(17)
    h.c8[:] = 1
    h.s_R[:] = np.float16(1.0)
    h.q4[:] = rng.integers(-8, 7, size=h.q4.shape, dtype=np.int8)   # at most 6
    cols = np.array([0, 77, 128, 255])
    h.q4[5000:5016, cols] = 7                                        # rows 5000..5015, span 4
    eye = np.zeros((N, D), np.float32)
    eye[np.arange(N), cols] = 1.0
    ah = ah_mod()
    head = ah.PackedHead.from_components(h)
    vals, idx = ah.archead_logits_topk(device_H(synth.f32_to_bf16_bits(eye)), head, k)
    torch_mod().cuda.synchronize()
    assert (idx.cpu().numpy() == np.arange(5000, 5016)).all() and (vals.cpu().numpy() == 7).all()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_topk_full_size_batched():
    """The batched workload (V=151936, D=4096, N=64), top-10, every row."""
    cfg = synth.config("batched")
    inp = synth.make("batched")
    ah = ah_mod()
    head = ah.PackedHead.from_components(inp.head)
    H = device_H(inp.H_bits)
    vals, idx = ah.archead_logits_topk(H, head, 10)
    torch_mod().cuda.synchronize()
    vals, idx = vals.cpu().numpy(), idx.cpu().numpy()
    own = _own_logits(head, H)
    ov, oi = oracle.row_topk(own, 10)
    assert np.array_equal(idx, oi)
    rows = np.arange(cfg["N"])
    Yr = oracle.logits(inp.H_bits, inp.head, rows=rows)
    rv, _ = oracle.row_topk(Yr, 10)
    assert np.abs(vals.astype(np.float64) - rv).max() <= TOL * np.abs(Yr).max()


@pytest.mark.parametrize("V,k", [(16, 16), (10, 10), (33, 16), (1, 1)])
def test_topk_small_vocabularies(V, k):
    """k equal to V (every index comes back, sorted), vocabularies smaller
    than one piece, and a single row of vocabulary."""
    D, N = 256, 20
    inp = synth.make("tiny", seed=V, V=V, D=D, N=N, r_c=8, r_r=8, g=32)
    ah = ah_mod()
    head = ah.PackedHead.from_components(inp.head)
    H = device_H(inp.H_bits)
    vals, idx = ah.archead_logits_topk(H, head, k)
    torch_mod().cuda.synchronize()
    vals, idx = vals.cpu().numpy(), idx.cpu().numpy()
    ov, oi = oracle.row_topk(_own_logits(head, H), k)
    assert np.array_equal(idx, oi) and np.array_equal(vals, ov.astype(np.float32))
    if k == V:
        assert (np.sort(idx, axis=1) == np.arange(V)).all()
