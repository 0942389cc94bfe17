"""GPU parity of the fused row statistics (archead_logits_stats) against the
fp64 oracle.

Bar: identical argmax to the oracle's (lowest index on ties); max and
log-sum-exp within 2e-3 * max|Y_ref| (log-sum-exp moves by at most the largest
logit error); cross-entropy within twice that.  Separately, the statistics
must agree to fp32 rounding with the oracle's statistics of the GPU's own
fp32 logits, which checks the piecewise reduction on its own.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, ah_mod, device_H, log, run, to_f64, torch_mod

pytestmark = pytest.mark.gpu


def _stats(head, H_bits, targets):
    torch = torch_mod()
    t = torch.as_tensor(np.asarray(targets, np.int32), device="cuda")
    out = ah_mod().archead_logits_stats(device_H(H_bits), head, targets=t)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _check(st, ref, scale, what):
    assert np.array_equal(st["argmax"], ref["argmax"]), f"{what}: argmax {st['argmax'][:8]} vs {ref['argmax'][:8]}"
    for k, tol in (("max", TOL), ("lse", TOL), ("ce", 2 * TOL)):
        err = np.abs(st[k].astype(np.float64) - ref[k]).max()
        log(f"  {what} {k}: max err / max|Y| = {err / scale:.3e}")
        assert err <= tol * scale, f"{what} {k}: {err / scale:.3e}"


CASES = [
    # V, D, r_c, r_r, g, N: decode path (N <= 16) and the three tile variants, ragged
    (1000, 512, 16, 8, 64, 1),
    (2048, 1024, 32, 32, 128, 3),
    (777, 256, 8, 0, 32, 16),
    (1000, 512, 16, 8, 64, 17),
    (2048, 1024, 32, 32, 128, 64),
    (530, 512, 40, 72, 256, 65),
    (1000, 512, 0, 0, 128, 130),
    (2048, 1024, 32, 32, 128, 300),
]


@pytest.mark.parametrize("V,D,r_c,r_r,g,N", CASES)
def test_stats_match_oracle(V, D, r_c, r_r, g, N):
    log(f"stats V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N}")
    inp = synth.make("tiny", seed=V + 7 * N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
    head = ah_mod().PackedHead.from_components(inp.head)
    rng = np.random.default_rng(N)
    targets = rng.integers(0, V, size=N)
    Yr = oracle.logits(inp.H_bits, inp.head)
    st = _stats(head, inp.H_bits, targets)
    _check(st, oracle.row_stats(Yr, targets), np.abs(Yr).max(), "vs oracle")
    # the reduction alone: statistics of the GPU's own fp32 logits (the logits
    # call may split a tile's hidden dimension where the statistics call does
    # not, so the two agree to fp32 rounding, not bit for bit)
    Yg = to_f64(run(head, inp.H_bits, 0))
    own = oracle.row_stats(Yg, targets)
    assert np.array_equal(st["argmax"], own["argmax"])
    for k in ("max", "lse", "ce"):
        assert np.allclose(st[k], own[k], rtol=0, atol=1e-5 * np.abs(Yg).max() + 1e-5), k


def test_stats_ties_and_bad_targets():
    """A zero head gives Y = 0: every logit ties, so argmax is 0 and
    lse = ce = log V; a target outside [0, V) gives a NaN cross-entropy."""
    V, D, N = 600, 256, 20  # N > 16: tile path
    inp = synth.make("tiny", seed=5, V=V, D=D, N=N, r_c=16, r_r=24, g=64)
    z = synth.zero_head(V, D, 16, 24, 64)
    head = ah_mod().PackedHead.from_components(z)
    targets = np.arange(N) * 31 % V
    targets[3], targets[7] = -1, V
    st = _stats(head, inp.H_bits, targets)
    assert (st["argmax"] == 0).all() and (st["max"] == 0).all()
    assert np.allclose(st["lse"], np.log(V), rtol=1e-6)
    ok = np.ones(N, bool)
    ok[[3, 7]] = False
    assert np.allclose(st["ce"][ok], np.log(V), rtol=1e-6)
    assert np.isnan(st["ce"][~ok]).all()
    # the decode path on the first rows
    st4 = _stats(head, inp.H_bits[:4], targets[:4])
    assert (st4["argmax"] == 0).all() and np.allclose(st4["lse"], np.log(V), rtol=1e-6)


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "batched", "prefill"])
def test_stats_full_size(name):
    """The full-size workloads; prefill on 48 seeded rows (all rows are
    computed, the oracle checks the sample)."""
    cfg = synth.config(name)
    log(f"full-size stats {name}: {cfg}")
    inp = synth.make(name)
    head = ah_mod().PackedHead.from_components(inp.head)
    N, V = cfg["N"], cfg["V"]
    targets = np.random.default_rng(99).integers(0, V, size=N)
    st = _stats(head, inp.H_bits, targets)
    if N <= 256:
        rows = np.arange(N)
    else:
        rng = np.random.default_rng(1234)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 46, replace=False)]))
    Yr = oracle.logits(inp.H_bits, inp.head, rows=rows)
    ref = oracle.row_stats(Yr, targets[rows])
    _check({k: v[rows] for k, v in st.items()}, ref, np.abs(Yr).max(), name)
