"""GPU parity of the whole construction (archead_fit) against the oracle.

The factorisations are not unique (signs, rotations within tied singular
values) and the GPU runs them in fp32, so the factors are compared through
what is unique:
  - packing: given the GPU's own fp32 factors, the packed buffer equals the
    oracle's packing of them byte for byte, and the GPU's core error E equals
    the oracle's E of them bit for bit;
  - core: the GPU core's residual ||W - A_c B_c||^2 matches the oracle's
    randomized SVD with the same test matrix (fp64) to 1e-3 and is within
    1e-3 of the Eckart-Young optimum;
  - correction: on the GPU's E, the metric objective ||(E - A_w B_w) T_p||^2
    (T_p from the oracle, fp64) matches the oracle's randomized SVD of E T_p
    with the same test matrix to 2e-3, and the correction lowers it.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import ah_mod, log, torch_mod

pytestmark = pytest.mark.gpu


def _dev(x):
    torch = torch_mod()
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _run(fi, r_c, r_r, g, p, lam, o, q):
    ah = ah_mod()
    head, f = ah.archead_fit(_dev(fi.W), _dev(fi.H), _dev(fi.omega_c), _dev(fi.omega_r), r_c, r_r, g, p=p, lam=lam,
                             oversample=o, power_iters=q, outputs=True)
    torch_mod().cuda.synchronize()
    return head.buffer.cpu().numpy(), {k: v.cpu().numpy() for k, v in f.items()}


CASES = [
    # V, D, r_c, r_r, g, N calibration tokens, p, lambda, oversample, power iterations
    (1000, 256, 16, 8, 64, 512, 0.75, 0.01, 8, 2),
    (2048, 512, 32, 32, 128, 1024, 0.5, 0.05, 8, 2),
    (777, 384, 8, 0, 128, 300, 0.75, 0.01, 4, 1),
    (600, 256, 0, 16, 32, 400, 1.0, 0.1, 8, 3),
    # larger than the V row chunks of the thin products (64) and the Gram chunks (256) by far
    (8192, 1024, 32, 32, 128, 2048, 0.75, 0.01, 8, 2),
]


@pytest.mark.parametrize("V,D,r_c,r_r,g,N,p,lam,o,q", CASES)
def test_fit_matches_oracle(V, D, r_c, r_r, g, N, p, lam, o, q):
    log(f"fit V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N} p={p} lam={lam} o={o} q={q}")
    fi = synth.draw_fit(np.random.default_rng(V + D), V, D, r_c, r_r, N, oversample=o)
    buf, f = _run(fi, r_c, r_r, g, p, lam, o, q)
    # packing of the GPU's own factors
    head_ref, E_ref = oracle.quantize(fi.W, f["A_c"], f["B_c"], f["A_w"], f["B_w"], g)
    assert np.array_equal(buf, oracle.pack(head_ref))
    assert np.array_equal(f["E"].view(np.uint32), E_ref.view(np.uint32))
    W64 = oracle.bf16_bits_to_f64(fi.W)
    # core
    if r_c:
        res_g = np.sum((W64 - f["A_c"].astype(np.float64) @ f["B_c"]) ** 2)
        A, B = oracle.rsvd(W64, r_c, fi.omega_c, q)
        res_o = np.sum((W64 - A @ B) ** 2)
        opt = np.sum(np.linalg.svd(W64, compute_uv=False)[r_c:] ** 2)
        log(f"  core residual: gpu {res_g:.6e} oracle {res_o:.6e} optimum {opt:.6e}")
        assert abs(res_g - res_o) <= 1e-3 * res_o and res_g <= (1 + 1e-3) * opt
    # correction, on the GPU's core error
    if r_r:
        T, Tinv = oracle.metric_transform(oracle.damped_covariance(oracle.bf16_bits_to_f64(fi.H), lam), p)
        E = f["E"].astype(np.float64)
        J0 = oracle.metric_objective(E, T)
        Jg = oracle.metric_objective(E - f["A_w"].astype(np.float64) @ f["B_w"], T)
        A, Bt = oracle.rsvd(E @ T, r_r, fi.omega_r, q)
        Jo = oracle.metric_objective(E - A @ (Bt @ Tinv), T)
        log(f"  metric objective: none {J0:.6e} gpu {Jg:.6e} oracle {Jo:.6e}")
        assert abs(Jg - Jo) <= 2e-3 * Jo and Jg < J0


def test_fit_rejects_nonpositive_damping_before_launch():
    """lambda <= 0 is an argument error (the metric's inverse power needs a
    positive definite C_lam); nothing runs."""
    ah = ah_mod()
    fi = synth.draw_fit(np.random.default_rng(1), 200, 256, 8, 8, 100)
    with pytest.raises(ah.ArcheadError):
        ah.archead_fit(_dev(fi.W), _dev(fi.H), _dev(fi.omega_c), _dev(fi.omega_r), 8, 8, 64, lam=0.0)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_fit_full_size_sampled_rows():
    """The decode/batched head shape (V=151936, D=4096, r_c=r_r=32, g=128) with
    4096 calibration tokens, in the configuration bench.py times (oversample 8,
    two power iterations, p=0.75, lambda=0.01).  On 64 seeded rows: the packing
    of the GPU's factors is exact; the core residual of each row matches the
    oracle's randomized SVD of the whole W (same test matrix, fp64) to 1e-3 of
    the rows' total; the correction lowers the rows' metric objective."""
    cfg = synth.config("decode")
    V, D, r_c, r_r, g = cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"]
    p, lam, o, q = 0.75, 0.01, 8, 2
    log(f"full-size fit V={V} D={D} r_c={r_c} r_r={r_r} N=4096")
    fi = synth.draw_fit(np.random.default_rng(77), V, D, r_c, r_r, 4096, oversample=o)
    buf, f = _run(fi, r_c, r_r, g, p, lam, o, q)
    rows = np.unique(np.concatenate([[0, V - 1], np.random.default_rng(8).choice(V, 62, replace=False)]))
    got = oracle.unpack(buf, V, D, r_c, r_r, g)
    ref, E_ref = oracle.quantize(fi.W[rows], f["A_c"][rows], f["B_c"], f["A_w"][rows], f["B_w"], g)
    for k in ("q4", "c8", "s_R", "A_c", "s_Ac", "A_w", "s_Aw"):
        a, b = np.ascontiguousarray(got[k][rows]), np.ascontiguousarray(getattr(ref, k))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), k
    for k in ("B_c", "s_Bc", "B_w", "s_Bw"):
        a, b = np.ascontiguousarray(got[k]), np.ascontiguousarray(getattr(ref, k))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), k
    assert np.array_equal(f["E"][rows].view(np.uint32), E_ref.view(np.uint32))
    log("  packing exact on sampled rows; oracle randomized SVD of the whole W ...")
    W64 = oracle.bf16_bits_to_f64(fi.W)
    A, B = oracle.rsvd(W64, r_c, fi.omega_c, q)
    res_o = np.sum((W64[rows] - A[rows] @ B) ** 2, axis=1)
    del W64, A
    res_g = np.sum((oracle.bf16_bits_to_f64(fi.W[rows]) - f["A_c"][rows].astype(np.float64) @ f["B_c"]) ** 2, axis=1)
    log(f"  core residual on the rows: gpu {res_g.sum():.6e} oracle {res_o.sum():.6e}")
    assert np.abs(res_g - res_o).max() <= 1e-3 * res_o.sum()
    T, _ = oracle.metric_transform(oracle.damped_covariance(oracle.bf16_bits_to_f64(fi.H), lam), p)
    E = f["E"][rows].astype(np.float64)
    J0 = oracle.metric_objective(E, T)
    Jg = oracle.metric_objective(E - f["A_w"][rows].astype(np.float64) @ f["B_w"], T)
    log(f"  metric objective on the rows: none {J0:.6e} corrected {Jg:.6e}")
    assert Jg < J0


def test_fit_with_no_factors_is_plain_sc4():
    """r_c = r_r = 0: the packed head is SC4 of W alone and E = W - SC4(W)."""
    V, D, g = 300, 256, 64
    fi = synth.draw_fit(np.random.default_rng(2), V, D, 0, 0, 200, oversample=4)
    buf, f = _run(fi, 0, 0, g, 0.75, 0.01, 4, 1)
    none = (np.zeros((V, 0), np.float32), np.zeros((0, D), np.float32))
    head_ref, E_ref = oracle.quantize(fi.W, *none, *none, g)
    assert np.array_equal(buf, oracle.pack(head_ref))
    assert np.array_equal(f["E"].view(np.uint32), E_ref.view(np.uint32))


def test_fit_fp32_strided_w():
    """W given as fp32 through a strided view (row stride D + 64) gives the
    same packed head as the contiguous bf16 values it holds."""
    V, D, r_c, r_r, g = 500, 256, 8, 8, 64
    fi = synth.draw_fit(np.random.default_rng(12), V, D, r_c, r_r, 300, oversample=4)
    torch = torch_mod()
    ah = ah_mod()
    W32 = oracle.bf16_bits_to_f64(fi.W).astype(np.float32)
    pad = np.zeros((V, D + 64), np.float32)
    pad[:, :D] = W32
    Wv = torch.from_numpy(pad).to("cuda")[:, :D]
    head_a, _ = ah.archead_fit(Wv, _dev(fi.H), _dev(fi.omega_c), _dev(fi.omega_r), r_c, r_r, g, oversample=4,
                               power_iters=1)
    head_b, _ = ah.archead_fit(_dev(fi.W), _dev(fi.H), _dev(fi.omega_c), _dev(fi.omega_r), r_c, r_r, g, oversample=4,
                               power_iters=1)
    torch.cuda.synchronize()
    assert torch.equal(head_a.buffer, head_b.buffer)


def test_fit_zero_head_drops_every_direction():
    """W = 0: every Cholesky pivot of the randomized SVDs' panels vanishes, so
    every direction is dropped and the factors come out zero (the same
    function as any orthonormal basis of a zero sketch would give); the packed
    head is all zero codes and E = 0, with no error."""
    V, D, r_c, r_r, g = 300, 256, 8, 8, 64
    fi = synth.draw_fit(np.random.default_rng(3), V, D, r_c, r_r, 200, oversample=4)
    fi.W[:] = 0
    buf, f = _run(fi, r_c, r_r, g, 0.75, 0.01, 4, 2)
    for k in ("A_c", "B_c", "A_w", "B_w", "E"):
        assert not f[k].any(), k
    zeros = (np.zeros((V, r_c), np.float32), np.zeros((r_c, D), np.float32))
    head_ref, _ = oracle.quantize(fi.W, *zeros, np.zeros((V, r_r), np.float32), np.zeros((r_r, D), np.float32), g)
    assert np.array_equal(buf, oracle.pack(head_ref))
