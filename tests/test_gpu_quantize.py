"""GPU parity of the packing step (archead_quantize) against the oracle's
quantizers (oracle.quantize, then oracle.pack).

Bar: the packed buffer is byte-identical to the oracle's (every code, scale,
padding byte and the header), and the error E = fp32(R) - SC4(R) is
bit-identical: both sides take every rounding decision in fp32 from the same
fp32 operands, and the fp64 core residual adds exact products in the same
order.  The head the GPU packs also goes through the forward, to show the
packed bytes are usable as they are.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import ah_mod, check_parity, device_H, log, run, to_f64, torch_mod

pytestmark = pytest.mark.gpu


def _dev(x):
    torch = torch_mod()
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _quantize(dense, g, with_error=True, W_dev=None):
    torch = torch_mod()
    ah = ah_mod()
    W = _dev(dense.W) if W_dev is None else W_dev
    head, E = ah.archead_quantize(W, _dev(dense.A_c), _dev(dense.B_c), _dev(dense.A_w), _dev(dense.B_w), g,
                                  with_error=with_error)
    torch.cuda.synchronize()
    return head, (E.cpu().numpy() if E is not None else None)


CASES = [
    # V, D, r_c, r_r, g, W dtype: ragged V (padding rows), every group size,
    # ranks 0 and odd ranks, D up to the register limit
    (1000, 512, 16, 8, 64, "bf16"),
    (777, 256, 8, 0, 32, "f32"),
    (530, 1024, 40, 72, 256, "bf16"),
    (64, 128, 0, 0, 128, "f32"),
    (300, 384, 5, 3, 128, "bf16"),
    (129, 8192, 16, 16, 128, "bf16"),
    (2048, 4096, 32, 32, 128, "f32"),
]


@pytest.mark.parametrize("V,D,r_c,r_r,g,wdt", CASES)
def test_quantize_matches_oracle(V, D, r_c, r_r, g, wdt):
    log(f"quantize V={V} D={D} r_c={r_c} r_r={r_r} g={g} W={wdt}")
    dense = synth.draw_dense(np.random.default_rng(V + D + r_c), V, D, r_c, r_r, wdt)
    head_ref, E_ref = oracle.quantize(dense.W, dense.A_c, dense.B_c, dense.A_w, dense.B_w, g)
    buf_ref = oracle.pack(head_ref)
    head, E = _quantize(dense, g)
    buf = head.buffer.cpu().numpy()
    assert buf.size == buf_ref.size
    diff = np.nonzero(buf != buf_ref)[0]
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8]}"
    assert np.array_equal(E.view(np.uint32), E_ref.view(np.uint32))


def test_quantize_zero_rows_and_strided_w():
    """Rows whose residual is zero give s_R = c8 = q4 = 0, zero factor rows give
    zero scales and codes, and W may be a strided view."""
    V, D, r_c, r_r, g = 200, 512, 8, 8, 64
    dense = synth.draw_dense(np.random.default_rng(3), V, D, r_c, r_r, "f32")
    dense.A_c[10] = 0.0
    dense.W[10] = 0.0          # residual row 10 is exactly zero
    dense.A_w[11] = 0.0
    dense.B_c[2, 64:128] = 0.0  # one zero group of B_c
    torch = torch_mod()
    Wpad = np.zeros((V, D + 64), np.float32)
    Wpad[:, :D] = dense.W
    W_dev = torch.from_numpy(Wpad).to("cuda")[:, :D]
    head, E = _quantize(dense, g, W_dev=W_dev)
    head_ref, E_ref = oracle.quantize(dense.W, dense.A_c, dense.B_c, dense.A_w, dense.B_w, g)
    assert head_ref.s_R[10] == 0 and (head_ref.c8[10] == 0).all() and head_ref.s_Aw[11] == 0
    assert np.array_equal(head.buffer.cpu().numpy(), oracle.pack(head_ref))
    assert np.array_equal(E.view(np.uint32), E_ref.view(np.uint32))


def test_quantized_head_runs_the_forward():
    """The GPU-packed head is a valid input of archead_logits: its logits match
    the oracle's logits of the oracle-quantized components."""
    V, D, r_c, r_r, g, N = 1000, 512, 16, 8, 64, 40
    dense = synth.draw_dense(np.random.default_rng(11), V, D, r_c, r_r, "bf16")
    head, _ = _quantize(dense, g, with_error=False)
    head_ref, _ = oracle.quantize(dense.W, dense.A_c, dense.B_c, dense.A_w, dense.B_w, g)
    inp = synth.make("tiny", seed=11, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g)
    Yr = oracle.logits(inp.H_bits, head_ref)
    for path in (0, 2):
        Yg = to_f64(run(head, inp.H_bits, path, H_dev=device_H(inp.H_bits)))
        check_parity(Yg, Yr, f"path {path}")
    # the decode path takes at most 16 tokens: the first 8 rows
    H8 = inp.H_bits[:8].copy()
    Yg = to_f64(run(head, H8, 1, H_dev=device_H(H8)))
    check_parity(Yg, Yr[:8], "path 1")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_quantize_full_size_sampled_rows():
    """The decode/batched head (V=151936, D=4096, r_c=r_r=32, g=128) packed
    whole on the GPU; 64 seeded rows (with the first and last) and every B
    row checked against the oracle, which quantises those rows on their own
    (the row steps depend on nothing outside their row; B is quantised whole)."""
    cfg = synth.config("decode")
    V, D, r_c, r_r, g = cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"]
    log(f"full-size quantize V={V} D={D} r_c={r_c} r_r={r_r} g={g}")
    dense = synth.draw_dense(np.random.default_rng(2024), V, D, r_c, r_r, "bf16")
    head, E = _quantize(dense, g)
    got = oracle.unpack(head.buffer.cpu().numpy(), V, D, r_c, r_r, g)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, V - 1], rng.choice(V, 62, replace=False)]))
    ref, E_ref = oracle.quantize(dense.W[rows], dense.A_c[rows], dense.B_c, dense.A_w[rows], dense.B_w, g)
    for k in ("q4", "c8", "s_R", "A_c", "s_Ac", "A_w", "s_Aw"):
        a, b = np.ascontiguousarray(got[k][rows]), np.ascontiguousarray(getattr(ref, k))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), k
    for k in ("B_c", "s_Bc", "B_w", "s_Bw"):
        a, b = np.ascontiguousarray(got[k]), np.ascontiguousarray(getattr(ref, k))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), k
    assert np.array_equal(E[rows].view(np.uint32), E_ref.view(np.uint32))


def test_quantize_at_the_core_rank_limit():
    """Core rank 1024, the most the residual kernel keeps in LDS (8 rows x 1024
    fp64 values = 64 KiB), and D = 8192 with 4 rows per workgroup."""
    for V, D, r_c, r_r in [(70, 256, 1024, 8), (40, 8192, 1024, 0)]:
        log(f"quantize at the rank limit V={V} D={D} r_c={r_c}")
        dense = synth.draw_dense(np.random.default_rng(D), V, D, r_c, r_r, "bf16")
        head_ref, E_ref = oracle.quantize(dense.W, dense.A_c, dense.B_c, dense.A_w, dense.B_w, 128)
        head, E = _quantize(dense, 128)
        assert np.array_equal(head.buffer.cpu().numpy(), oracle.pack(head_ref))
        assert np.array_equal(E.view(np.uint32), E_ref.view(np.uint32))
