"""GPU parity of the storage-matched comparison heads (group INT4 with fp16 group
scales, row INT8; ARCHead paper, results discussion of Tables 7 and 8) against
the oracle's fp64 logits (oracle.logits_alt), through archead_logits.

Both heads run on the batched streaming kernel, 32 tokens per launch: the
cases span one and several launches with a ragged last one, ragged vocabulary
tails, every group size, and one-hot rows that must return the dequantised
weights bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import ah_mod, check_parity, device_H, log, run, to_f64, torch_mod

pytestmark = pytest.mark.gpu

G4, R8 = 1, 2

CASES = [
    # fmt, V, D, g, N
    (G4, 1000, 512, 32, 1),
    (G4, 1000, 512, 64, 17),
    (G4, 2003, 1024, 128, 32),
    (G4, 777, 512, 256, 70),
    (G4, 4099, 2048, 32, 16),
    (R8, 1000, 512, 64, 1),
    (R8, 2003, 1024, 128, 33),
    (R8, 777, 2048, 32, 70),
    (R8, 4099, 512, 256, 16),
    (R8, 300, 8192, 32, 5),        # 64 k-tiles, 256 groups (the row INT8 head keeps no groups)
]


@pytest.mark.parametrize("fmt,V,D,g,N", CASES)
def test_alt_head_matches_oracle(fmt, V, D, g, N):
    log(f"alt fmt={fmt} V={V} D={D} g={g} N={N}")
    ah = ah_mod()
    torch = torch_mod()
    H_bits, h = synth.make_alt(fmt, 7 * V + N + fmt, V, D, N, g)
    head = ah.PackedHead.from_components(h)
    assert ah.archead_main_kernel(V, D, 0, 0, g, N, fmt=fmt) == "batch_kernel"
    Yr = oracle.logits_alt(H_bits, h)
    H = device_H(H_bits)
    y_auto = run(head, H_bits, 0, "f32", H_dev=H)
    check_parity(to_f64(y_auto), Yr, f"fmt={fmt} auto")
    y_dec = run(head, H_bits, 1, "f32", H_dev=H)           # the forced decode path is the same kernel
    assert torch.equal(y_auto.view(torch.int32), y_dec.view(torch.int32))
    y16 = run(head, H_bits, 0, "bf16", H_dev=H)
    assert torch.equal(y_auto.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))
    y2 = run(head, H_bits, 0, "f32", H_dev=H)               # same bits on every run
    assert torch.equal(y_auto.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("fmt", [G4, R8])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_alt_one_hot_rows_recover_weights_bit_exactly(fmt, g):
    """H = unit rows e_k: Y[n, v] = W_hat[v, k], the product of an exact code
    and an fp16 scale, so the GPU must return it exactly (extreme codes,
    subnormal, zero, largest and negative scales included)."""
    V, D = 300, 512
    h = synth.draw_alt_head(np.random.default_rng(g + 10 * fmt), fmt, V, D, g)
    lo, hi = (-8, 7) if fmt == G4 else (-127, 127)
    h.codes[0, :] = lo
    h.codes[1, :] = hi
    sv = h.scales.view(np.uint16)
    for row, bits in ((4, 0x0001), (5, 0x03FF), (6, 0x0000), (7, 0x7BFF), (8, 0x8400)):
        sv[row] = bits
    ks = np.array(sorted(set([0, 1, 7, 8, 31, 32, 33, 63, 64, 127, 128, 255, 256, 300, 511] +
                             list(range(2, D, 37)))))[:64]
    eye = np.zeros((ks.size, D), np.float32)
    eye[np.arange(ks.size), ks] = 1.0
    Hb = synth.f32_to_bf16_bits(eye)
    head = ah_mod().PackedHead.from_components(h)
    Y = run(head, Hb, 0).cpu().numpy()                      # 64 rows: two launches of 32
    W = oracle.w_hat_alt(h)                                   # exact in fp64 and fp32
    want = W[:, ks].T.astype(np.float32)
    assert not np.isnan(Y).any()
    assert np.array_equal(Y, want), f"max diff {np.abs(Y.astype(np.float64) - W[:, ks].T).max()}"


@pytest.mark.parametrize("fmt", [G4, R8])
def test_alt_row_strides_and_zero_tokens(fmt):
    """Strided H and Y views (rows of a larger tensor) give the dense result;
    N = 0 writes nothing."""
    ah = ah_mod()
    torch = torch_mod()
    V, D, g, N = 1000, 512, 64, 40
    H_bits, h = synth.make_alt(fmt, 99 + fmt, V, D, N, g)
    head = ah.PackedHead.from_components(h)
    Hbig = torch.zeros((N, D + 64), dtype=torch.bfloat16, device="cuda")
    Hbig[:, :D] = device_H(H_bits)
    Ybig = torch.full((N, V + 24), float("nan"), dtype=torch.float32, device="cuda")
    ah.archead_logits_path(Hbig[:, :D], head, Ybig[:, :V], 0)
    torch.cuda.synchronize()
    assert torch.isnan(Ybig[:, V:]).all()
    check_parity(to_f64(Ybig[:, :V]), oracle.logits_alt(H_bits, h), f"fmt={fmt} strided")
    Y0 = torch.full((0, V), float("nan"), device="cuda")
    ah.archead_logits_path(Hbig[:0, :D], head, Y0, 0)


@pytest.mark.parametrize("fmt", [G4, R8])
def test_alt_topk_serves_comparison_heads(fmt):
    """archead_logits_topk, built on archead_logits, takes a comparison head:
    its top-k equals the oracle's selection from the GPU's own logits."""
    ah = ah_mod()
    V, D, g, N, k = 1000, 512, 64, 37, 8
    H_bits, h = synth.make_alt(fmt, 5 + fmt, V, D, N, g)
    head = ah.PackedHead.from_components(h)
    H = device_H(H_bits)
    vals, idx = ah.archead_logits_topk(H, head, k)
    own = run(head, H_bits, 0, "f32", H_dev=H).cpu().numpy()
    ov, oi = oracle.row_topk(own, k)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(vals.cpu().numpy().view(np.uint32), ov.astype(np.float32).view(np.uint32))


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", [G4, R8])
@pytest.mark.parametrize("N", [1, 64])
def test_alt_full_size(fmt, N):
    """The comparison heads at the full decode shape (V = 128256, D = 4096,
    g = 128), every row and column against the oracle."""
    V, D, g = 128256, 4096, 128
    log(f"alt full size fmt={fmt} N={N}")
    ah = ah_mod()
    H_bits, h = synth.make_alt(fmt, 1000 + fmt + N, V, D, N, g)
    head = ah.PackedHead.from_components(h)
    Y = run(head, H_bits, 0, "f32")
    check_parity(to_f64(Y), oracle.logits_alt(H_bits, h), f"fmt={fmt} V={V} N={N}")
