"""GPU parity of archead_logit_error (Eq. 1's logit error of a packed head
against its dense original) with the oracle's fp64 logit_error.

Tolerances: the reference energy sum (H W^T)^2 within 1e-4 (fp32 logits of
a bf16 product); the error sum within 2e-3 of the oracle's when the packed
head approximates W (the GPU's per-logit error, about 1e-6 of max|Y|, is
small against logit differences of about 1e-2 of |Y|), and within 1e-4 for an
unrelated head.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import ah_mod, device_H, log, torch_mod

pytestmark = pytest.mark.gpu


def _gpu(head_components, H_bits, W_bits):
    torch = torch_mod()
    ah = ah_mod()
    head = ah.PackedHead.from_components(head_components)
    W = torch.from_numpy(np.ascontiguousarray(W_bits).view(np.int16)).view(torch.bfloat16).to("cuda")
    return ah.archead_logit_error(device_H(H_bits), head, W)


@pytest.mark.parametrize("N", [1, 300, 600])
def test_logit_error_of_a_quantized_head(N):
    V, D, r_c, r_r, g = 1000, 512, 16, 8, 64
    log(f"logit error, quantized head, V={V} D={D} N={N}")
    dense = synth.draw_dense(np.random.default_rng(N), V, D, r_c, r_r, "bf16")
    head, _ = oracle.quantize(dense.W, dense.A_c, dense.B_c, dense.A_w, dense.B_w, g)
    H = synth.make("tiny", seed=N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g).H_bits
    err, ref = _gpu(head, H, dense.W)
    err_o, ref_o = oracle.logit_error(H, head, dense.W)
    log(f"  error {err:.6e} vs {err_o:.6e}; reference {ref:.6e} vs {ref_o:.6e}")
    assert abs(ref - ref_o) <= 1e-4 * ref_o
    assert abs(err - err_o) <= 2e-3 * err_o


def test_logit_error_of_an_unrelated_head():
    V, D, N = 777, 256, 40
    inp = synth.make("tiny", seed=9, V=V, D=D, N=N, r_c=8, r_r=8, g=32)
    W = synth.f32_to_bf16_bits(np.random.default_rng(4).normal(0, 0.05, size=(V, D)).astype(np.float32))
    err, ref = _gpu(inp.head, inp.H_bits, W)
    err_o, ref_o = oracle.logit_error(inp.H_bits, inp.head, W)
    assert abs(ref - ref_o) <= 1e-4 * ref_o and abs(err - err_o) <= 1e-4 * err_o


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_logit_error_full_size_batched():
    """The batched workload (V=151936, D=4096, N=64): its seeded packed head
    against an independent seeded dense bf16 head, every logit, against the
    oracle's fp64 sums."""
    cfg = synth.config("batched")
    inp = synth.make("batched")
    V, D = cfg["V"], cfg["D"]
    log(f"full-size logit error V={V} D={D} N={cfg['N']}")
    W = synth.f32_to_bf16_bits(np.random.default_rng(31).normal(0, 0.02, size=(V, D)).astype(np.float32))
    err, ref = _gpu(inp.head, inp.H_bits, W)
    err_o, ref_o = oracle.logit_error(inp.H_bits, inp.head, W)
    log(f"  error {err:.6e} vs {err_o:.6e}; reference {ref:.6e} vs {ref_o:.6e}")
    assert abs(ref - ref_o) <= 1e-4 * ref_o and abs(err - err_o) <= 1e-4 * err_o
