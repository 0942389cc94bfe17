"""GPU parity on the four full-size workloads, in the launch configuration the
benchmark times (one archead_logits call on the whole batch).

decode / batched / head70b: every row is compared with the oracle.  prefill
(N=4096): 48 seeded rows, including the first and last, are compared with the
oracle on the fp32-output run; the bf16-output run (the timed format) must
equal the fp32 run rounded to bf16 on every element, and stay within
2e-3*max|Y_ref| + 2^-8*|Y_ref| of the oracle on the sampled rows (bf16 output
rounding alone can exceed 2e-3*max|Y|).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import ah_mod, check_parity, device_H, log, run, to_f64, torch_mod

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "batched", "head70b", "prefill"])
def test_full_size_workload(name):
    torch = torch_mod()
    ah = ah_mod()
    cfg = synth.config(name)
    log(f"full-size {name}: {cfg}")
    inp = synth.make(name)
    head = ah.PackedHead.from_components(inp.head)
    N = cfg["N"]
    if N <= 256:
        rows = np.arange(N)
    else:
        rng = np.random.default_rng(1234)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 46, replace=False)]))
    H = device_H(inp.H_bits)
    Yr = oracle.logits(inp.H_bits, inp.head, rows=rows)
    paths = (0, 2) if N <= 64 else (0,)  # auto = decode path up to 64 tokens; forced tile path
    for path in paths:
        Y = run(head, inp.H_bits, path, "f32", H_dev=H)
        check_parity(to_f64(Y[torch.as_tensor(rows, device="cuda")]), Yr, f"{name} path={path}")
        if path == 0:
            y32 = Y
    if cfg["y_dtype"] == "bf16":
        y16 = run(head, inp.H_bits, 0, "bf16", H_dev=H)
        assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))
        Ys = to_f64(y16[torch.as_tensor(rows, device="cuda")])
        bound = 2e-3 * np.abs(Yr).max() + 2.0 ** -8 * np.abs(Yr)
        assert (np.abs(Ys - Yr) <= bound).all()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("N", [3, 9, 17, 63])
def test_full_size_decode_head_token_counts(N):
    """The decode head (V=151936, D=4096, r_c=r_r=32, g=128) at token counts
    that run the other decode-path kernels and workgroup shapes: 3 (two 8-wave
    few-token workgroups per CU), 9 (one 16-wave workgroup), 17 and 63 (the
    batched kernel with two and four token tiles); every row against the
    oracle."""
    ah = ah_mod()
    cfg = synth.config("decode")
    log(f"full-size decode head, N={N}")
    inp = synth.make("decode", N=N)
    head = ah.PackedHead.from_components(inp.head)
    want = "small_decode_kernel" if N <= 16 else "batch_kernel"
    assert ah.archead_main_kernel(cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"], N) == want
    Yr = oracle.logits(inp.H_bits, inp.head)
    check_parity(to_f64(run(head, inp.H_bits, 0)), Yr, f"decode head N={N}")
