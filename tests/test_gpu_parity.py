"""GPU parity: the HIP path against the fp64 oracle, element by element.

Bar (per output tensor): max|Y_gpu - Y_ref| <= 2e-3 * max|Y_ref|, every
element written (outputs are NaN-poisoned first), identical per-row argmax,
and bit-exact dequantised weights (one-hot hidden states make every logit a
single product, so Y equals the stored weight exactly).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import ah_mod, check_parity, device_H, log, run, to_f64, torch_mod

pytestmark = pytest.mark.gpu

DECODE, TILE = 1, 2


def _head(inp):
    return ah_mod().PackedHead.from_components(inp.head)


def test_tiny_workload_both_paths():
    inp = synth.make("tiny")
    log("tiny workload V=1024 D=256 N=4 r_c=16 r_r=8 g=64")
    head = _head(inp)
    Yr = oracle.logits(inp.H_bits, inp.head)
    for path in (DECODE, TILE):
        check_parity(to_f64(run(head, inp.H_bits, path)), Yr, f"tiny path={path}")


SHAPES = [
    # V (ragged: not a multiple of 16/64), D, r_c, r_r, g
    (1000, 512, 16, 8, 64),
    (1000, 512, 0, 0, 128),
    (777, 256, 8, 0, 32),
    (777, 384, 0, 24, 128),
    (530, 512, 40, 72, 256),
    (2048, 1024, 32, 32, 128),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 17, 63, 64, 65, 130])
def test_shapes_and_ragged_tails(shape, N):
    V, D, r_c, r_r, g = shape
    log(f"shape V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N}")
    inp = synth.make("tiny", seed=V + N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
    head = _head(inp)
    Yr = oracle.logits(inp.H_bits, inp.head)
    paths = (DECODE, TILE) if N <= 64 else (TILE,)
    outs = {}
    for path in paths:
        outs[path] = to_f64(run(head, inp.H_bits, path))
        check_parity(outs[path], Yr, f"path={path}")
    # the auto path takes the decode path up to 16 tokens, else the tile path,
    # and must give the same bits as the path it takes
    auto = to_f64(run(head, inp.H_bits, 0))
    assert np.array_equal(auto, outs[DECODE if N <= 16 else TILE])


LARGE_N_SHAPES = [
    (1000, 512, 16, 8, 64),   # odd number of 16-row blocks: the last 32-row block is half empty
    (2048, 1024, 32, 32, 128),
    (530, 512, 40, 72, 256),
    (777, 256, 8, 0, 32),
    (1000, 512, 0, 0, 128),
]


@pytest.mark.parametrize("shape", LARGE_N_SHAPES)
@pytest.mark.parametrize("N", [129, 300, 1100])
def test_large_n_tiles(shape, N):
    """N > 128: 256x256 workgroup tiles, ragged in tokens and vocabulary, with
    token-tile counts that leave partial groups and grid sizes that are not
    multiples of the XCD count."""
    V, D, r_c, r_r, g = shape
    log(f"large-N shape V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N}")
    inp = synth.make("tiny", seed=V + N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
    head = _head(inp)
    Yr = oracle.logits(inp.H_bits, inp.head)
    Yt = to_f64(run(head, inp.H_bits, TILE))
    check_parity(Yt, Yr, "path=tile")
    assert np.array_equal(to_f64(run(head, inp.H_bits, 0)), Yt)


@pytest.mark.parametrize("path,rows", [(DECODE, 64), (TILE, 64), (TILE, 256)])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_one_hot_rows_recover_weights_bit_exactly(path, g, rows):
    """H = unit rows e_k, r_c = r_r = 0: Y[n, v] = q4[v,k] * c8[v,k//g] * s_R[v],
    a single product of exact operands, so the GPU must return it exactly.
    256 rows take the large-N kernel, 64 rows the small-N ones."""
    V, D = 300, 512
    inp = synth.make("tiny", seed=g, V=V, D=D, N=1, r_c=0, r_r=0, g=g)
    h = inp.head
    # special values: extreme codes, c8 in {0, 255}, zero / subnormal / large scales
    h.q4[0, :] = -8
    h.q4[1, :] = 7
    h.c8[2, :] = 0
    h.c8[3, :] = 255
    h.s_R.view(np.uint16)[4] = 0x0001          # smallest subnormal
    h.s_R.view(np.uint16)[5] = 0x03FF          # largest subnormal
    h.s_R.view(np.uint16)[6] = 0x0000          # zero
    h.s_R.view(np.uint16)[7] = 0x7BFF          # 65504
    h.s_R.view(np.uint16)[8] = 0x8400          # negative scale
    ks = np.array(sorted(set([0, 1, 7, 8, 31, 32, 33, 63, 64, 127, 128, 255, 256, 300, 511] +
                             list(range(2, D, 37 if rows <= 64 else 3)))))
    ks = ks[ks < D][:rows]
    eye = np.zeros((ks.size, D), np.float32)
    eye[np.arange(ks.size), ks] = 1.0
    Hb = synth.f32_to_bf16_bits(eye)
    head = _head(inp)
    Y = run(head, Hb, path).cpu().numpy()
    R = oracle.dequant_R(h.q4, h.c8, h.s_R, g)          # exact in fp64 and fp32
    want = R[:, ks].T.astype(np.float32)
    # value equality (+0 and -0 are the same weight); no NaN anywhere
    assert not np.isnan(Y).any()
    assert np.array_equal(Y, want), f"max diff {np.abs(Y.astype(np.float64) - R[:, ks].T).max()}"


@pytest.mark.parametrize("path", [DECODE, TILE])
def test_low_rank_only_and_zero_head(path):
    inp = synth.make("tiny", seed=5, V=600, D=256, N=8, r_c=16, r_r=24, g=64)
    inp.head.q4[:] = 0
    head = _head(inp)
    check_parity(to_f64(run(head, inp.H_bits, path)), oracle.logits(inp.H_bits, inp.head), "low-rank only")
    z = synth.zero_head(600, 256, 16, 24, 64)
    Yz = to_f64(run(_head(synth.Inputs(inp.H_bits, z)), inp.H_bits, path))
    assert not Yz.any()


@pytest.mark.parametrize("path", [DECODE, TILE])
def test_hidden_state_edge_values(path):
    """All-zero rows, a row of tiny values, a row with a single huge value,
    and bf16 subnormals: the per-token fp16 scaling keeps them in range."""
    inp = synth.make("tiny", seed=9, V=400, D=256, N=6, r_c=8, r_r=8, g=64)
    H = inp.H_bits.copy()
    H[0] = 0
    H[1] = synth.f32_to_bf16_bits(np.full(256, 3e-30, np.float32))
    H[2] = 0
    H[2, 17] = synth.f32_to_bf16_bits(np.array([1e30], np.float32))[0]
    H[3] = synth.f32_to_bf16_bits(np.full(256, 5e4, np.float32) * np.sign(np.arange(256) - 127.5))
    H[4, ::3] = 0x0001                               # bf16 subnormals
    head = _head(inp)
    Yr = oracle.logits(H, inp.head)
    Yg = to_f64(run(head, H, path))
    assert not np.isnan(Yg).any()
    for n in range(6):
        scale = np.abs(Yr[n]).max()
        err = np.abs(Yg[n] - Yr[n]).max()
        assert err <= 2e-3 * scale or (scale == 0 and err == 0), (n, err, scale)


@pytest.mark.parametrize("path", [DECODE, TILE])
def test_deterministic(path):
    inp = synth.make("tiny", seed=3, V=2000, D=512, N=33, r_c=16, r_r=16, g=128)
    head = _head(inp)
    a = run(head, inp.H_bits, path).cpu().numpy()
    b = run(head, inp.H_bits, path).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("path", [DECODE, TILE])
def test_bf16_output_is_rounded_fp32_output(path):
    torch = torch_mod()
    inp = synth.make("tiny", seed=11, V=1500, D=256, N=20, r_c=16, r_r=8, g=64)
    head = _head(inp)
    y32 = run(head, inp.H_bits, path, "f32")
    y16 = run(head, inp.H_bits, path, "bf16")
    assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))


def test_row_strides_and_offsets():
    """H and Y as row-strided views into larger buffers."""
    torch = torch_mod()
    ah = ah_mod()
    inp = synth.make("tiny", seed=13, V=500, D=256, N=10, r_c=8, r_r=8, g=64)
    head = _head(inp)
    Hbig = torch.zeros((10, 256 + 64), dtype=torch.bfloat16, device="cuda")
    Hbig[:, 8:8 + 256] = device_H(inp.H_bits)
    H = Hbig[:, 8:8 + 256]
    Ybig = torch.full((10, 700), float("nan"), device="cuda")
    Y = Ybig[:, 100:600]
    Yr = oracle.logits(inp.H_bits, inp.head)
    for path in (DECODE, TILE):
        ah.archead_logits_path(H, head, Y, path)
        torch.cuda.synchronize()
        check_parity(Y.cpu().numpy().astype(np.float64), Yr, f"strided path={path}")
        assert torch.isnan(Ybig[:, :100]).all() and torch.isnan(Ybig[:, 600:]).all()


@pytest.mark.parametrize("N", [40, 200])
def test_split_tiles_with_unaligned_outputs(N):
    """Few vocabulary tiles on a deep hidden dimension: the tile path splits
    every tile's hidden dimension over several workgroups and adds the parts
    in a second kernel; here into fp32 and bf16 outputs whose rows are
    neither 16-byte aligned nor a multiple of 4 elements apart."""
    torch = torch_mod()
    ah = ah_mod()
    V, D = 1000, 2048
    inp = synth.make("tiny", seed=N, V=V, D=D, N=N, r_c=16, r_r=8, g=64, n_outlier=4)
    head = _head(inp)
    H = device_H(inp.H_bits)
    Yr = oracle.logits(inp.H_bits, inp.head)
    for dt in (torch.float32, torch.bfloat16):
        Ybig = torch.full((N, V + 7), float("nan"), dtype=dt, device="cuda")
        Y = Ybig[:, 3:3 + V]  # row stride V + 7, start 3 elements in
        ah.archead_logits_path(H, head, Y, TILE)
        torch.cuda.synchronize()
        assert torch.isnan(Ybig[:, :3]).all() and torch.isnan(Ybig[:, 3 + V:]).all()
        Yg = Y.float().cpu().numpy().astype(np.float64)
        if dt == torch.float32:
            check_parity(Yg, Yr, f"split N={N} fp32")
            y32 = Y.clone()
        else:
            assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), Y.contiguous().view(torch.int16))
