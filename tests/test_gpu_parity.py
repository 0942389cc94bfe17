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


def decode_takes(D, r_c, r_r, g, N):
    """The decode path's rule for the shapes below: every call of up to 16
    tokens; 17 to 64 tokens (the batched kernel) when the ranks rounded up to
    32 sum to at most 128, a row has at most 64 groups and D is a multiple of
    512."""
    up32 = lambda x: (x + 31) // 32 * 32
    return N <= 16 or (N <= 64 and up32(r_c) + up32(r_r) <= 128 and D // g <= 64 and D % 512 == 0)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 16, 17, 24, 33, 48, 63, 64, 65, 130])
def test_shapes_and_ragged_tails(shape, N):
    V, D, r_c, r_r, g = shape
    log(f"shape V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N}")
    inp = synth.make("tiny", seed=V + N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
    head = _head(inp)
    Yr = oracle.logits(inp.H_bits, inp.head)
    dec = decode_takes(D, r_c, r_r, g, N)
    assert ah_mod().archead_main_kernel(V, D, r_c, r_r, g, N) == (
        "tile32_kernel" if not dec else "batch_kernel" if N > 16 else
        ah_mod().archead_main_kernel(V, D, r_c, r_r, g, N, DECODE))
    paths = (DECODE, TILE) if dec else (TILE,)
    outs = {}
    for path in paths:
        outs[path] = to_f64(run(head, inp.H_bits, path))
        check_parity(outs[path], Yr, f"path={path}")
    # the auto path takes the decode path when it can, else the tile path, and
    # must give the same bits as the path it takes
    auto = to_f64(run(head, inp.H_bits, 0))
    assert np.array_equal(auto, outs[DECODE if dec else TILE])
    if not dec:  # a forced decode path it does not take is refused
        with pytest.raises(ah_mod().ArcheadError, match="UNSUPPORTED"):
            run(head, inp.H_bits, DECODE)


# More groups per row than the tile and batched kernels' group-code tables hold
# (D/g > 64): the decode kernel for up to 16 tokens reads the group codes with
# every tile and takes them; the other paths refuse them.
MANY_GROUPS = [(1000, 4096, 16, 16, 32), (600, 8192, 16, 8, 64)]


@pytest.mark.parametrize("shape", MANY_GROUPS)
@pytest.mark.parametrize("N", [1, 7, 8])
def test_many_groups_per_row_decode(shape, N):
    V, D, r_c, r_r, g = shape
    log(f"many groups V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N}")
    inp = synth.make("tiny", seed=V + N + g, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
    head = _head(inp)
    Yr = oracle.logits(inp.H_bits, inp.head)
    Yd = to_f64(run(head, inp.H_bits, DECODE))
    check_parity(Yd, Yr, "decode")
    assert np.array_equal(to_f64(run(head, inp.H_bits, 0)), Yd)
    with pytest.raises(ah_mod().ArcheadError, match="UNSUPPORTED"):
        run(head, inp.H_bits, TILE)
    for n in (17, 64):  # past 16 tokens: no path takes such a head
        with pytest.raises(ah_mod().ArcheadError, match="UNSUPPORTED"):
            run(head, np.repeat(inp.H_bits[:1], n, axis=0), 0)


# Few-token calls whose copy of H and Z needs more than 76 KiB of LDS: the
# few-token kernel runs one workgroup of 16 waves per CU that shares one copy
# (up to 152 KiB: 16 tokens at D = 4096, 8 at D = 8192) instead of two of 8
# waves; past that another kernel takes the call.
WIDE = [(1000, 4096, 32, 32, 128), (700, 8192, 16, 16, 128), (900, 4096, 8, 24, 32), (800, 2048, 16, 16, 64)]


@pytest.mark.parametrize("shape", WIDE)
@pytest.mark.parametrize("N", [3, 5, 8, 9, 12, 16])
def test_few_token_wide_workgroup(shape, N):
    V, D, r_c, r_r, g = shape
    lds = (N + 1) * (D + 8) * 2 + N * (r_c + r_r) * 4
    kern = ah_mod().archead_main_kernel(V, D, r_c, r_r, g, N)
    log(f"few-token wide V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N} lds={lds} -> {kern}")
    assert (kern == "small_decode_kernel") == (lds <= 152 * 1024)
    inp = synth.make("tiny", seed=V + D + N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=8)
    head = _head(inp)
    Yr = oracle.logits(inp.H_bits, inp.head)
    Yd = to_f64(run(head, inp.H_bits, 0))
    check_parity(Yd, Yr, f"auto {kern}")
    if kern != "tile32_kernel":
        assert np.array_equal(to_f64(run(head, inp.H_bits, DECODE)), Yd)
    torch = torch_mod()
    y16 = run(head, inp.H_bits, 0, "bf16")
    assert torch.equal(torch.from_numpy(Yd.astype(np.float32)).to(torch.bfloat16).view(torch.int16),
                       y16.cpu().view(torch.int16))


@pytest.mark.parametrize("g", [32, 128])
def test_one_hot_wide_workgroup_bit_exact(g):
    """One-hot hidden states, 16 per call at D = 4096 (the 16-wave few-token
    workgroup): every stored weight comes back exactly."""
    V, D = 400, 4096
    inp = synth.make("tiny", seed=g + 1, V=V, D=D, N=1, r_c=0, r_r=0, g=g)
    h = inp.head
    h.q4[0, :] = -8
    h.c8[1, :] = 255
    h.s_R.view(np.uint16)[2] = 0x0001
    ks = np.array(sorted(set([0, 1, 31, 32, 127, 128, 511, 512, 2047, 2048, 4095] + list(range(3, D, 97)))))
    assert ah_mod().archead_main_kernel(V, D, 0, 0, g, 16) == "small_decode_kernel"
    eye = np.zeros((ks.size, D), np.float32)
    eye[np.arange(ks.size), ks] = 1.0
    Hb = synth.f32_to_bf16_bits(eye)
    head = _head(inp)
    Y = np.concatenate([run(head, Hb[i:i + 16], DECODE).cpu().numpy() for i in range(0, ks.size, 16)])
    want = oracle.dequant_R(h.q4, h.c8, h.s_R, g)[:, ks].T.astype(np.float32)
    assert not np.isnan(Y).any()
    assert np.array_equal(Y, want)


# The few-token pre-projection splits each element of Z over slices of D
# (D/512 slices for up to 2 tokens, D/1024 up to 8, D/2048 beyond, at least
# one), which need not divide the row's 8-column chunks evenly.
@pytest.mark.parametrize("D", [1536, 2560])
@pytest.mark.parametrize("N", [1, 2, 3, 9])
def test_few_token_uneven_z_slices(D, N):
    V, r_c, r_r, g = 900, 16, 24, 128
    log(f"few-token Z slices V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N}")
    assert ah_mod().archead_main_kernel(V, D, r_c, r_r, g, N) == "small_decode_kernel"
    inp = synth.make("tiny", seed=D + N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
    head = _head(inp)
    check_parity(to_f64(run(head, inp.H_bits, 0)), oracle.logits(inp.H_bits, inp.head), f"D={D} N={N}")


# The tile path's fp32 Z over parts of the hidden dimension: up to D/2048
# parts (D/4096 for g = 256) when the 32-token x 32-rank tiles alone give
# fewer than about 128 workgroups.
@pytest.mark.parametrize("shape,N", [((700, 8192, 32, 32, 128), 70), ((700, 8192, 32, 32, 256), 100),
                                     ((700, 4096, 32, 32, 64), 130), ((500, 8192, 64, 64, 128), 300)])
def test_tile_z_parts(shape, N):
    V, D, r_c, r_r, g = shape
    log(f"tile Z parts V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N}")
    inp = synth.make("tiny", seed=V + D + N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
    head = _head(inp)
    check_parity(to_f64(run(head, inp.H_bits, TILE)), oracle.logits(inp.H_bits, inp.head), "tile")


# 64 groups per row (D/g = 64) and D = 8192 on the batched kernel
@pytest.mark.parametrize("N", [17, 40, 64])
def test_batched_deep_rows(N):
    V, D, r_c, r_r, g = 700, 8192, 32, 32, 128
    log(f"batched deep rows V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N}")
    inp = synth.make("tiny", seed=N + 7, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=8)
    head = _head(inp)
    assert ah_mod().archead_main_kernel(V, D, r_c, r_r, g, N) == "batch_kernel"
    Yr = oracle.logits(inp.H_bits, inp.head)
    Yd = to_f64(run(head, inp.H_bits, DECODE))
    check_parity(Yd, Yr, "batched D=8192")
    check_parity(to_f64(run(head, inp.H_bits, TILE)), Yr, "tile D=8192")


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


@pytest.mark.parametrize("path,rows,step", [(DECODE, 64, 16), (DECODE, 64, 64), (DECODE, 60, 20),
                                            (TILE, 64, 64), (TILE, 256, 256)])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_one_hot_rows_recover_weights_bit_exactly(path, g, rows, step):
    """H = unit rows e_k, r_c = r_r = 0: Y[n, v] = q4[v,k] * c8[v,k//g] * s_R[v],
    a single product of exact operands, so the GPU must return it exactly.
    The tile path takes 64 or 256 rows per call (its two token-tile sizes);
    the decode path 16 per call (its k-tile-major kernel), or 64 or 20 (its
    batched kernel)."""
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
    Y = np.concatenate([run(head, Hb[i:i + step], path).cpu().numpy() for i in range(0, ks.size, step)])
    R = oracle.dequant_R(h.q4, h.c8, h.s_R, g)          # exact in fp64 and fp32
    want = R[:, ks].T.astype(np.float32)
    # value equality (+0 and -0 are the same weight); no NaN anywhere
    assert not np.isnan(Y).any()
    assert np.array_equal(Y, want), f"max diff {np.abs(Y.astype(np.float64) - R[:, ks].T).max()}"


@pytest.mark.parametrize("path,N", [(DECODE, 8), (DECODE, 40), (TILE, 8)])
def test_low_rank_only_and_zero_head(path, N):
    D = 512  # a multiple of 512: the batched kernel takes the 40-token call
    inp = synth.make("tiny", seed=5, V=600, D=D, N=N, r_c=16, r_r=24, g=64)
    inp.head.q4[:] = 0
    head = _head(inp)
    check_parity(to_f64(run(head, inp.H_bits, path)), oracle.logits(inp.H_bits, inp.head), "low-rank only")
    z = synth.zero_head(600, D, 16, 24, 64)
    Yz = to_f64(run(_head(synth.Inputs(inp.H_bits, z)), inp.H_bits, path))
    assert not Yz.any()


@pytest.mark.parametrize("path,N", [(DECODE, 6), (DECODE, 21), (TILE, 6)])
def test_hidden_state_edge_values(path, N):
    """All-zero rows, a row of tiny values, a row with a single huge value,
    and bf16 subnormals: the per-token fp16 scaling keeps them in range."""
    D = 512
    inp = synth.make("tiny", seed=9, V=400, D=D, N=N, r_c=8, r_r=8, g=64)
    H = inp.H_bits.copy()
    H[0] = 0
    H[1] = synth.f32_to_bf16_bits(np.full(D, 3e-30, np.float32))
    H[2] = 0
    H[2, 17] = synth.f32_to_bf16_bits(np.array([1e30], np.float32))[0]
    H[3] = synth.f32_to_bf16_bits(np.full(D, 5e4, np.float32) * np.sign(np.arange(D) - 255.5))
    H[4, ::3] = 0x0001                               # bf16 subnormals
    head = _head(inp)
    Yr = oracle.logits(H, inp.head)
    Yg = to_f64(run(head, H, path))
    assert not np.isnan(Yg).any()
    for n in range(N):
        scale = np.abs(Yr[n]).max()
        err = np.abs(Yg[n] - Yr[n]).max()
        assert err <= 2e-3 * scale or (scale == 0 and err == 0), (n, err, scale)


@pytest.mark.parametrize("path,N", [(DECODE, 13), (DECODE, 50), (TILE, 33)])
def test_deterministic(path, N):
    inp = synth.make("tiny", seed=3, V=2000, D=512, N=N, r_c=16, r_r=16, g=128)
    head = _head(inp)
    a = run(head, inp.H_bits, path).cpu().numpy()
    b = run(head, inp.H_bits, path).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("path,N", [(DECODE, 12), (DECODE, 45), (TILE, 20)])
def test_bf16_output_is_rounded_fp32_output(path, N):
    torch = torch_mod()
    inp = synth.make("tiny", seed=11, V=1500, D=512, N=N, r_c=16, r_r=8, g=64)
    head = _head(inp)
    y32 = run(head, inp.H_bits, path, "f32")
    y16 = run(head, inp.H_bits, path, "bf16")
    assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))


@pytest.mark.parametrize("N", [10, 30])
def test_row_strides_and_offsets(N):
    """H and Y as row-strided views into larger buffers."""
    torch = torch_mod()
    ah = ah_mod()
    D = 512
    inp = synth.make("tiny", seed=13, V=500, D=D, N=N, r_c=8, r_r=8, g=64)
    head = _head(inp)
    Hbig = torch.zeros((N, D + 64), dtype=torch.bfloat16, device="cuda")
    Hbig[:, 8:8 + D] = device_H(inp.H_bits)
    H = Hbig[:, 8:8 + D]
    Ybig = torch.full((N, 700), float("nan"), device="cuda")
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


# archead_logits_events: the launches record the caller's events (main
# kernel start, last kernel end); the logits are those of archead_logits_path,
# and a later call without events leaves the events as they were.
EVENT_CASES = [
    # label, V, D, r_c, r_r, g, N, path, comparison format (0: ARCHead)
    ("few-token", 1000, 512, 16, 8, 64, 4, 0, 0),
    ("few-token 16 waves", 900, 4096, 16, 16, 128, 12, 0, 0),
    ("k-tile-major", 777, 384, 0, 24, 128, 5, 0, 0),
    ("batched", 1000, 512, 16, 8, 64, 40, 0, 0),
    ("tile", 2048, 1024, 32, 32, 128, 300, 2, 0),
    ("tile, split tail", 2048, 1024, 32, 32, 128, 1100, 2, 0),
    ("group INT4, three launches", 777, 512, 0, 0, 64, 70, 0, 1),
]


@pytest.mark.parametrize("label,V,D,r_c,r_r,g,N,path,fmt", EVENT_CASES)
def test_logits_events_from_the_launches(label, V, D, r_c, r_r, g, N, path, fmt):
    torch = torch_mod()
    ah = ah_mod()
    log(f"events {label}: V={V} D={D} r_c={r_c} r_r={r_r} g={g} N={N} path={path} fmt={fmt}")
    if fmt:
        H_bits, h = synth.make_alt(fmt, V + N, V, D, N, g)
    else:
        h = synth.make("tiny", seed=V + N, V=V, D=D, N=N, r_c=r_c, r_r=r_r, g=g, n_outlier=4)
        H_bits, h = h.H_bits, h.head
    head = ah.PackedHead.from_components(h)
    H = device_H(H_bits)
    y_plain = run(head, H_bits, path, H_dev=H)
    eb, ee = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eb.record()
    ee.record()
    Y = torch.full((N, V), float("nan"), device="cuda")
    ah.archead_logits_events(H, head, Y, path, eb, ee)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int32), y_plain.view(torch.int32))
    span = eb.elapsed_time(ee)
    assert span > 0.0
    run(head, H_bits, path, H_dev=H)  # no events: the pair keeps its times
    assert eb.elapsed_time(ee) == span
