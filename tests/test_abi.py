"""The C-ABI library on the host: exports, layout, packer and argument checks.

No test here launches a kernel: each call either is pure host work or fails
validation before the first HIP call, so the file runs without a GPU.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import ROOT


@pytest.fixture(scope="module")
def ah():
    lib_path = os.path.join(ROOT, "compressed_output_head_amd", "libarchead.so")
    if not os.path.exists(lib_path):
        import runpy
        runpy.run_path(os.path.join(ROOT, "compressed_output_head_amd", "build.py"))["build"]()
    import compressed_output_head_amd as m
    return m


def test_exports_match_header(ah):
    hdr = open(os.path.join(ROOT, "include", "archead.h")).read()
    declared = set(re.findall(r"ARCHEAD_API\s+[\w\s\*]*?\b(archead_\w+)\s*\(", hdr))
    assert declared == set(ah.EXPORTS)
    for name in declared:
        assert hasattr(ah.lib, name), name
    assert ah.archead_format_version() == oracle.FORMAT_VERSION


DIMS = [(1024, 256, 16, 8, 64), (151936, 4096, 32, 32, 128), (151936, 4096, 64, 64, 128),
        (128256, 8192, 64, 64, 128), (20, 256, 8, 8, 64), (1, 128, 0, 0, 32), (37, 384, 0, 24, 2),
        (1000, 512, 6, 6, 128)]


@pytest.mark.parametrize("dims", DIMS)
def test_layout_matches_oracle(ah, dims):
    a = ah.archead_pack_layout(*dims)
    b = oracle.layout(*dims)
    for n in ["header", "r_codes", "r_gcodes", "r_rowscale", "a_codes", "a_scales", "b_codes", "b_scales"]:
        assert tuple(a[n]) == tuple(b[n]), n
    assert a["total_bytes"] == b["total_bytes"] and a["payload_bytes"] == b["payload_bytes"]
    assert a["V16"] == b["V16"] and a["alignment"] == 256


@pytest.mark.parametrize("V,D,r_c,r_r,g", [(1024, 256, 16, 8, 64), (37, 128, 0, 0, 128), (50, 512, 0, 24, 32),
                                           (16, 256, 40, 0, 256), (129, 384, 8, 8, 64), (3, 256, 6, 2, 8)])
def test_library_packer_matches_oracle_packer(ah, V, D, r_c, r_r, g):
    h = synth.draw_head(np.random.default_rng(V * 7 + D), V, D, r_c, r_r, g)
    assert np.array_equal(ah.archead_pack(h), oracle.pack(h))


def test_library_packer_golden_positions(ah, golden_dir):
    G = json.load(open(os.path.join(golden_dir, "format_v1_cases.json")))
    d = G["dims"]
    h = synth.zero_head(d["V"], d["D"], d["r_c"], d["r_r"], d["g"])
    for c in G["nibbles"]:
        h.q4[c["v"], c["k"]] = c["code"]
    buf = ah.archead_pack(h)
    for c in G["nibbles"]:
        byte = int(buf[c["byte"]])
        nib = byte & 0xF if c["half"] == "lo" else byte >> 4
        assert nib == c["code"] & 0xF, c


def test_pack_rejects_bad_codes_and_small_buffers(ah):
    h = synth.draw_head(np.random.default_rng(1), 32, 128, 8, 8, 32)
    h.q4[3, 5] = 8
    with pytest.raises(ah.ArcheadError) as e:
        ah.archead_pack(h)
    assert e.value.status == 9
    h.q4[3, 5] = -9
    with pytest.raises(ah.ArcheadError):
        ah.archead_pack(h)
    h.q4[3, 5] = 0
    d = ah.ArcheadDims(32, 128, 8, 8, 32)
    comp = ah.ArcheadHostComponents()
    arrs = {}
    for n in ("q4", "c8", "s_R", "A_c", "A_w", "s_Ac", "s_Aw", "B_c", "B_w", "s_Bc", "s_Bw"):
        arrs[n] = np.ascontiguousarray(getattr(h, n))
        setattr(comp, n, arrs[n].ctypes.data)
    total = ah.archead_pack_layout(32, 128, 8, 8, 32)["total_bytes"]
    out = np.zeros(total, np.uint8)
    assert ah.lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), out.ctypes.data, total - 1) == 10
    assert ah.lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), None, total) == 1
    comp.A_w = None
    assert ah.lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), out.ctypes.data, total) == 1


def test_layout_dims_errors(ah):
    L = ah.ArcheadLayout()
    for dims, want in [((0, 256, 0, 0, 64), 2), ((16, 200, 0, 0, 8), 2), ((16, 256, 0, 0, 3), 2),
                       ((16, 256, -1, 0, 64), 2), ((16, 256, 0, 0, 96), 2), ((1 << 32, 256, 0, 0, 64), 3)]:
        assert ah.lib.archead_pack_layout(ctypes.byref(ah.ArcheadDims(*dims)), ctypes.byref(L)) == want, dims
    assert ah.lib.archead_pack_layout(None, ctypes.byref(L)) == 1
    assert ah.lib.archead_pack_layout(ctypes.byref(ah.ArcheadDims(16, 256, 0, 0, 64)), None) == 1


def _zmm_parts(N, D, r, g):
    """Parts of the k range of the tile path's fp32 Z: workgroups (32-token by
    32-rank tiles) times parts reach about 128, each of the 16 waves of a part
    keeps at least one unit of whole groups."""
    n32 = (N + 31) // 32 * 32
    base = (n32 // 32) * ((r + 31) // 32)
    units = D // 128 // (g // 128 if g > 128 else 1)
    p = min(-(-128 // base) if base else 1, units // 16)
    return max(p, 1)


def _tile_workspace(V, D, r_c, r_r, g, N):
    """hf (N32*D*2) | hscale (N32*4) | zf (N32*2*(rc32+rr32)*2) | zscale (N32*4) |
    z32 (parts*N32*r*4) | split-tile partial sums (64 MiB); each 256-aligned."""
    up = lambda x: (x + 255) // 256 * 256
    n32 = (N + 31) // 32 * 32
    rc32, rr32 = (r_c + 31) // 32 * 32, (r_r + 31) // 32 * 32
    r = r_c + r_r
    parts = _zmm_parts(N, D, r, g) if r else 1
    return (up(n32 * D * 2) + up(n32 * 4) + up(n32 * 2 * (rc32 + rr32) * 2) + up(n32 * 4) +
            up(parts * n32 * r * 4) + (64 << 20))


def _few_tokens(V, D, r_c, r_r, g, N):
    """The few-token decode kernel takes the call: H (N + 1 rows of D + 8
    halves) and Z (N r fp32) within 152 KiB of LDS (two workgroups of 8 waves
    per CU up to 76 KiB, else one of 16 waves), k-tiles a multiple of 4."""
    return 1 <= N <= 16 and (D // 128) % 4 == 0 and (N + 1) * (D + 8) * 2 + N * (r_c + r_r) * 4 <= 152 * 1024


def _batched(V, D, r_c, r_r, g, N):
    """The batched decode kernel takes the call: 17 to 64 tokens, ranks rounded
    up to 32 summing to at most 128, at most 64 groups per row, D a multiple
    of 512."""
    up32 = lambda x: (x + 31) // 32 * 32
    return 17 <= N <= 64 and up32(r_c) + up32(r_r) <= 128 and D // g <= 64 and D % 512 == 0


def test_workspace_bytes(ah):
    # calls the decode kernel takes (up to 16 tokens whose H fits its LDS,
    # 32-rank steps rc32 + rr32 <= 256) need the partial sums of Z; the tile
    # path needs its operand fragments and the split-tile partial sums
    for (V, D, r_c, r_r, g), N, decode in [((1024, 256, 16, 8, 64), 4, True), ((151936, 4096, 32, 32, 128), 1, True),
                                           ((1024, 256, 64, 96, 64), 4, True), ((1024, 256, 64, 96, 64), 16, True),
                                           ((1024, 256, 129, 128, 64), 1, False),
                                           ((151936, 4096, 32, 32, 128), 16, True),
                                           ((128256, 8192, 64, 64, 128), 8, True),
                                           ((128256, 8192, 64, 64, 128), 9, False),
                                           ((151936, 4096, 64, 64, 128), 4096, False), ((64, 128, 0, 0, 32), 17, False),
                                           ((64, 512, 0, 0, 32), 17, True),
                                           ((151936, 4096, 32, 32, 128), 64, True),
                                           ((151936, 4096, 32, 32, 128), 65, False),
                                           ((1024, 256, 64, 96, 64), 17, False),
                                           ((1000, 4096, 16, 16, 64), 40, True),
                                           ((1000, 4096, 16, 16, 32), 63, False)]:
        up = lambda x: (x + 255) // 256 * 256
        if not decode:
            want = _tile_workspace(V, D, r_c, r_r, g, N)
        elif _few_tokens(V, D, r_c, r_r, g, N) or _batched(V, D, r_c, r_r, g, N):
            # converted H [N][D] fp16, its scales, Z [S][N][r] fp32: partial sums over S
            # slices of D for the few-token kernel (one to four 8-column chunks per
            # lane as N grows), S = 1 for the batched kernel
            cpl = 1 if N <= 2 else 2 if N <= 8 else 4
            S = max(1, D // (512 * cpl)) if _few_tokens(V, D, r_c, r_r, g, N) else 1
            want = up(N * D * 2) + up(N * 4) + up(S * N * (r_c + r_r) * 4)
        else:  # Z partial sums per element: slices of 8 k-tiles, padded to 4
            zst = (-(-(D // 128) // 8) + 3) // 4 * 4
            want = up(N * (r_c + r_r) * zst * 4)
        assert ah.archead_workspace_bytes(V, D, r_c, r_r, g, N) == want, (V, D, N)
        assert ah.archead_workspace_bytes_path(V, D, r_c, r_r, g, N, 0) == want
        assert ah.archead_workspace_bytes_path(V, D, r_c, r_r, g, N, 1) == want
        assert ah.archead_workspace_bytes_path(V, D, r_c, r_r, g, N, 2) == _tile_workspace(V, D, r_c, r_r, g, N)
        kern = ("tile32_kernel" if not decode else
                "small_decode_kernel" if _few_tokens(V, D, r_c, r_r, g, N) else
                "batch_kernel" if _batched(V, D, r_c, r_r, g, N) else "decode_kernel")
        assert ah.archead_main_kernel(V, D, r_c, r_r, g, N) == kern, (V, D, N)
        assert ah.archead_main_kernel(V, D, r_c, r_r, g, N, 2) == "tile32_kernel"
        if decode:
            assert ah.archead_main_kernel(V, D, r_c, r_r, g, N, 1) == kern
        else:
            with pytest.raises(ah.ArcheadError):
                ah.archead_main_kernel(V, D, r_c, r_r, g, N, 1)
    assert ah.archead_workspace_bytes(1024, 256, 16, 8, 64, 0) == 0
    with pytest.raises(ah.ArcheadError):
        ah.archead_workspace_bytes_path(1024, 256, 16, 8, 64, 4, 3)


# ------------------------------------------------ argument checks of logits ---

FAKE = 1 << 40  # never dereferenced: every call below fails validation first


def _args(ah, N=4, V=1024, D=256, r_c=16, r_r=8, g=64, ydt=2, hdt=1, ws=None, buf=None):
    try:
        total = ah.archead_pack_layout(V, D, r_c, r_r, g)["total_bytes"]
        need = ah.archead_workspace_bytes(V, D, r_c, r_r, g, N)
    except ah.ArcheadError:
        total = need = 1 << 20
    H = ah.ArcheadTensor(FAKE, N, D, D, hdt)
    Y = ah.ArcheadTensor(FAKE + (1 << 30), N, V, V, ydt)
    P = ah.ArcheadPackedHead(ah.ArcheadDims(V, D, r_c, r_r, g), FAKE + (2 << 30),
                             total if buf is None else buf, FAKE + (3 << 30), need if ws is None else ws)
    return H, P, Y, need, total


def _call(ah, H, P, Y, path=0):
    return ah.lib.archead_logits_path(ctypes.byref(H), ctypes.byref(P), ctypes.byref(Y), path, None)


def test_logits_error_paths(ah):
    H, P, Y, need, total = _args(ah)
    assert ah.lib.archead_logits(None, ctypes.byref(P), ctypes.byref(Y), None) == 1
    assert ah.lib.archead_logits(ctypes.byref(H), None, ctypes.byref(Y), None) == 1
    assert ah.lib.archead_logits(ctypes.byref(H), ctypes.byref(P), None, None) == 1

    cases = []
    H, P, Y, need, total = _args(ah, hdt=2); cases.append((H, P, Y, 0, 4))            # H not bf16
    H, P, Y, need, total = _args(ah, ydt=3); cases.append((H, P, Y, 0, 4))            # Y dtype
    H, P, Y, need, total = _args(ah); H.cols = 255; cases.append((H, P, Y, 0, 5))      # D mismatch
    H, P, Y, need, total = _args(ah); Y.cols = 1000; cases.append((H, P, Y, 0, 5))     # V mismatch
    H, P, Y, need, total = _args(ah); Y.rows = 5; cases.append((H, P, Y, 0, 5))        # N mismatch
    H, P, Y, need, total = _args(ah); H.row_stride = 100; cases.append((H, P, Y, 0, 5))
    H, P, Y, need, total = _args(ah); H.rows = Y.rows = -1; cases.append((H, P, Y, 0, 5))
    H, P, Y, need, total = _args(ah, g=16); cases.append((H, P, Y, 0, 3))             # g unsupported
    H, P, Y, need, total = _args(ah, r_c=12); cases.append((H, P, Y, 0, 3))           # rank % 8
    H, P, Y, need, total = _args(ah, r_r=2048); cases.append((H, P, Y, 0, 3))         # rank cap
    H, P, Y, need, total = _args(ah, V=0); cases.append((H, P, Y, 0, 2))
    H, P, Y, need, total = _args(ah); cases.append((H, P, Y, 7, 3))                    # bad path
    H, P, Y, need, total = _args(ah, N=65); cases.append((H, P, Y, 1, 3))             # decode path: <= 64
    H, P, Y, need, total = _args(ah, N=9, V=128256, D=8192, r_c=64, r_r=64, g=128)
    cases.append((H, P, Y, 1, 3))                                                       # ... whose H fits LDS
    H, P, Y, need, total = _args(ah); H.data = None; cases.append((H, P, Y, 0, 1))
    H, P, Y, need, total = _args(ah); P.workspace = None; cases.append((H, P, Y, 2, 1))  # the tile path needs one
    H, P, Y, need, total = _args(ah, N=20); P.workspace = None; cases.append((H, P, Y, 0, 1))
    H, P, Y, need, total = _args(ah); P.buffer = FAKE + 16; cases.append((H, P, Y, 0, 6))
    H, P, Y, need, total = _args(ah); P.workspace = FAKE + 128; cases.append((H, P, Y, 0, 6))
    H, P, Y, need, total = _args(ah); H.data = FAKE + 2; cases.append((H, P, Y, 0, 6))
    H, P, Y, need, total = _args(ah); H.row_stride = 260; cases.append((H, P, Y, 0, 6))  # 520-byte rows
    H, P, Y, need, total = _args(ah); Y.data = FAKE + 2; cases.append((H, P, Y, 0, 6))   # fp32 Y at 2 mod 4
    H, P, Y, need, total = _args(ah, buf=100); cases.append((H, P, Y, 0, 10))
    H, P, Y, need, total = _args(ah, ws=1); cases.append((H, P, Y, 2, 7))             # tile path: too small
    H, P, Y, need, total = _args(ah, N=20, ws=1); cases.append((H, P, Y, 0, 7))
    H, P, Y, need, total = _args(ah, N=4096, V=151936, D=4096, r_c=64, r_r=64, g=128, ydt=1, ws=12345)
    cases.append((H, P, Y, 2, 7))
    for i, (H, P, Y, path, want) in enumerate(cases):
        assert _call(ah, H, P, Y, path) == want, i


def test_stats_workspace_bytes(ah):
    # the logits workspace, then statistics pieces (N * max(64, ceil(V16/256)) * 16 B)
    # and, for calls the decode kernel takes, Y in fp32 (N * V * 4 B); each 256-aligned
    up = lambda x: (x + 255) // 256 * 256
    for (V, D, r_c, r_r, g), N in [((1024, 256, 16, 8, 64), 4), ((151936, 4096, 32, 32, 128), 1),
                                   ((151936, 4096, 64, 64, 128), 4096), ((64, 128, 0, 0, 32), 17)]:
        pieces = max(64, ((V + 15) // 16 * 16 + 255) // 256)
        want = (ah.archead_workspace_bytes(V, D, r_c, r_r, g, N) + up(N * pieces * 16) +
                up(N * V * 4 if N <= 16 or _batched(V, D, r_c, r_r, g, N) else 0))
        assert ah.archead_stats_workspace_bytes(V, D, r_c, r_r, g, N) == want
    assert ah.archead_stats_workspace_bytes(1024, 256, 16, 8, 64, 0) == 0


def test_stats_error_paths(ah):
    def call(H, P, st):
        return ah.lib.archead_logits_stats(ctypes.byref(H), ctypes.byref(P), st and ctypes.byref(st), None)

    def args(**kw):
        H, P, Y, need, total = _args(ah, **kw)
        P.workspace_bytes = ah.archead_stats_workspace_bytes(1024, 256, 16, 8, 64, H.rows) if H.rows >= 0 else 0
        return H, P, ah.ArcheadRowStats(FAKE + (4 << 30), FAKE + (5 << 30), FAKE + (6 << 30), None, None)

    H, P, st = args()
    assert call(H, P, None) == 1
    assert ah.lib.archead_logits_stats(None, ctypes.byref(P), ctypes.byref(st), None) == 1
    H, P, st = args(); st.row_ce = FAKE + (7 << 30); assert call(H, P, st) == 1         # ce without targets
    H, P, st = args(); st.row_lse = FAKE + 2; assert call(H, P, st) == 6                # misaligned output
    H, P, st = args(); st.row_ce = FAKE + (7 << 30); st.targets = FAKE + 1; assert call(H, P, st) == 6
    H, P, st = args(hdt=2); assert call(H, P, st) == 4
    H, P, st = args(); H.cols = 255; assert call(H, P, st) == 5
    H, P, st = args(g=16); assert call(H, P, st) == 3
    H, P, st = args(); P.workspace_bytes = ah.archead_workspace_bytes(1024, 256, 16, 8, 64, 4)
    assert call(H, P, st) == 7                                                          # logits-sized workspace
    H, P, st = args(N=0); H.data = None; P.workspace = None; assert call(H, P, st) == 0


def test_quantize_error_paths(ah):
    """archead_quantize rejects bad arguments on the host, before any HIP call."""
    V, D, r_c, r_r, g = 1000, 512, 16, 8, 64
    total = ah.archead_pack_layout(V, D, r_c, r_r, g)["total_bytes"]

    def call(dims=(V, D, r_c, r_r, g), W=FAKE, ws=D, wdt=1, A_c=FAKE + (1 << 30), B_c=FAKE + (2 << 30),
             A_w=FAKE + (3 << 30), B_w=FAKE + (4 << 30), buf=FAKE + (8 << 30), nbytes=total, E=None):
        src = ah.ArcheadDenseHead(W, ws, wdt, A_c, B_c, A_w, B_w)
        return ah.lib.archead_quantize(ctypes.byref(ah._dims(*dims)), ctypes.byref(src), buf, nbytes,
                                       ctypes.byref(E) if E is not None else None, None)

    def E(**kw):
        f = dict(data=FAKE + (16 << 30), rows=V, cols=D, row_stride=D, dtype=2)
        f.update(kw)
        return ah.ArcheadTensor(f["data"], f["rows"], f["cols"], f["row_stride"], f["dtype"])

    assert ah.lib.archead_quantize(None, None, None, 0, None, None) == 1
    assert call(W=None) == 1
    assert call(buf=None) == 1
    assert call(A_c=None) == 1
    assert call(B_w=None) == 1
    assert call(dims=(V, D, 0, 8, g), A_c=None, B_c=None, nbytes=0) == 10        # rank-0 part may be NULL
    assert call(dims=(V, 500, r_c, r_r, g)) == 2                                 # D not a multiple of 128
    assert call(dims=(V, D, r_c, r_r, 16)) == 3                                  # group size
    assert call(dims=(V, 8192 + 128, r_c, r_r, g)) == 3                          # D above the register limit
    assert call(dims=(V, D, 1032, r_r, g)) == 3                                  # core rank above the LDS limit
    assert call(wdt=3) == 4
    assert call(ws=D - 1) == 5
    assert call(W=FAKE + 8) == 6                                                  # W not 16-byte aligned
    assert call(ws=D + 4, wdt=1) == 6                                             # bf16 rows of 1032 bytes
    assert call(A_w=FAKE + 2) == 6
    assert call(buf=FAKE + 128) == 6
    assert call(nbytes=total - 1) == 10
    assert call(E=E(data=None)) == 1
    assert call(E=E(dtype=1)) == 4
    assert call(E=E(rows=V - 1)) == 5
    assert call(E=E(row_stride=D - 4)) == 5
    assert call(E=E(row_stride=D + 2)) == 6


def test_topk_workspace_bytes(ah):
    up = lambda x: (x + 255) // 256 * 256
    for (V, D, r_c, r_r, g) in [(1024, 256, 16, 8, 64), (151936, 4096, 64, 64, 128)]:
        for N in (1, 16, 17, 256, 257, 4096):
            rows = min(N, 256)
            spans = rows * -(-V // 4096) * 4   # spans of 1024 logits
            # fp32 logits of one chunk, then each span's largest key
            want = up(ah.archead_workspace_bytes(V, D, r_c, r_r, g, rows)) + up(rows * V * 4) + up(spans * 4)
            assert ah.archead_topk_workspace_bytes(V, D, r_c, r_r, g, N) == want
    assert ah.archead_topk_workspace_bytes(1024, 256, 16, 8, 64, 0) == 0


def test_topk_error_paths(ah):
    def call(H, P, k, val=FAKE + (4 << 30), idx=FAKE + (5 << 30)):
        return ah.lib.archead_logits_topk(ctypes.byref(H), ctypes.byref(P), k, val, idx, None)

    def args(**kw):
        H, P, Y, need, total = _args(ah, **kw)
        P.workspace_bytes = ah.archead_topk_workspace_bytes(1024, 256, 16, 8, 64, H.rows) if H.rows >= 0 else 0
        return H, P

    H, P = args()
    assert ah.lib.archead_logits_topk(None, ctypes.byref(P), 5, FAKE, FAKE, None) == 1
    assert call(H, P, 0) == 5
    assert call(H, P, 17) == 3
    assert call(H, P, 5, val=None) == 1
    assert call(H, P, 5, idx=FAKE + 2) == 6
    H, P = args(); P.workspace_bytes -= 1; assert call(H, P, 5) == 7
    H, P = args(); P.workspace_bytes = ah.archead_workspace_bytes(1024, 256, 16, 8, 64, 4); assert call(H, P, 5) == 7
    H, P = args(V=8); assert call(H, P, 9) == 5                                  # k above V
    H, P = args(N=0); H.data = None; P.workspace = None; assert call(H, P, 5, None, None) == 0


def test_fit_workspace_bytes(ah):
    up = lambda x: (x + 255) // 256 * 256
    for (V, D, r_c, r_r, g, o) in [(1000, 256, 16, 8, 64, 8), (151936, 4096, 32, 32, 128, 8), (500, 384, 0, 24, 128, 4)]:
        k = max(r_c, r_r) + o
        # W and E in fp32; V x k, D x k and k x D panels (two, three, two); 65 chunk products of D x k;
        # 256 fp64 Gram partials, the Gram matrix, eigenvalues and scratch; R^{-1}, U S, U S^{-1};
        # status ints; covariance, eigenvalues, eigensolver scratch, three more D x D; the factors
        parts = [V * D * 4, V * D * 4, V * k * 4, V * k * 4, D * k * 4, D * k * 4, D * k * 4, k * D * 4,
                 k * D * 4, 65 * D * k * 4, 256 * k * k * 8, k * k * 8, k * 8, k * 8, k * k * 4, k * k * 4,
                 k * k * 4, 64, D * D * 4, D * 4, D * 4, D * D * 4, D * D * 4, D * D * 4,
                 V * r_c * 4, r_c * D * 4, V * r_r * 4, r_r * D * 4, r_r * D * 4]
        assert ah.archead_fit_workspace_bytes(V, D, r_c, r_r, g, o) == sum(up(x) for x in parts)
    with pytest.raises(ah.ArcheadError):
        ah.archead_fit_workspace_bytes(20, 128, 16, 8, 64, 8)     # rank + oversample above V
    with pytest.raises(ah.ArcheadError):
        ah.archead_fit_workspace_bytes(4096, 1024, 128, 8, 64, 1)  # rank + oversample above 128
    assert ah.archead_fit_workspace_bytes(4096, 1024, 120, 8, 64, 8) > 0


def test_fit_error_paths(ah):
    """archead_fit rejects bad arguments on the host, before any HIP call."""
    V, D, r_c, r_r, g, o = 1000, 256, 16, 8, 64, 8
    total = ah.archead_pack_layout(V, D, r_c, r_r, g)["total_bytes"]
    ws = ah.archead_fit_workspace_bytes(V, D, r_c, r_r, g, o)

    def call(dims=(V, D, r_c, r_r, g), buf=FAKE + (8 << 30), nbytes=total, w=FAKE + (16 << 30), nws=ws, **kw):
        f = dict(W=FAKE, W_stride=D, W_dtype=1, H=FAKE + (1 << 30), H_rows=512, H_stride=D, omega_c=FAKE + (2 << 30),
                 omega_r=FAKE + (3 << 30), p=0.75, lam=0.01, oversample=o, power_iters=2)
        f.update(kw)
        inp = ah.ArcheadFitInputs(*(f[k] for k in ("W", "W_stride", "W_dtype", "H", "H_rows", "H_stride", "omega_c",
                                                   "omega_r", "p", "lam", "oversample", "power_iters")))
        return ah.lib.archead_fit(ctypes.byref(ah._dims(*dims)), ctypes.byref(inp), buf, nbytes, w, nws, None, None)

    assert ah.lib.archead_fit(None, None, None, 0, None, 0, None, None) == 1
    assert call(W=None) == 1 and call(H=None) == 1 and call(buf=None) == 1 and call(w=None) == 1
    assert call(omega_r=None) == 1
    assert call(dims=(V, D, r_c, 0, g), omega_r=None, nbytes=0) == 10           # rank-0 part may be NULL
    assert call(dims=(V, 200, r_c, r_r, g)) == 2
    assert call(dims=(V, D, r_c, r_r, 16)) == 3
    assert call(W_dtype=3) == 4
    assert call(W_stride=D - 1) == 5 and call(H_stride=D - 2) == 5 and call(H_rows=0) == 5
    assert call(oversample=-1) == 5 and call(power_iters=17) == 5
    assert call(dims=(20, D, r_c, r_r, g)) == 5                                   # rank + oversample above V
    assert call(dims=(V, D, r_c, 128, g)) == 3                                    # rank + oversample above 128
    assert call(lam=0.0) == 9 and call(p=float("nan")) == 9
    assert call(buf=FAKE + 128) == 6 and call(w=FAKE + 64) == 6 and call(H=FAKE + 1) == 6
    assert call(nbytes=total - 1) == 10
    assert call(nws=ws - 1) == 7


def test_logit_error_workspace_and_errors(ah):
    up = lambda x: (x + 255) // 256 * 256
    for N in (1, 255, 256, 1000):
        rows = min(N, 256)
        want = up(ah.archead_workspace_bytes(1024, 256, 16, 8, 64, rows)) + 2 * up(rows * 1024 * 4) + 16384 + 256
        assert ah.archead_logit_error_workspace_bytes(1024, 256, 16, 8, 64, N) == want
    assert ah.archead_logit_error_workspace_bytes(1024, 256, 16, 8, 64, 0) == 0
    sums = (ctypes.c_double * 2)()

    def call(H, P, W, out=sums):
        return ah.lib.archead_logit_error(ctypes.byref(H), ctypes.byref(P), ctypes.byref(W), out, None)

    def args():
        H, P, Y, need, total = _args(ah)
        P.workspace_bytes = ah.archead_logit_error_workspace_bytes(1024, 256, 16, 8, 64, 4)
        return H, P, ah.ArcheadTensor(FAKE + (9 << 30), 1024, 256, 256, 1)

    H, P, W = args(); assert call(H, P, W, None) == 1
    H, P, W = args(); W.dtype = 2; assert call(H, P, W) == 4
    H, P, W = args(); W.rows = 1000; assert call(H, P, W) == 5
    H, P, W = args(); W.row_stride = 255; assert call(H, P, W) == 5
    H, P, W = args(); W.data = FAKE + 1; assert call(H, P, W) == 6
    H, P, W = args(); P.workspace_bytes -= 1; assert call(H, P, W) == 7
    H, P, W = args(); H.rows = 0; H.data = None; P.workspace = None; sums[0] = 5.0
    assert call(H, P, W) == 0 and sums[0] == 0.0


def test_logits_offsets_past_32_bits_are_unsupported(ah):
    """A head whose residual section reaches 4 GiB (V = 2^21 rows of D = 4096)
    is refused on every path before any HIP call: the kernels address every
    section with 32-bit offsets."""
    for path in (0, 1, 2):
        H, P, Y, need, total = _args(ah, N=1, V=1 << 21, D=4096, r_c=0, r_r=0, g=128)
        P.workspace_bytes = ah.archead_workspace_bytes_path(1 << 21, 4096, 0, 0, 128, 1, 2)
        assert _call(ah, H, P, Y, path) == 3, path


def test_logits_zero_tokens_is_a_noop(ah):
    H, P, Y, need, total = _args(ah, N=0)
    H.data = Y.data = None
    P.workspace = None
    assert _call(ah, H, P, Y, 0) == 0
    assert _call(ah, H, P, Y, 1) == 0
    assert _call(ah, H, P, Y, 2) == 0


def test_status_strings(ah):
    for code in range(11):
        s = ah.archead_status_string(code)
        assert s.startswith("ARCHEAD_")
        assert ah.STATUS[code] in s
    assert "unknown" in ah.archead_status_string(99)


def test_header_is_plain_c(tmp_path):
    """include/archead.h compiles as strict C99 (the ABI is C, not C++)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use.c"
    src.write_text('#include "archead.h"\nint main(void) { archead_fit_inputs f; archead_layout l; '
                   '(void)f; (void)l; return ARCHEAD_FORMAT_VERSION == 1 ? 0 : 1; }\n')
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                          "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_every_kernel_has_its_host_launch_stub(ah):
    """A kernel whose host-side instantiation is dropped leaves an undefined
    launch stub behind, and the library then fails to load on a machine with a GPU."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", ah.LIB_PATH], capture_output=True, text=True, check=True).stdout
    stubs = [l for l in out.splitlines() if "device_stub" in l]
    assert not stubs, stubs

