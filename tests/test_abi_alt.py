"""C ABI of the storage-matched comparison heads (group INT4 with fp16 group
scales, row INT8; ARCHead paper, results discussion of Tables 7 and 8), no GPU:
section layout and packed bytes against the oracle's packer and the
hand-derived golden positions, which kernel a call takes, and the entry points
that serve the ARCHead format only."""
import ctypes
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests.test_abi import FAKE, ah  # noqa: F401  (module fixture)

FMT_G4, FMT_R8 = 1, 2
SECTIONS = ["header", "r_codes", "r_gcodes", "r_rowscale", "a_codes", "a_scales", "b_codes", "b_scales"]


@pytest.mark.parametrize("fmt", [FMT_G4, FMT_R8])
@pytest.mark.parametrize("V,D,g", [(20, 256, 64), (128256, 4096, 128), (151936, 8192, 32), (1, 128, 2),
                                   (1000, 512, 256)])
def test_alt_layout_matches_oracle(ah, fmt, V, D, g):
    a = ah.archead_pack_layout(V, D, 0, 0, g, fmt)
    b = oracle.layout(V, D, 0, 0, g, fmt)
    for n in SECTIONS:
        assert tuple(a[n]) == tuple(b[n]), n
    assert a["total_bytes"] == b["total_bytes"] and a["payload_bytes"] == b["payload_bytes"]
    V16 = (V + 15) // 16 * 16
    assert a["payload_bytes"] == oracle.alt_persistent_bytes(V16, D, g, fmt)


@pytest.mark.parametrize("fmt,V,D,g", [(FMT_G4, 37, 256, 64), (FMT_G4, 16, 128, 128), (FMT_G4, 50, 512, 32),
                                       (FMT_G4, 3, 512, 256), (FMT_R8, 37, 256, 64), (FMT_R8, 129, 384, 128),
                                       (FMT_R8, 16, 128, 32)])
def test_alt_library_packer_matches_oracle_packer(ah, fmt, V, D, g):
    h = synth.draw_alt_head(np.random.default_rng(V * 11 + D + fmt), fmt, V, D, g)
    assert np.array_equal(ah.archead_pack(h), oracle.pack_alt(h))


def test_alt_library_packer_golden_positions(ah, golden_dir):
    G = json.load(open(os.path.join(golden_dir, "format_alt_cases.json")))
    for key, fmt in (("f1", FMT_G4), ("f2", FMT_R8)):
        c = G[key]
        d = c["dims"]
        L = ah.archead_pack_layout(d["V"], d["D"], 0, 0, d["g"], fmt)
        for name, (off, size) in c["sections"].items():
            assert tuple(L[name]) == (off, size), (key, name)
        assert L["total_bytes"] == c["total_bytes"] and L["payload_bytes"] == c["payload_bytes"]
        ng = d["D"] // d["g"]
        codes = np.zeros((d["V"], d["D"]), np.int8)
        scales = np.zeros((d["V"], ng) if fmt == FMT_G4 else d["V"], np.float16)
        for e in c.get("nibbles", []) + c.get("codes", []):
            codes[e["v"], e["k"]] = e["code"]
        for e in c.get("group_scales", []):
            scales[e["v"], e["t"]] = np.uint16(e["f16_bits"]).view(np.float16)
        for e in c.get("row_scale", []):
            scales[e["v"]] = np.uint16(e["f16_bits"]).view(np.float16)
        buf = ah.archead_pack(synth.AltHead(fmt, d["V"], d["D"], d["g"], codes, scales))
        assert int(buf[36:40].view(np.uint32)[0]) == fmt  # the header's flags word holds the format
        for e in c.get("nibbles", []):
            byte = int(buf[e["byte"]])
            assert (byte & 0xF if e["half"] == "lo" else byte >> 4) == e["code"] & 0xF, e
        for e in c.get("codes", []):
            assert int(buf[e["byte"]]) == e["code"] & 0xFF, e
        for e in c.get("group_scales", []) + c.get("row_scale", []):
            assert int(buf[e["byte"]:e["byte"] + 2].view(np.uint16)[0]) == e["f16_bits"], e
        # every other payload byte is zero
        nz = np.flatnonzero(buf[256:])
        want = sorted({e["byte"] - 256 for e in c.get("nibbles", []) + c.get("codes", [])} |
                      {e["byte"] - 256 + i for e in c.get("group_scales", []) + c.get("row_scale", [])
                       for i in (0, 1) if (e["f16_bits"] >> (8 * i)) & 0xFF})
        assert list(nz) == want, key


def _alt_components(ah, fmt, V=32, D=128, g=32, seed=3):
    h = synth.draw_alt_head(np.random.default_rng(seed), fmt, V, D, g)
    comp = ah.ArcheadHostComponents()
    codes, scales = np.ascontiguousarray(h.codes), np.ascontiguousarray(h.scales)
    if fmt == FMT_G4:
        comp.q4, comp.s_G = codes.ctypes.data, scales.ctypes.data
    else:
        comp.q8, comp.s_R = codes.ctypes.data, scales.ctypes.data
    total = ah.archead_pack_layout(V, D, 0, 0, g, fmt)["total_bytes"]
    return h, comp, (codes, scales), total


def test_alt_pack_errors(ah):
    for fmt in (FMT_G4, FMT_R8):
        h, comp, keep, total = _alt_components(ah, fmt)
        d = ah.ArcheadDims(32, 128, 0, 0, 32, fmt)
        out = np.zeros(total, np.uint8)
        assert ah.lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), out.ctypes.data, total) == 0
        assert np.array_equal(out, oracle.pack_alt(h))
        assert ah.lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), out.ctypes.data, total - 1) == 10
        codes = keep[0]
        codes[7, 9] = 8 if fmt == FMT_G4 else -128                  # outside the format's range
        out2 = np.zeros(total, np.uint8)
        assert ah.lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), out2.ctypes.data, total) == 9
        assert not out2.any()                                        # nothing written on failure
        if fmt == FMT_G4:
            codes[7, 9] = -9
            assert ah.lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), out2.ctypes.data, total) == 9
            comp.s_G = None
        else:
            comp.s_R = None
        assert ah.lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), out.ctypes.data, total) == 1
    L = ah.ArcheadLayout()
    for dims, want in [((32, 128, 0, 0, 32, 3), 2), ((32, 128, 0, 0, 32, -1), 2), ((32, 128, 8, 0, 32, 1), 2),
                       ((32, 128, 0, 8, 32, 2), 2), ((32, 128, 0, 0, 32, 2), 0)]:
        assert ah.lib.archead_pack_layout(ctypes.byref(ah.ArcheadDims(*dims)), ctypes.byref(L)) == want, dims


@pytest.mark.parametrize("fmt", [FMT_G4, FMT_R8])
def test_alt_main_kernel_and_workspace(ah, fmt):
    V, D, g = 128256, 4096, 128
    up = lambda x: (x + 255) // 256 * 256
    for N in (0, 1, 5, 16, 17, 32, 33, 64, 4096):
        assert ah.archead_main_kernel(V, D, 0, 0, g, N, 0, fmt=fmt) == "batch_kernel"
        assert ah.archead_main_kernel(V, D, 0, 0, g, N, 1, fmt=fmt) == "batch_kernel"
        # one launch's rows (at most 32) of converted H and their scales
        c = min(N, 32)
        want = up(c * D * 2) + up(c * 4) if N else 0
        assert ah.archead_workspace_bytes(V, D, 0, 0, g, N, fmt=fmt) == want
        assert ah.archead_workspace_bytes_path(V, D, 0, 0, g, N, 1, fmt=fmt) == want
    for args in [(V, D, 0, 0, g, 4, 2), (V, 384, 0, 0, g, 4, 0), (V, 640, 0, 0, 128, 40, 0)]:
        with pytest.raises(ah.ArcheadError) as e:                    # tile path; D not a multiple of 512
            ah.archead_main_kernel(*args, fmt=fmt)
        assert e.value.status == 3
    with pytest.raises(ah.ArcheadError) as e:
        ah.archead_workspace_bytes_path(V, D, 0, 0, g, 4, 2, fmt=fmt)
    assert e.value.status == 3
    # D/g > 64 groups per row: the group INT4 head keeps its scales in LDS; the row INT8 head has none
    if fmt == FMT_G4:
        with pytest.raises(ah.ArcheadError):
            ah.archead_main_kernel(V, 8192, 0, 0, 32, 4, fmt=fmt)
    else:
        assert ah.archead_main_kernel(V, 8192, 0, 0, 32, 4, fmt=fmt) == "batch_kernel"


@pytest.mark.parametrize("fmt", [FMT_G4, FMT_R8])
def test_alt_archead_only_entry_points(ah, fmt):
    V, D, g, N = 1024, 512, 64, 4
    d = ah.ArcheadDims(V, D, 0, 0, g, fmt)
    b = ctypes.c_uint64()
    assert ah.lib.archead_stats_workspace_bytes(ctypes.byref(d), N, ctypes.byref(b)) == 3
    assert ah.lib.archead_fit_workspace_bytes(ctypes.byref(d), 8, ctypes.byref(b)) == 3
    H = ah.ArcheadTensor(FAKE, N, D, D, 1)
    Y = ah.ArcheadTensor(FAKE + (1 << 30), N, V, V, 2)
    P = ah.ArcheadPackedHead(d, FAKE + (2 << 30), 1 << 20, FAKE + (3 << 30), 1 << 20)
    st = ah.ArcheadRowStats(FAKE + (4 << 30), FAKE + (5 << 30), FAKE + (6 << 30), None, None)
    assert ah.lib.archead_logits_stats(ctypes.byref(H), ctypes.byref(P), ctypes.byref(st), None) == 3
    assert ah.lib.archead_logits_noalloc(ctypes.byref(H), ctypes.byref(P), ctypes.byref(Y), None) == 3
    dense = ah.ArcheadDenseHead(FAKE, D, 1, None, None, None, None)
    assert ah.lib.archead_quantize(ctypes.byref(d), ctypes.byref(dense), FAKE, 1 << 30, None, None) == 3
    # the tile path is not served for a comparison head
    assert ah.lib.archead_logits_path(ctypes.byref(H), ctypes.byref(P), ctypes.byref(Y), 2, None) == 3
    # the entry points built on archead_logits size their workspace for a comparison head too
    assert ah.archead_topk_workspace_bytes(V, D, 0, 0, g, N, fmt=fmt) > 0
    assert ah.archead_logit_error_workspace_bytes(V, D, 0, 0, g, N, fmt=fmt) > 0
