"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: the hand-derived golden files,
exact integer arithmetic, a textbook reduction (group-INT4 dequantisation), a
brute-force loop, or an algebraic invariant.  A wrong sign, index, dropped term
or transposed operand anywhere in the oracle fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

# ----------------------------------------------------------------- helpers ---


def _f16_exact(bits: int) -> Fraction:
    """IEEE binary16 decoded from its bits with integer arithmetic only."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    assert e != 31
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    return sign * Fraction(1024 + m, 1 << 10) * (Fraction(2) ** (e - 15))


def _bf16_exact(bits: int) -> Fraction:
    """bfloat16 (8 exponent bits, 7 fraction bits) decoded with integers only."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 255
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(2) ** (-126)
    return sign * Fraction(128 + m, 1 << 7) * Fraction(2) ** (e - 127)


def _head_close(a, b):
    """Bitwise equality of every stored component (a rank-0 part stores no scale)."""
    keys = ["q4", "c8", "s_R", "A_c", "A_w", "B_c", "B_w", "s_Bc", "s_Bw"]
    keys += ["s_Ac"] if a.r_c else []
    keys += ["s_Aw"] if a.r_r else []
    for k in keys:
        x = np.ascontiguousarray(getattr(a, k) if not isinstance(a, dict) else a[k])
        y = np.ascontiguousarray(b[k] if isinstance(b, dict) else getattr(b, k))
        assert x.shape == y.shape, k
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), k


# ------------------------------------------------------------ number decode ---

def test_f16_decode_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 10) & 0x1F) != 31
    bits = bits[finite].astype(np.uint16)
    got = oracle.f16_to_f64(bits.view(np.float16))
    want = np.array([float(_f16_exact(int(b))) for b in bits])
    assert np.array_equal(got, want)


def test_bf16_decode_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 255
    bits = bits[finite].astype(np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    want = np.array([float(_bf16_exact(int(b))) for b in bits])
    assert np.array_equal(got, want)


# -------------------------------------------------------------- the format ---

def test_nibble_code_table():
    """Signed INT4 in two's complement: the 16 nibble patterns and their values."""
    table = [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]
    h = synth.zero_head(16, 128, 0, 0, 32)
    # put every nibble value at every low/high position of row 0 and row 9
    for k in range(128):
        h.q4[0, k] = table[k % 16]
        h.q4[9, k] = table[(k * 7 + 3) % 16]
    buf = oracle.pack(h)
    u = oracle.unpack(buf, **h.dims)
    assert np.array_equal(u["q4"], h.q4)
    off = oracle.layout(**h.dims)["r_codes"][0]
    # row 0, k = 0,1 -> tile 0 byte 0: low nibble code 0 (0x0), high nibble code 1 (0x1)
    assert buf[off] == 0x10
    # row 0, k = 14, 15 -> codes -2, -1 -> nibbles 0xE, 0xF; kk=14: s=0 q=1 c=3 -> l=16 -> byte 16*16+3
    assert buf[off + 16 * 16 + 3] == 0xFE


def test_golden_format_positions(golden_dir):
    G = json.load(open(os.path.join(golden_dir, "format_v1_cases.json")))
    d = G["dims"]
    L = oracle.layout(**d)
    for name, (off, size) in G["sections"].items():
        assert tuple(L[name]) == (off, size), name
    assert L["total_bytes"] == G["total_bytes"]
    assert L["payload_bytes"] == G["payload_bytes"]

    h = synth.zero_head(d["V"], d["D"], d["r_c"], d["r_r"], d["g"])
    h.c8[:] = 0
    h.s_R[:] = 0
    h.s_Ac[:] = 0
    h.s_Aw[:] = 0
    h.s_Bc[:] = 0
    h.s_Bw[:] = 0
    for c in G["nibbles"]:
        h.q4[c["v"], c["k"]] = c["code"]
    for c in G["group_codes"]:
        h.c8[c["v"], c["t"]] = c["code"]
    for c in G["row_scale"]:
        h.s_R.view(np.uint16)[c["v"]] = c["f16_bits"]
    for c in G["a_codes"]:
        (h.A_c if c["part"] == "c" else h.A_w)[c["v"], c["j"]] = c["code"]
    for c in G["a_scales"]:
        (h.s_Ac if c["part"] == "c" else h.s_Aw).view(np.uint16)[c["v"]] = c["f16_bits"]
    for c in G["b_codes"]:
        (h.B_c if c["part"] == "c" else h.B_w)[c["j"], c["k"]] = c["code"]
    for c in G["b_scales"]:
        (h.s_Bc if c["part"] == "c" else h.s_Bw).view(np.uint16)[c["j"], c["t"]] = c["f16_bits"]
    buf = oracle.pack(h)
    assert buf.size == G["total_bytes"]

    expect = {}
    for c in G["nibbles"]:
        nib = c["code"] & 0xF
        expect[c["byte"]] = expect.get(c["byte"], 0) | (nib if c["half"] == "lo" else nib << 4)
    for c in G["group_codes"]:
        expect[c["byte"]] = c["code"]
    for c in G["row_scale"] + G["a_scales"] + G["b_scales"]:
        expect[c["byte"]] = c["f16_bits"] & 0xFF
        expect[c["byte"] + 1] = c["f16_bits"] >> 8
    for c in G["a_codes"] + G["b_codes"]:
        expect[c["byte"]] = c["code"] & 0xFF
    # header
    hdr = np.frombuffer(np.array([0x48435241, 1], np.uint32).tobytes() +
                        np.array([d["V"], d["D"]], np.uint64).tobytes() +
                        np.array([d["r_c"], d["r_r"], d["g"], 0], np.uint32).tobytes(), np.uint8)
    for i, b in enumerate(hdr):
        expect[i] = int(b)
    nz = {int(i): int(buf[i]) for i in np.flatnonzero(buf)}
    want = {k: v for k, v in expect.items() if v}
    assert nz == want
    for c in G["row_scale"] + G["a_scales"] + G["b_scales"]:
        assert float(_f16_exact(c["f16_bits"])) == c["value"]


def _tile_pack_loop(q4_padded):
    """Element-by-element reading of the residual tile order (tiny shapes only)."""
    V16, D = q4_padded.shape
    out = np.zeros(V16 * D // 2, np.uint8)
    nb = V16 // 16
    for v in range(V16):
        for k in range(0, D, 2):
            b, i = divmod(v, 16)
            kt, kk = divmod(k, 128)
            s, rem = divmod(kk, 32)
            q, rem8 = divmod(rem, 8)
            c = rem8 // 2
            lane = 16 * q + i
            pos = (kt * nb + b) * 1024 + 16 * lane + 4 * s + c
            lo = int(q4_padded[v, k]) & 0xF
            hi = int(q4_padded[v, k + 1]) & 0xF
            out[pos] = lo | (hi << 4)
    return out


@pytest.mark.parametrize("V,D", [(16, 128), (33, 256), (5, 384)])
def test_tile_order_matches_loop(V, D):
    rng = np.random.default_rng(V * D)
    h = synth.draw_head(rng, V, D, 8, 0, 32)
    buf = oracle.pack(h)
    L = oracle.layout(**h.dims)
    off, size = L["r_codes"]
    q = np.zeros((L["V16"], D), np.int8)
    q[:V] = h.q4
    assert np.array_equal(buf[off:off + size], _tile_pack_loop(q))


@pytest.mark.parametrize("V,D,r_c,r_r,g", [
    (1024, 256, 16, 8, 64), (37, 128, 0, 0, 128), (50, 512, 0, 24, 32),
    (16, 256, 40, 0, 256), (129, 384, 8, 8, 64), (1, 128, 6, 6, 128)])
def test_pack_unpack_roundtrip(V, D, r_c, r_r, g):
    rng = np.random.default_rng(V + D + r_c)
    h = synth.draw_head(rng, V, D, r_c, r_r, g)
    buf = oracle.pack(h)
    u = oracle.unpack(buf, V, D, r_c, r_r, g)
    assert (u["magic"], u["version"]) == (oracle.MAGIC, oracle.FORMAT_VERSION)
    assert (u["V"], u["D"], u["r_c"], u["r_r"], u["g"]) == (V, D, r_c, r_r, g)
    assert u["pad_rows_zero"]
    _head_close(h, u)


def test_layout_sections_aligned_disjoint_and_no_dense_matrix():
    for c in synth.CONFIGS:
        d = dict(V=c["V"], D=c["D"], r_c=c["r_c"], r_r=c["r_r"], g=c["g"])
        L = oracle.layout(**d)
        spans = sorted(L[n] for n in ["header", "r_codes", "r_gcodes", "r_rowscale",
                                      "a_codes", "a_scales", "b_codes", "b_scales"])
        end = 0
        for off, size in spans:
            assert off % 256 == 0 and off >= end
            end = off + size
        assert L["total_bytes"] >= end and L["total_bytes"] % 256 == 0
        # a dense V x D matrix at 8 bits or more would need V*D bytes; no section is that big
        biggest = max(size for _, size in spans)
        assert biggest == L["r_codes"][1] == c["V"] * c["D"] // 2 < c["V"] * c["D"]


def test_persistent_size_equals_sum_of_stored_tensors():
    """Sec. 3 persistent-size equation: the payload is the sum over the stored
    tensors of numel x element size.  Values for the five workloads were worked
    out from that closed form independently."""
    expect = {"tiny": 172224, "decode": 326928640, "batched": 326928640,
              "prefill": 336918784, "head70b": 551796224}
    for c in synth.CONFIGS:
        d = dict(V=c["V"], D=c["D"], r_c=c["r_c"], r_r=c["r_r"], g=c["g"])
        assert oracle.layout(**d)["payload_bytes"] == oracle.persistent_bytes(**d) == expect[c["name"]]
    # no factors: a plain group-INT4 head with a uint8 group code and an fp16 row scale
    assert oracle.persistent_bytes(1024, 4096, 0, 0, 128) == 1024 * 2048 + 1024 * 32 + 2048


def test_storage_ratio_matches_pages():
    """The pages quote 25.61% of the BF16 head for the packed Qwen3-8B head
    (discussion of Table 7, comparison with GPTQ) and a rank-6 correction
    (Table 9 ablation);
    read with r_c = r_r = 6 and g = 128 the format gives the same 25.61%, i.e. a
    3.90x reduction (the abstract's 3.7-3.9x range)."""
    V, D = 151936, 4096
    ratio = oracle.persistent_bytes(V, D, 6, 6, 128) / (2 * V * D)
    assert round(100 * ratio, 2) == 25.61
    assert 3.7 <= 1 / ratio <= 3.91
    # the GPTQ-style INT4 head quoted beside it: 4 bits + one fp16 per 128 weights
    assert round(100 * (4 + 16 / 128) / 16, 2) == 25.78


# ------------------------------------------------------------ dequantisation ---

def test_golden_dequant_cases(golden_dir):
    G = json.load(open(os.path.join(golden_dir, "dequant_cases.json")))
    for c in G["cases"]:
        q4 = np.array([[c["q4"]] * 2], np.int8)
        c8 = np.array([[c["c8"]]], np.uint8)
        sR = np.array([c["s_R_bits"]], np.uint16).view(np.float16)
        R = oracle.dequant_R(q4, c8, sR, 2)
        assert R[0, 0] == c["expect"] and R[0, 1] == c["expect"], c


def test_dequant_group_boundaries():
    """Column k uses group k // g: move one group code and only that group changes."""
    V, D, g = 3, 256, 64
    q4 = np.ones((V, D), np.int8)
    c8 = np.array([[1, 2, 3, 4]] * V, np.uint8)
    sR = np.array([1.0, 0.5, 2.0], np.float16)
    R = oracle.dequant_R(q4, c8, sR, g)
    for k in range(D):
        assert np.array_equal(R[:, k], (k // g + 1) * np.array([1.0, 0.5, 2.0]))
    B = oracle.dequant_groups(np.full((2, D), -2, np.int8),
                              np.array([[1, 2, 4, 8], [0.25, 0.5, 1, 2]], np.float16), g)
    assert B[0, 63] == -2 and B[0, 64] == -4 and B[1, 255] == -4 and B[1, 0] == -0.5
    A = oracle.dequant_rows(np.array([[1, -127], [127, 0]], np.int8), np.array([0.5, 4.0], np.float16))
    assert A.tolist() == [[0.5, -63.5], [508.0, 0.0]]


# ------------------------------------------------------------- the forward ---

def _exact_logits(H_bits, h):
    """Y computed exactly with Python integers.  Every stored value is an
    integer times a power of two: bf16 H values are multiples of 2^-133 and fp16
    scales are multiples of 2^-24, so scaling by those powers gives integers."""
    N, D = H_bits.shape
    SH = 133
    Hi = np.array([[int(_bf16_exact(int(b)) * (1 << SH)) for b in row] for row in H_bits], dtype=object)
    f16i = lambda a: np.array([int(_f16_exact(int(b)) * (1 << 24)) for b in np.asarray(a).view(np.uint16).reshape(-1)],
                              dtype=object).reshape(np.asarray(a).shape)
    g = h.g
    # residual: integer weight q4 * c8 * (s_R * 2^24), column by column of the D axis
    sR = f16i(h.s_R)
    Wq = np.empty((h.V, D), dtype=object)
    for v in range(h.V):
        for k in range(D):
            Wq[v, k] = int(h.q4[v, k]) * int(h.c8[v, k // g]) * sR[v]
    Yint = (Hi.dot(Wq.T)) * (1 << 48)                       # units 2^-(SH+24) -> 2^-(SH+72)
    for A, sA, B, sB in ((h.A_c, h.s_Ac, h.B_c, h.s_Bc), (h.A_w, h.s_Aw, h.B_w, h.s_Bw)):
        r = A.shape[1]
        if r == 0:
            continue
        sAi, sBi = f16i(sA), f16i(sB)
        Bq = np.empty((r, D), dtype=object)
        for j in range(r):
            for k in range(D):
                Bq[j, k] = int(B[j, k]) * sBi[j, k // g]
        Aq = np.empty((h.V, r), dtype=object)
        for v in range(h.V):
            for j in range(r):
                Aq[v, j] = int(A[v, j]) * sAi[v]
        # Hi*Bq is in units of 2^-(SH+24), times Aq 2^-(SH+48); bring to 2^-(SH+72)
        Yint = Yint + (Hi.dot(Bq.T)).dot(Aq.T) * (1 << 24)
    return Yint, SH + 72


def test_exact_rational_tiny_workload():
    """The fp64 oracle against exact integer evaluation on the tiny workload."""
    inp = synth.make("tiny")
    h = inp.head
    SH = 133
    Yint, _ = _exact_logits_scaled(inp.H_bits, h, SH)
    Y = oracle.logits(inp.H_bits, h)
    exact = np.array([[float(Fraction(int(x), 1 << (SH + 72))) for x in row] for row in Yint])
    scale = np.abs(exact).max()
    assert scale > 0
    assert np.abs(Y - exact).max() <= 1e-12 * scale


def _exact_logits_scaled(H_bits, h, SH):
    """Integer Y in units of 2^-(SH+72): residual term (units 2^-(SH+24)) times
    2^48 plus each low-rank term (units 2^-(SH+48)) times 2^24."""
    N, D = H_bits.shape
    Hi = np.array([[int(_bf16_exact(int(b)) * (1 << SH)) for b in row] for row in H_bits], dtype=object)

    def f16i(a):
        a = np.asarray(a)
        flat = [int(_f16_exact(int(b)) * (1 << 24)) for b in a.view(np.uint16).reshape(-1)]
        return np.array(flat, dtype=object).reshape(a.shape)

    g = h.g
    sR = f16i(h.s_R)
    c8 = h.c8.astype(object)
    Wq = h.q4.astype(object) * np.repeat(c8, g, axis=1) * sR[:, None]
    Y = Hi.dot(Wq.T) * (1 << 48)
    for A, sA, B, sB in ((h.A_c, h.s_Ac, h.B_c, h.s_Bc), (h.A_w, h.s_Aw, h.B_w, h.s_Bw)):
        if A.shape[1] == 0:
            continue
        Bq = B.astype(object) * np.repeat(f16i(sB), g, axis=1)
        Aq = A.astype(object) * f16i(sA)[:, None]
        Y = Y + Hi.dot(Bq.T).dot(Aq.T) * (1 << 24)
    return Y, SH + 72


def test_exact_rational_loop_form_small():
    """Same exactness pin, written as scalar loops, on a shape small enough for them."""
    inp = synth.make("tiny", V=40, D=128, N=3, r_c=8, r_r=16, g=32, n_outlier=2)
    h = inp.head
    Yint, _ = _exact_logits(inp.H_bits, h)
    exact = np.array([[float(Fraction(int(x), 1 << (133 + 72))) for x in row] for row in Yint])
    Y = oracle.logits(inp.H_bits, h)
    assert np.abs(Y - exact).max() <= 1e-12 * np.abs(exact).max()


def test_no_factors_reduces_to_group_int4():
    """r_c = r_r = 0: the forward is the textbook group-INT4 matvec,
    Y[n,v] = s_R[v] * sum_t c8[v,t] * sum_{k in group t} q4[v,k] h[n,k],
    computed here in the integer-group-sum association order."""
    inp = synth.make("tiny", r_c=0, r_r=0, V=300, N=5)
    h = inp.head
    Y = oracle.logits(inp.H_bits, h)
    H = oracle.bf16_bits_to_f64(inp.H_bits)
    g, ng = h.g, h.D // h.g
    part = np.einsum("vtk,ntk->nvt", h.q4.reshape(h.V, ng, g).astype(np.float64),
                     H.reshape(H.shape[0], ng, g))
    Y2 = np.einsum("nvt,vt->nv", part, h.c8.astype(np.float64)) * h.s_R.astype(np.float64)[None, :]
    assert np.allclose(Y, Y2, rtol=0, atol=1e-12 * np.abs(Y).max())


def test_low_rank_term_brute_force():
    """q4 = 0: Y = H (A_c_hat B_c_hat + A_w_hat B_w_hat)^T, checked with a
    triple loop and with the (H B_hat^T) A_hat^T order of the inference step."""
    inp = synth.make("tiny", V=24, D=128, N=3, r_c=8, r_r=8, g=32, n_outlier=1)
    h = inp.head
    h.q4[:] = 0
    Y = oracle.logits(inp.H_bits, h)
    H = oracle.bf16_bits_to_f64(inp.H_bits)
    sBc = h.s_Bc.astype(np.float64)
    sBw = h.s_Bw.astype(np.float64)
    brute = np.zeros_like(Y)
    for n in range(3):
        for v in range(h.V):
            acc = 0.0
            for k in range(h.D):
                w = 0.0
                for j in range(h.r_c):
                    w += float(h.A_c[v, j]) * float(h.s_Ac[v]) * float(h.B_c[j, k]) * sBc[j, k // h.g]
                for j in range(h.r_r):
                    w += float(h.A_w[v, j]) * float(h.s_Aw[v]) * float(h.B_w[j, k]) * sBw[j, k // h.g]
                acc += H[n, k] * w
            brute[n, v] = acc
    assert np.allclose(Y, brute, rtol=0, atol=1e-12 * np.abs(Y).max())
    Bc = h.B_c * np.repeat(sBc, h.g, axis=1)
    Bw = h.B_w * np.repeat(sBw, h.g, axis=1)
    Zc, Zw = H @ Bc.T, H @ Bw.T
    Y3 = (Zc @ (h.A_c * h.s_Ac.astype(np.float64)[:, None]).T +
          Zw @ (h.A_w * h.s_Aw.astype(np.float64)[:, None]).T)
    assert np.allclose(Y, Y3, rtol=0, atol=1e-12 * np.abs(Y).max())


def test_one_hot_rows_give_the_dequantised_weights():
    inp = synth.make("tiny", V=64, D=256, r_c=0, r_r=0)
    h = inp.head
    eye = synth.f32_to_bf16_bits(np.eye(h.D, dtype=np.float32))
    Y = oracle.logits(eye, h)
    R = oracle.dequant_R(h.q4, h.c8, h.s_R, h.g)
    assert np.array_equal(Y, R.T)


def test_invariants():
    inp = synth.make("tiny")
    h = inp.head
    Y = oracle.logits(inp.H_bits, h)
    # scaling H by 2 (an exponent bump in bf16) scales Y by 2 exactly
    H2 = (inp.H_bits.astype(np.uint32) + (1 << 7)).astype(np.uint16)
    assert np.array_equal(oracle.logits(H2, h), 2 * Y)
    # permuting vocabulary rows permutes the columns of Y
    perm = np.random.default_rng(0).permutation(h.V)
    hp = synth.Head(h.V, h.D, h.r_c, h.r_r, h.g, h.q4[perm], h.c8[perm], h.s_R[perm],
                    h.A_c[perm], h.A_w[perm], h.s_Ac[perm], h.s_Aw[perm],
                    h.B_c, h.B_w, h.s_Bc, h.s_Bw)
    assert np.array_equal(oracle.logits(inp.H_bits, hp), Y[:, perm])
    # all-zero codes give Y = 0
    z = synth.zero_head(h.V, h.D, h.r_c, h.r_r, h.g)
    assert not np.any(oracle.logits(inp.H_bits, z))
    # linearity in H over exactly representable sums (disjoint supports)
    Ha = inp.H_bits.copy()
    Hb = inp.H_bits.copy()
    Ha[:, 1::2] = 0
    Hb[:, 0::2] = 0
    assert np.allclose(oracle.logits(Ha, h) + oracle.logits(Hb, h), Y, rtol=0, atol=1e-12 * np.abs(Y).max())
    # doubling one row scale doubles that column's residual part exactly
    hz = synth.make("tiny", r_c=0, r_r=0).head
    Yz = oracle.logits(inp.H_bits, hz)
    hz.s_R[7] = hz.s_R[7] * np.float16(2)
    Y7 = oracle.logits(inp.H_bits, hz)
    assert np.array_equal(Y7[:, 7], 2 * Yz[:, 7])
    assert np.array_equal(np.delete(Y7, 7, 1), np.delete(Yz, 7, 1))


def test_row_selection_and_chunking_agree():
    inp = synth.make("tiny")
    h = inp.head
    Y = oracle.logits(inp.H_bits, h)
    # BLAS may block differently per chunk: agreement to fp64 rounding
    assert np.allclose(oracle.logits(inp.H_bits, h, v_chunk=100), Y, rtol=0, atol=1e-12 * np.abs(Y).max())
    cols = np.array([5, 900, 3, 1023])
    assert np.allclose(oracle.logits(inp.H_bits, h, rows=[2, 0], cols=cols), Y[[2, 0]][:, cols],
                       rtol=0, atol=1e-12 * np.abs(Y).max())


def test_argmax_ties_and_gap():
    Y = np.array([[1.0, 3.0, 3.0, -1.0], [0.0, 0.0, 0.0, 0.0], [-5.0, -4.0, -4.5, -9.0]])
    assert oracle.row_argmax(Y).tolist() == [1, 0, 1]
    assert oracle.top2_gap(Y).tolist() == [0.0, 0.0, 0.5]


# ------------------------------------------------------------ row statistics ---


def test_row_stats_closed_forms():
    """Constant rows: every logit ties, so argmax is 0, lse = c + log V and the
    cross-entropy of any target is log V; a row with one dominant logit has
    lse equal to it up to exp(-gap)."""
    V = 37
    Y = np.full((3, V), 2.5)
    Y[1] = -1e4
    Y[2, :] = 0.0
    Y[2, 11] = 800.0
    st = oracle.row_stats(Y, targets=[5, 0, 11])
    assert st["argmax"].tolist() == [0, 0, 11]
    assert st["max"].tolist() == [2.5, -1e4, 800.0]
    assert abs(st["lse"][0] - (2.5 + np.log(V))) < 1e-14
    assert abs(st["lse"][1] - (-1e4 + np.log(V))) < 1e-11
    assert st["lse"][2] == 800.0  # exp(-800) * 36 is far below one ulp of 800
    assert abs(st["ce"][0] - np.log(V)) < 1e-14 and abs(st["ce"][1] - np.log(V)) < 1e-11
    assert st["ce"][2] == 0.0


def test_row_stats_brute_force_and_library():
    """Small rows against a pure-Python loop (math.fsum of math.exp), and
    larger ones against scipy's log-sum-exp and softmax, which are written
    independently of the oracle."""
    import math
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(7)
    Y = rng.normal(0.0, 3.0, size=(5, 50))
    t = rng.integers(0, 50, size=5)
    st = oracle.row_stats(Y, targets=t)
    for n in range(5):
        row = [float(x) for x in Y[n]]
        lse = math.log(math.fsum(math.exp(x) for x in row))
        assert abs(st["lse"][n] - lse) < 1e-12
        assert st["argmax"][n] == max(range(50), key=lambda v: (row[v], -v))
        assert abs(st["ce"][n] - (lse - row[t[n]])) < 1e-12
    Z = rng.normal(0.0, 400.0, size=(4, 20000))  # logits of the size the synthetic heads give
    tz = rng.integers(0, 20000, size=4)
    sz = oracle.row_stats(Z, targets=tz)
    assert np.allclose(sz["lse"], logsumexp(Z, axis=1), rtol=1e-15, atol=1e-12)
    p = softmax(Z, axis=1)[np.arange(4), tz]
    assert np.allclose(np.exp(-sz["ce"]), p, rtol=1e-12, atol=0)


def test_row_stats_invariants():
    """Shift: lse(Y + c) = lse(Y) + c and the cross-entropy is unchanged;
    bounds: max <= lse <= max + log V and ce >= 0; ties go to the lowest index."""
    rng = np.random.default_rng(8)
    Y = rng.normal(0.0, 50.0, size=(6, 300))
    t = rng.integers(0, 300, size=6)
    a, b = oracle.row_stats(Y, t), oracle.row_stats(Y + 1234.5, t)
    assert np.allclose(b["lse"], a["lse"] + 1234.5, rtol=0, atol=1e-9)
    assert np.allclose(b["ce"], a["ce"], rtol=0, atol=1e-9)
    assert (a["lse"] >= a["max"]).all() and (a["lse"] <= a["max"] + np.log(300) + 1e-12).all()
    assert (a["ce"] >= 0).all()
    T = np.array([[1.0, 3.0, 3.0, -1.0], [0.0, 0.0, 0.0, 0.0]])
    assert oracle.row_stats(T)["argmax"].tolist() == [1, 0]


def test_row_topk_worked_cases_and_brute_force():
    """Hand-worked rows (ties to the lower index, negative values), top-1 =
    argmax, distinct values against a descending sort, and brute force on
    tiny rows: no excluded entry ranks before an included one."""
    T = np.array([[1.0, 3.0, 3.0, -1.0, 2.0], [0.0, 0.0, 0.0, 0.0, 0.0], [-5.0, -1.0, -3.0, -1.0, -2.0]])
    v, i = oracle.row_topk(T, 3)
    assert i.tolist() == [[1, 2, 4], [0, 1, 2], [1, 3, 4]]
    assert v.tolist() == [[3.0, 3.0, 2.0], [0.0, 0.0, 0.0], [-1.0, -1.0, -2.0]]
    rng = np.random.default_rng(9)
    Y = rng.normal(size=(7, 50))
    assert np.array_equal(oracle.row_topk(Y, 1)[1][:, 0], oracle.row_stats(Y)["argmax"])
    v, i = oracle.row_topk(Y, 10)
    assert np.array_equal(v, -np.sort(-Y, axis=1)[:, :10])
    Yq = rng.integers(-2, 3, size=(20, 9)).astype(np.float64)   # many ties
    for k in (1, 4, 9):
        v, i = oracle.row_topk(Yq, k)
        for n in range(Yq.shape[0]):
            before = lambda a, b: Yq[n, a] > Yq[n, b] or (Yq[n, a] == Yq[n, b] and a < b)
            assert len(set(i[n])) == k
            assert all(before(i[n][j], i[n][j + 1]) for j in range(k - 1))
            assert all(before(i[n][-1], x) for x in range(9) if x not in set(i[n]))


# -------------------------------------------------------------- quantizers ---


def test_int8_quantizers_recover_exact_codes():
    """Matrices built as code x fp16 scale, each row (group) holding a code of
    magnitude 127, quantise back to the same codes and scales; an all-zero
    row gets scale 0 and codes 0."""
    rng = np.random.default_rng(21)
    codes = rng.integers(-127, 128, size=(6, 40)).astype(np.int8)
    codes[np.arange(6), rng.integers(0, 40, size=6)] = rng.choice([-127, 127], size=6)
    codes[5] = 0
    s = np.abs(rng.normal(0, 1e-2, size=6)).astype(np.float16)
    s[5] = 0
    M = codes.astype(np.float32) * s.astype(np.float32)[:, None]      # exact in fp32
    q, sq = oracle.quant_int8_rows(M)
    assert np.array_equal(q, codes) and np.array_equal(sq.view(np.uint16), s.view(np.uint16))
    g = 8
    cg = rng.integers(-127, 128, size=(3, 32)).astype(np.int8)
    cg[:, ::g] = 127
    sg = np.abs(rng.normal(0, 1e-3, size=(3, 4))).astype(np.float16)
    Mg = cg.astype(np.float32) * np.repeat(sg.astype(np.float32), g, axis=1)
    qg, sqg = oracle.quant_int8_groups(Mg, g)
    assert np.array_equal(qg, cg) and np.array_equal(sqg.view(np.uint16), sg.view(np.uint16))


def test_int8_rounding_and_bounds():
    """Ties round to even; every unclamped code is within half a step; the
    largest magnitude of a row lands on 127 (or 126 after the scale's fp16
    rounding)."""
    s = np.float32(np.float16(0.25))
    M = np.array([[127 * s, 0.5 * s, 1.5 * s, -2.5 * s, 2.5 * s, -0.5 * s]], np.float32)
    q, sq = oracle.quant_int8_rows(M)
    assert q.tolist() == [[127, 0, 2, -2, 2, 0]] and float(sq[0]) == 0.25
    rng = np.random.default_rng(22)
    X = rng.normal(0, 3.0, size=(50, 33)).astype(np.float32)
    q, sq = oracle.quant_int8_rows(X)
    step = sq.astype(np.float64)[:, None]
    assert (np.abs(X - q * step) <= step / 2 + 1e-12 * np.abs(X)).all()
    top = np.abs(q[np.arange(50), np.abs(X).argmax(axis=1)])
    assert ((top == 127) | (top == 126)).all()


def test_sc4_recovers_exact_codes_and_zero_groups():
    """R built as q4 x c8 x s_R with a code of magnitude 7 in every group and
    a group code of 255 in every row quantises back to the same components;
    an all-zero group gets group code 1, an all-zero row group codes 0."""
    rng = np.random.default_rng(23)
    V, D, g = 5, 64, 16
    q4 = rng.integers(-7, 8, size=(V, D)).astype(np.int8)
    q4[:, ::g] = 7
    c8 = rng.integers(1, 256, size=(V, D // g)).astype(np.uint8)
    c8[:, 1] = 255
    s_R = np.abs(rng.normal(0, 1e-3, size=V)).astype(np.float16)
    q4[1, 2 * g:3 * g] = 0                      # a zero group
    q4[4] = 0                                   # a zero row
    R = q4.astype(np.float32) * np.repeat(c8.astype(np.float32) * s_R.astype(np.float32)[:, None], g, axis=1)
    q, c, s = oracle.quant_sc4(R, g)
    want_c8 = c8.copy()
    want_c8[1, 2] = 1
    want_c8[4] = 0
    want_s = s_R.copy()
    want_s[4] = 0
    assert np.array_equal(q, q4) and np.array_equal(c, want_c8)
    assert np.array_equal(s.view(np.uint16), want_s.view(np.uint16))


def test_core_residual_brute_force():
    """R = W - Q(A_c) Q(B_c) against exact rational arithmetic."""
    rng = np.random.default_rng(24)
    V, D, r, g = 3, 8, 3, 4
    W = rng.normal(0, 1, size=(V, D))
    qa = rng.integers(-127, 128, size=(V, r)).astype(np.int8)
    sa = np.abs(rng.normal(0, 1e-2, size=V)).astype(np.float16)
    qb = rng.integers(-127, 128, size=(r, D)).astype(np.int8)
    sb = np.abs(rng.normal(0, 1e-2, size=(r, D // g))).astype(np.float16)
    R = oracle.core_residual(W, qa, sa, qb, sb, g)
    for v in range(V):
        for k in range(D):
            core = sum(Fraction(int(qa[v, j])) * Fraction(float(sa[v])) * Fraction(int(qb[j, k])) *
                       Fraction(float(sb[j, k // g])) for j in range(r))
            exact = Fraction(float(W[v, k])) - core
            assert abs(float(exact) - R[v, k]) <= 1e-15 * max(1.0, abs(float(exact)))


def test_quantize_end_to_end_reconstructs_w():
    """The packed head's dequantised weights plus the returned error E give
    back W (to the fp32 rounding of the residual); the packed bytes decode to
    the same components."""
    rng = np.random.default_rng(25)
    V, D, r_c, g = 37, 256, 8, 64
    W = rng.normal(0, 0.02, size=(V, D)).astype(np.float32)
    A = rng.normal(0, 1, size=(V, r_c)).astype(np.float32)
    B = rng.normal(0, 0.01, size=(r_c, D)).astype(np.float32)
    head, E = oracle.quantize(W, A, B, np.zeros((V, 0), np.float32), np.zeros((0, D), np.float32), g)
    back = oracle.w_hat(head) + E.astype(np.float64)
    assert np.allclose(back, W, rtol=0, atol=2.0 ** -23 * np.abs(W).max())
    u = oracle.unpack(oracle.pack(head), V, D, r_c, 0, g)
    assert np.array_equal(u["q4"], head.q4) and np.array_equal(u["c8"], head.c8)
    # the error is what SC4 cannot represent: half a group step (the group
    # code rounds up, so no code clamps beyond the fp16 rounding of s_R)
    step = np.repeat(head.c8.astype(np.float64) * head.s_R.astype(np.float64)[:, None], g, axis=1)
    assert (np.abs(E) <= step * (0.5 + 7 * 2.0 ** -10)).all()
    # a group whose amax is 1.3 steps of the row's unit needs group code 2
    # (rounding to 1 would clamp its largest code from 9 to 7)
    small = oracle.quant_sc4(np.array([[1.0, 0.0, 0.0051, -0.002]], np.float32), 2)
    assert small[1].tolist() == [[255, 2]] and small[0].tolist() == [[7, 0, 5, -2]]


# ---------------------------------------------------------------- fitting ---

def test_damped_covariance_worked_example():
    """H = [[1, 2], [3, 4]]: H^T H / 2 = [[5, 7], [7, 10]], mean diagonal 7.5;
    lam = 0.2 adds 1.5 on the diagonal.  bf16 inputs are exact here."""
    H = np.array([[1.0, 2.0], [3.0, 4.0]])
    C = oracle.damped_covariance(H, 0.2)
    assert np.array_equal(C, np.array([[6.5, 7.0], [7.0, 11.5]]))
    assert np.array_equal(oracle.damped_covariance(H, 0.0), np.array([[5.0, 7.0], [7.0, 10.0]]))


def test_metric_transform_closed_forms():
    """T_1 = C, T_{1/2}^2 = C, T_p T_p^{-1} = I, T_0 = I; a diagonal C gives
    diag(c^p); a rotated diagonal matrix gives the rotated powers."""
    rng = np.random.default_rng(4)
    X = rng.normal(size=(40, 6))
    C = oracle.damped_covariance(X, 0.1)
    T1, _ = oracle.metric_transform(C, 1.0)
    Th, _ = oracle.metric_transform(C, 0.5)
    Tp, Tpi = oracle.metric_transform(C, 0.75)
    T0, _ = oracle.metric_transform(C, 0.0)
    assert np.allclose(T1, C, atol=1e-12) and np.allclose(Th @ Th, C, atol=1e-12)
    assert np.allclose(Tp @ Tpi, np.eye(6), atol=1e-12) and np.allclose(T0, np.eye(6), atol=1e-12)
    d = np.array([4.0, 9.0, 16.0])
    T, Ti = oracle.metric_transform(np.diag(d), 0.5)
    assert np.allclose(T, np.diag([2.0, 3.0, 4.0]), atol=1e-14) and np.allclose(Ti, np.diag(1 / np.array([2.0, 3.0, 4.0])))
    c, s_ = np.cos(0.3), np.sin(0.3)
    Rm = np.array([[c, -s_], [s_, c]])
    T, _ = oracle.metric_transform(Rm @ np.diag([1.0, 25.0]) @ Rm.T, 0.5)
    assert np.allclose(T, Rm @ np.diag([1.0, 5.0]) @ Rm.T, atol=1e-12)


def test_rsvd_exact_on_low_rank_and_near_optimal():
    """An exactly rank-5 matrix is recovered by a rank-5 randomized SVD (to
    rounding), with the exact singular values; on a matrix with decaying
    spectrum, power iterations bring the residual to the Eckart-Young optimum
    (and never below it)."""
    rng = np.random.default_rng(5)
    M = rng.normal(size=(60, 5)) @ rng.normal(size=(5, 40))
    A, B = oracle.rsvd(M, 5, rng.normal(size=(40, 9)), 1)
    assert np.abs(A @ B - M).max() <= 1e-10 * np.abs(M).max()
    s_exact = np.linalg.svd(M, compute_uv=False)[:5]
    assert np.allclose(np.linalg.norm(A, axis=0), s_exact, rtol=1e-10)   # A = Q U S, Q U orthonormal
    U, S, Vt = np.linalg.svd(rng.normal(size=(80, 50)), full_matrices=False)
    M = (U * (0.7 ** np.arange(50))) @ Vt
    opt = np.sum((0.7 ** np.arange(50))[6:] ** 2)
    A, B = oracle.rsvd(M, 6, rng.normal(size=(50, 12)), 3)
    res = np.sum((M - A @ B) ** 2)
    assert opt * (1 - 1e-12) <= res <= opt * (1 + 1e-6)


def test_metric_correction_is_the_conditional_optimum():
    """Sec. 3.2: at p = 1/2 the metric objective is the damped logit error,
    ||Delta T||^2 = ||H Delta^T||^2 / N + lam c_bar ||Delta||^2, and the
    correction [E T]_r T^{-1} (exact SVD) attains its minimum over rank r,
    sum_{i > r} sigma_i(E T)^2; random rank-r candidates and small
    perturbations of the optimum do worse."""
    rng = np.random.default_rng(6)
    N, V, D, r, lam = 200, 30, 16, 3, 0.05
    H = rng.normal(size=(N, D)) * np.where(np.arange(D) < 2, 10.0, 1.0)
    E = rng.normal(size=(V, D))
    C = oracle.damped_covariance(H, lam)
    T, Ti = oracle.metric_transform(C, 0.5)
    cbar = np.mean(np.sum(H * H, axis=0) / N)
    Dl = rng.normal(size=(V, D))
    lhs = oracle.metric_objective(Dl, T)
    assert np.isclose(lhs, np.sum((H @ Dl.T) ** 2) / N + lam * cbar * np.sum(Dl ** 2), rtol=1e-12)
    U, S, Vt = np.linalg.svd(E @ T, full_matrices=False)
    Af, Bf = U[:, :r] * S[:r], Vt[:r] @ Ti
    best = oracle.metric_objective(E - Af @ Bf, T)
    assert np.isclose(best, np.sum(S[r:] ** 2), rtol=1e-12)
    for _ in range(20):
        Mr = rng.normal(size=(V, r)) @ rng.normal(size=(r, D))
        assert oracle.metric_objective(E - Mr, T) > best
        P = (Af + 1e-3 * rng.normal(size=(V, r))) @ (Bf + 1e-3 * rng.normal(size=(r, D)))   # still rank r
        assert oracle.metric_objective(E - P, T) > best
    # the randomized routine with power iterations reaches it closely
    A, B = oracle.rsvd(E @ T, r, rng.normal(size=(D, r + 8)), 4)
    assert oracle.metric_objective(E - A @ B @ Ti, T) <= best * (1 + 1e-3)


def test_fit_end_to_end_properties():
    """Algorithm 1 on a tiny head: the core factors span W's dominant part,
    E is W - W_d exactly (W_d rebuilt from the packed components), and the
    correction lowers the metric objective of E as the quantised factors
    allow."""
    rng = np.random.default_rng(7)
    V, D, r_c, r_r, g, N = 96, 128, 8, 8, 32, 300
    W = (rng.normal(size=(V, r_c)) @ rng.normal(size=(r_c, D)) * 0.05 + rng.normal(size=(V, D)) * 0.002)
    W = W.astype(np.float32)
    H = synth.f32_to_bf16_bits(rng.normal(size=(N, D)).astype(np.float32) * np.where(np.arange(D) < 3, 15.0, 1.0).astype(np.float32))
    head, f = oracle.fit(W, H, r_c, r_r, g, 0.5, 0.01, rng.normal(size=(D, r_c + 8)), rng.normal(size=(D, r_r + 8)), 2)
    core = f["A_c"].astype(np.float64) @ f["B_c"]
    assert np.sum((W - core) ** 2) <= 1.01 * np.sum(np.linalg.svd(W.astype(np.float64), compute_uv=False)[r_c:] ** 2)
    Wd = oracle.dequant_R(head.q4, head.c8, head.s_R, g) + \
        oracle.dequant_rows(head.A_c, head.s_Ac) @ oracle.dequant_groups(head.B_c, head.s_Bc, g)
    assert np.abs((W - Wd) - f["E"]).max() <= 1e-6 * np.abs(W).max()
    T = f["T"]
    J0 = oracle.metric_objective(f["E"], T)
    Jf = oracle.metric_objective(f["E"] - f["A_w"].astype(np.float64) @ f["B_w"], T)
    Jq = oracle.metric_objective(f["E"] - oracle.dequant_rows(head.A_w, head.s_Aw) @ oracle.dequant_groups(head.B_w, head.s_Bw, g), T)
    assert Jf < 0.8 * J0 and Jq < 0.85 * J0


def test_logit_error_pins():
    """Eq. 1: a zero head leaves the whole reference energy as error; a zero W
    leaves the packed logits' energy; brute force over tokens on a tiny case;
    divided by N it equals the metric objective at p = 1/2 without damping."""
    inp = synth.make("tiny", seed=3, V=40, D=128, N=6, r_c=8, r_r=8, g=32)
    W = synth.f32_to_bf16_bits(np.random.default_rng(2).normal(0, 0.05, size=(40, 128)).astype(np.float32))
    z = synth.zero_head(40, 128, 8, 8, 32)
    err, ref = oracle.logit_error(inp.H_bits, z, W)
    assert err == ref > 0
    err0, _ = oracle.logit_error(inp.H_bits, inp.head, np.zeros_like(W))
    assert np.isclose(err0, np.sum(oracle.logits(inp.H_bits, inp.head) ** 2), rtol=1e-14)
    H = oracle.bf16_bits_to_f64(inp.H_bits)
    Wd, Wh = oracle.bf16_bits_to_f64(W), oracle.w_hat(inp.head)
    brute = sum(float(np.dot(H[n], Wd[v] - Wh[v])) ** 2 for n in range(6) for v in range(40))
    err, _ = oracle.logit_error(inp.H_bits, inp.head, W)
    assert np.isclose(err, brute, rtol=1e-10)
    Hm = np.random.default_rng(5).normal(size=(300, 16))
    Dl = np.random.default_rng(6).normal(size=(10, 16))
    T, _ = oracle.metric_transform(oracle.damped_covariance(Hm, 0.0), 0.5)
    assert np.isclose(np.sum((Hm @ Dl.T) ** 2) / 300, oracle.metric_objective(Dl, T), rtol=1e-10)


def _fit_case():
    """A tiny head with a dominant rank-r_c part and calibration tokens whose
    first channels are outliers (so the metric is far from the identity)."""
    rng = np.random.default_rng(31)
    V, D, r_c, r_r, g, N = 48, 128, 8, 8, 32, 400
    W = (rng.normal(size=(V, r_c)) @ rng.normal(size=(r_c, D)) * 0.05 + rng.normal(size=(V, D)) * 0.002)
    W = W.astype(np.float32)
    sc = np.where(np.arange(D) < 4, 15.0, 1.0).astype(np.float32)
    H = synth.f32_to_bf16_bits(rng.normal(size=(N, D)).astype(np.float32) * sc)
    # V + 8 test columns for the correction: the sketch spans all of E T's
    # column space, so the randomized SVD is exact
    return dict(W=W, H_bits=H, r_c=r_c, r_r=r_r, g=g, p=0.75, lam=0.01,
                omega_c=rng.normal(size=(D, r_c + 8)), omega_r=rng.normal(size=(D, V + 8)), q=1)


def _correction_gap(case, f):
    """(J_f / J_opt - 1, max |A_w B_w - [E T]_r T^-1| / max |[E T]_r T^-1|):
    how far the fitted correction is from the conditional optimum, with T the
    metric of the case's calibration tokens (computed here, not taken from f)."""
    T, Ti = oracle.metric_transform(oracle.damped_covariance(oracle.bf16_bits_to_f64(case["H_bits"]), case["lam"]),
                                    case["p"])
    E = f["E"].astype(np.float64)
    U, S, Vt = np.linalg.svd(E @ T, full_matrices=False)
    r = case["r_r"]
    opt = float(np.sum(S[r:] ** 2))
    prod = f["A_w"].astype(np.float64) @ f["B_w"].astype(np.float64)
    Jf = oracle.metric_objective(E - prod, T)
    closed = (U[:, :r] * S[:r]) @ Vt[:r] @ Ti
    return Jf / opt - 1.0, float(np.abs(prod - closed).max() / np.abs(closed).max())


def test_fit_correction_reaches_the_conditional_optimum():
    """Sec. 3.2 (conditional optimum) with the Sec. 3 metric transform and
    Algorithm 1's map-back: for the core error E that oracle.fit leaves, the
    rank-r_r correction it returns attains min over rank r_r of
    ||(E - A_w B_w) T_p||_F^2 = sum_{i > r_r} sigma_i(E T_p)^2 (Eckart-Young
    in the metric), i.e. A_w B_w = [E T_p]_{r_r} T_p^{-1}.  The test matrices
    make the randomized SVD exact, so only the fp32 storage of the factors
    separates the two (the objective is flat to first order at its minimum)."""
    case = _fit_case()
    _, f = oracle.fit(case["W"], case["H_bits"], case["r_c"], case["r_r"], case["g"], case["p"], case["lam"],
                      case["omega_c"], case["omega_r"], case["q"])
    dJ, dP = _correction_gap(case, f)
    assert abs(dJ) <= 1e-6, dJ
    assert dP <= 1e-6, dP


@pytest.mark.parametrize("mutant", ["frobenius", "map_back_with_T", "metric_p_zero"])
def test_fit_pin_rejects_plausible_mistakes(monkeypatch, mutant):
    """The pin above fails for the mistakes it is there to catch, each planted
    in the oracle on the CPU: fitting E itself (T_p = I, an ordinary low-rank
    fix of the core error, which the pages say does not repair the loss),
    mapping the right factor back through T_p instead of T_p^{-1}, and
    ignoring the exponent p (T = C_lam^0)."""
    case = _fit_case()
    real = oracle.archead_oracle.metric_transform
    if mutant == "frobenius":
        fake = lambda C, p: (np.eye(C.shape[0]), np.eye(C.shape[0]))  # noqa: E731
    elif mutant == "map_back_with_T":
        fake = lambda C, p: (real(C, p)[0], real(C, p)[0])  # noqa: E731
    else:
        fake = lambda C, p: real(C, 0.0)  # noqa: E731
    monkeypatch.setattr(oracle.archead_oracle, "metric_transform", fake)
    _, f = oracle.fit(case["W"], case["H_bits"], case["r_c"], case["r_r"], case["g"], case["p"], case["lam"],
                      case["omega_c"], case["omega_r"], case["q"])
    monkeypatch.setattr(oracle.archead_oracle, "metric_transform", real)
    dJ, dP = _correction_gap(case, f)
    assert dJ > 1e-2 and dP > 1e-2, (mutant, dJ, dP)


# -------------------------------------------------------- comparison heads ---
# The storage-matched heads set beside ARCHead (results discussion of Tables 7
# and 8): group INT4 with fp16 group scales (format 1) and row INT8 (format 2).

def _alt_header_bytes(d, flags):
    return np.frombuffer(np.array([0x48435241, 1], np.uint32).tobytes() +
                         np.array([d["V"], d["D"]], np.uint64).tobytes() +
                         np.array([0, 0, d["g"], flags], np.uint32).tobytes(), np.uint8)


@pytest.mark.parametrize("fmt", [1, 2])
def test_alt_golden_positions(golden_dir, fmt):
    G = json.load(open(os.path.join(golden_dir, "format_alt_cases.json")))[f"f{fmt}"]
    d = G["dims"]
    L = oracle.layout(d["V"], d["D"], 0, 0, d["g"], fmt)
    for name, (off, size) in G["sections"].items():
        assert tuple(L[name]) == (off, size), name
    assert L["total_bytes"] == G["total_bytes"] and L["payload_bytes"] == G["payload_bytes"]
    V, D, g = d["V"], d["D"], d["g"]
    codes = np.zeros((V, D), np.int8)
    scales = np.zeros((V, D // g) if fmt == 1 else V, np.float16)
    expect = {}
    if fmt == 1:
        for c in G["nibbles"]:
            codes[c["v"], c["k"]] = c["code"]
            nib = c["code"] & 0xF
            expect[c["byte"]] = expect.get(c["byte"], 0) | (nib if c["half"] == "lo" else nib << 4)
        for c in G["group_scales"]:
            scales.view(np.uint16)[c["v"], c["t"]] = c["f16_bits"]
            expect[c["byte"]] = c["f16_bits"] & 0xFF
            expect[c["byte"] + 1] = c["f16_bits"] >> 8
            assert float(_f16_exact(c["f16_bits"])) == c["value"]
    else:
        for c in G["codes"]:
            codes[c["v"], c["k"]] = c["code"]
            expect[c["byte"]] = c["code"] & 0xFF
        for c in G["row_scale"]:
            scales.view(np.uint16)[c["v"]] = c["f16_bits"]
            expect[c["byte"]] = c["f16_bits"] & 0xFF
            expect[c["byte"] + 1] = c["f16_bits"] >> 8
    for i, b in enumerate(_alt_header_bytes(d, fmt)):
        expect[i] = int(b)
    buf = oracle.pack_alt(synth.AltHead(fmt, V, D, g, codes, scales))
    assert buf.size == G["total_bytes"]
    nz = {int(i): int(buf[i]) for i in np.flatnonzero(buf)}
    assert nz == {k: v for k, v in expect.items() if v}


def _tile8_pack_loop(q8_padded):
    """Element-by-element reading of the row-INT8 tile order (tiny shapes only)."""
    V16, D = q8_padded.shape
    out = np.zeros(V16 * D, np.uint8)
    nb = V16 // 16
    P = (0, 1, 4, 5, 2, 3, 6, 7)
    for v in range(V16):
        for k in range(D):
            b, i = divmod(v, 16)
            kt, kk = divmod(k, 128)
            s, rem = divmod(kk, 32)
            q, j = divmod(rem, 8)
            pos = (kt * nb + b) * 2048 + 32 * (16 * q + i) + 8 * s + P.index(j)
            out[pos] = int(q8_padded[v, k]) & 0xFF
    return out


@pytest.mark.parametrize("V,D", [(16, 128), (33, 256)])
def test_alt_tile8_order_matches_loop(V, D):
    _, h = synth.make_alt(2, V + D, V, D, 1, 64)
    L = oracle.layout(V, D, 0, 0, 64, 2)
    q = np.zeros((L["V16"], D), np.int8)
    q[:V] = h.codes
    off, size = L["r_codes"]
    assert np.array_equal(oracle.pack_alt(h)[off:off + size], _tile8_pack_loop(q))


@pytest.mark.parametrize("fmt,V,D,g", [(1, 100, 512, 64), (1, 37, 256, 128), (2, 100, 512, 64), (2, 9, 384, 32)])
def test_alt_pack_unpack_roundtrip(fmt, V, D, g):
    _, h = synth.make_alt(fmt, 7, V, D, 1, g)
    u = oracle.unpack_alt(oracle.pack_alt(h), V, D, g, fmt)
    assert u["magic"] == 0x48435241 and u["flags"] == fmt
    assert np.array_equal(u["codes"], h.codes)
    assert np.array_equal(u["scales"].view(np.uint16), h.scales.view(np.uint16))


def test_alt_storage_matches_pages():
    """Table 7 discussion: the GPTQ-style INT4 head takes 25.78% of the BF16
    head (4 bits per weight + one fp16 scale per 128); Table 8 discussion: row
    INT8 takes about twice the storage of the 25.6% ARCHead head."""
    V, D = 151936, 4096
    f1 = oracle.alt_persistent_bytes(V, D, 128, 1)
    assert f1 / (2 * V * D) == (4 + 16 / 128) / 16 == 0.2578125
    assert round(100 * f1 / (2 * V * D), 2) == 25.78
    f2 = oracle.alt_persistent_bytes(V, D, 128, 2)
    assert f2 / (2 * V * D) == 0.5 + 1 / D
    ratio = f2 / oracle.persistent_bytes(V, D, 6, 6, 128)
    assert 1.9 < ratio < 2.0
    for fmt in (1, 2):  # the layout's payload is the persistent size, and nothing is V x D at 16 bits
        L = oracle.layout(V, D, 0, 0, 128, fmt)
        assert L["payload_bytes"] == oracle.alt_persistent_bytes(V, D, 128, fmt)
        assert L["total_bytes"] < 2 * V * D


def test_alt_group_int4_is_sc4_when_scales_factor():
    """A group scale that is exactly c8 * s_R (s_R a power of two, so the
    product is exact in fp16) makes the format-1 head the same matrix as the
    format-0 head with r_c = r_r = 0: two different decode routines of the
    oracle must agree."""
    inp = synth.make("tiny", seed=21, V=200, D=256, N=3, r_c=0, r_r=0, g=64)
    h = inp.head
    h.s_R[:] = np.float16(2.0 ** -12)
    sg = (h.c8.astype(np.float64) * 2.0 ** -12).astype(np.float16)
    assert np.array_equal(sg.astype(np.float64), h.c8.astype(np.float64) * 2.0 ** -12)
    alt = synth.AltHead(1, h.V, h.D, h.g, h.q4.copy(), sg)
    Y0 = oracle.logits(inp.H_bits, h)
    Y1 = oracle.logits_alt(inp.H_bits, alt)
    assert np.abs(Y0 - Y1).max() <= 1e-12 * np.abs(Y0).max()


@pytest.mark.parametrize("fmt", [1, 2])
def test_alt_exact_rational(fmt):
    """Comparison-head logits against exact integer evaluation."""
    H_bits, h = synth.make_alt(fmt, 31 + fmt, 40, 256, 3, 64)
    SH = 133
    Hi = np.array([[int(_bf16_exact(int(b)) * (1 << SH)) for b in row] for row in H_bits], dtype=object)

    def f16i(a):
        a = np.asarray(a)
        return np.array([int(_f16_exact(int(b)) * (1 << 24)) for b in a.view(np.uint16).reshape(-1)],
                        dtype=object).reshape(a.shape)

    s = f16i(h.scales)
    Wq = h.codes.astype(object) * (np.repeat(s, h.g, axis=1) if fmt == 1 else s[:, None])
    exact = np.array([[float(Fraction(int(x), 1 << (SH + 24))) for x in row] for row in Hi.dot(Wq.T)])
    Y = oracle.logits_alt(H_bits, h)
    assert np.abs(Y - exact).max() <= 1e-12 * np.abs(exact).max()


def test_quant_group_int4_worked_cases():
    """Worked groups (g = 4): amax 0.7 -> s = fp16(0.1); codes rint(x / s);
    a group of zeros has scale 0 and codes 0; |code| never passes 7 on the
    largest element, and -8 is reachable only through rounding below -7.5."""
    M = np.array([[0.7, -0.35, 0.07, -0.7, 0.0, 0.0, 0.0, 0.0]], np.float32)
    q, s = oracle.quant_group_int4(M, 4)
    s0 = np.float32(np.float16(np.float32(0.7) / np.float32(7)))
    assert s.view(np.uint16)[0, 0] == np.float16(np.float32(0.7) / np.float32(7)).view(np.uint16)
    assert q[0, :4].tolist() == [int(np.rint(np.float32(x) / s0)) for x in M[0, :4]]
    assert q[0, 0] == 7 and q[0, 3] == -7
    assert s[0, 1] == 0 and not q[0, 4:].any()
    rng = np.random.default_rng(3)
    R = rng.standard_normal((50, 256)).astype(np.float32)
    q, s = oracle.quant_group_int4(R, 64)
    deq = q.astype(np.float32) * np.repeat(s.astype(np.float32), 64, axis=1)
    assert np.abs(q).max() <= 8
    assert np.all(np.abs(R - deq) <= 0.5 * np.repeat(s.astype(np.float32), 64, axis=1) * 1.01 + 1e-7)
