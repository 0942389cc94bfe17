"""CPU oracle for the packed ARCHead LM-head forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import or call this module.  The product path never does: it runs on
the HIP kernels and fails loudly when they are missing.

Source of the definitions: "ARCHead: Activation-Metric Residual Correction for
Large Language Model Output Heads" (arXiv:2608.02703), Sec. 3 and Algorithm 1.

* The head is a quantised low-rank core plus an SC4 residual,
  W_d = Q(A_c) Q(B_c) + SC4(R)  (Sec. 3, quantized-core equation and the
  sentence after it: SC4 is a packed signed-INT4 residual with quantised group
  scales; A_c B_c has rank r_c).
* The correction factors are stored with row-wise INT8 (A_w) and group-wise
  INT8 (B_w) quantisation (Sec. 3, packed-variant paragraph; Algorithm 1).
* Inference evaluates Y = H W_d^T + (H B_w^T) A_w^T (Algorithm 1, last step).
  There is no approximation at inference time, so the oracle writes out the
  plain definition: decode every stored code exactly, rebuild
  W_hat = R_hat + A_c_hat B_c_hat + A_w_hat B_w_hat in fp64, and return
  H W_hat^T in fp64.
* The serialized module holds only the residual codes and scales, the core
  factors, the correction factors and shape metadata; its persistent size is
  the sum of numel x element size over those tensors (Sec. 3, persistent-size
  equation).  ``layout``/``pack``/``unpack`` below implement the byte format of
  that module independently of the library.

Readings taken where the page leaves the format open (the bit width of Q_b,
SC4 internals, nibble order, the tile order of the stored residual) are the
byte format described in ``FORMAT`` below.  The forward is fp64 throughout;
all dequantised values are exact in fp64.

Around the forward, each with its own section below: per-row statistics and
top-k of the logits (the quantities of the pages' quality metrics), the
quantisers and the core residual of the packing step (decisions in fp32, as
their section states), the fitting steps of Algorithm 1 (damped covariance,
metric transform, randomized SVD, correction map-back) and the logit error of
Eq. 1.  Every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, worked examples, library routines or brute force.
"""
from __future__ import annotations

import numpy as np

FORMAT = """
Packed head, format version 1 (all integers little-endian).
  V16 = ceil(V/16)*16 rows (rows >= V are zero), nb = V16/16 row blocks,
  nkt = D/128 k-tiles, ng = D/g groups, r = r_c + r_r, nA = [r_c>0] + [r_r>0].
  Sections in order, each starting on a 256-byte boundary:
   header     64 B: u32 magic 0x48435241, u32 version 1, u64 V, u64 D,
                    u32 r_c, u32 r_r, u32 g, u32 flags 0, 24 zero bytes
   r_codes    nkt*nb tiles of 1024 B, k-tile major: tile (b, kt) starts at
              (kt*nb + b)*1024.  In tile (b, kt), byte 16*l + 4*s + c
              (l in [0,64), s in [0,4), c in [0,4)) holds the two INT4 codes
              (two's complement) of row v = 16*b + (l mod 16) at
              k = 128*kt + 32*s + 8*(l div 16) + 2*c   (low nibble)
              and k + 1                                (high nibble).
   r_gcodes   V16*ng B, row-major: byte v*ng + t = uint8 group code of row v,
              group t (columns t*g .. t*g+g-1).
   r_rowscale V16 fp16: per-row residual scale s_R.
   a_codes    V16*r int8, row-major; row v = [A_c[v, :r_c] | A_w[v, :r_r]].
   a_scales   V16*nA fp16; row v = [s_Ac[v] if r_c>0, s_Aw[v] if r_r>0].
   b_codes    r*D int8, row-major; rows [B_c; B_w].
   b_scales   r*ng fp16, row-major; rows [s_Bc; s_Bw].
  Dequantisation:
   R_hat[v,k] = q4[v,k] * c8[v, k//g] * s_R[v]
   A_hat[v,j] = a_codes[v,j] * (s_Ac[v] if j < r_c else s_Aw[v])
   B_hat[j,k] = b_codes[j,k] * b_scales[j, k//g]
"""

MAGIC = 0x48435241
FORMAT_VERSION = 1
ALIGN = 256
HEADER_BYTES = 64

_SECTIONS = ("r_codes", "r_gcodes", "r_rowscale", "a_codes", "a_scales",
             "b_codes", "b_scales")


def _up(x, a):
    return (x + a - 1) // a * a


def layout(V, D, r_c, r_r, g, fmt=0):
    """Offsets and sizes of every section of the packed buffer (see FORMAT;
    fmt 1 and 2 are the comparison heads of ALT_FORMAT)."""
    if V < 1 or D < 128 or D % 128 or g < 2 or g % 2 or D % g or r_c < 0 or r_r < 0:
        raise ValueError("unsupported dims")
    if fmt not in (0, 1, 2) or (fmt and (r_c or r_r)):
        raise ValueError("unsupported format")
    V16 = _up(V, 16)
    r = r_c + r_r
    ng = D // g
    nA = int(r_c > 0) + int(r_r > 0)
    if fmt == 0:
        sizes = dict(
            r_codes=V16 * D // 2,
            r_gcodes=V16 * ng,
            r_rowscale=2 * V16,
            a_codes=V16 * r,
            a_scales=2 * V16 * nA,
            b_codes=r * D,
            b_scales=2 * r * ng,
        )
    else:
        sizes = {name: 0 for name in _SECTIONS}
        if fmt == 1:
            sizes.update(r_codes=V16 * D // 2, r_gcodes=2 * V16 * ng)
        else:
            sizes.update(r_codes=V16 * D, r_rowscale=2 * V16)
    out = dict(header=(0, HEADER_BYTES))
    off = _up(HEADER_BYTES, ALIGN)
    for name in _SECTIONS:
        out[name] = (off, sizes[name])
        off = _up(off + sizes[name], ALIGN)
    out["total_bytes"] = off
    out["payload_bytes"] = sum(sizes.values())
    out["V16"] = V16
    return out


def persistent_bytes(V, D, r_c, r_r, g):
    """Sum of numel x element size over the stored tensors, for V a multiple
    of 16 (Sec. 3, persistent-size equation): residual codes at 4 bits, group
    codes at 8 bits, fp16 row scale, INT8 factor codes, fp16 factor scales."""
    r = r_c + r_r
    nA = int(r_c > 0) + int(r_r > 0)
    elems = [
        (V * D, 0.5),           # SC4 codes, two per byte
        (V * (D // g), 1),      # uint8 group codes
        (V, 2),                 # fp16 row scale
        (V * r, 1),             # INT8 A_c | A_w
        (V * nA, 2),            # fp16 A row scales
        (r * D, 1),             # INT8 B_c ; B_w
        (r * (D // g), 2),      # fp16 B group scales
    ]
    return int(sum(n * b for n, b in elems))


# ---------------------------------------------------------------- packing ---

def _nibbles_to_tiles(nib):
    """[V16, D] nibbles -> r_codes bytes.  Writing k = 128*kt + 32*s + 8*q + 2*c + h
    and v = 16*b + i, the byte order is (kt, b, q, i, s, c) and h selects the
    low (h=0) or high (h=1) nibble; lane l = 16*q + i."""
    V16, D = nib.shape
    t = nib.reshape(V16 // 16, 16, D // 128, 4, 4, 4, 2)        # b i kt s q c h
    t = t.transpose(2, 0, 4, 1, 3, 5, 6)                        # kt b q i s c h
    return (t[..., 0] | (t[..., 1] << 4)).astype(np.uint8).reshape(-1)


def _tiles_to_nibbles(raw, V16, D):
    """Inverse of ``_nibbles_to_tiles``."""
    t = raw.reshape(D // 128, V16 // 16, 4, 16, 4, 4)            # kt b q i s c
    both = np.stack([t & 0xF, t >> 4], axis=-1)                  # kt b q i s c h
    return both.transpose(1, 3, 0, 4, 2, 5, 6).reshape(V16, D)   # b i kt s q c h


def pack(head) -> np.ndarray:
    """Serialise a ``synth.Head`` into the packed byte format (FORMAT)."""
    V, D, r_c, r_r, g = head.V, head.D, head.r_c, head.r_r, head.g
    L = layout(V, D, r_c, r_r, g)
    V16 = L["V16"]
    buf = np.zeros(L["total_bytes"], np.uint8)

    hdr = np.zeros(HEADER_BYTES, np.uint8)
    hdr[0:4] = np.frombuffer(np.uint32(MAGIC).tobytes(), np.uint8)
    hdr[4:8] = np.frombuffer(np.uint32(FORMAT_VERSION).tobytes(), np.uint8)
    hdr[8:16] = np.frombuffer(np.uint64(V).tobytes(), np.uint8)
    hdr[16:24] = np.frombuffer(np.uint64(D).tobytes(), np.uint8)
    hdr[24:28] = np.frombuffer(np.uint32(r_c).tobytes(), np.uint8)
    hdr[28:32] = np.frombuffer(np.uint32(r_r).tobytes(), np.uint8)
    hdr[32:36] = np.frombuffer(np.uint32(g).tobytes(), np.uint8)
    buf[0:HEADER_BYTES] = hdr

    def put(name, arr):
        off, size = L[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert raw.size == size, (name, raw.size, size)
        buf[off:off + size] = raw

    q = np.zeros((V16, D), np.int8)
    q[:V] = head.q4
    if q.min() < -8 or q.max() > 7:
        raise ValueError("INT4 code out of range")
    nib = (q.view(np.uint8) & 0xF)                               # two's complement nibble
    put("r_codes", _nibbles_to_tiles(nib))

    ng = D // g
    c8 = np.zeros((V16, ng), np.uint8)
    c8[:V] = head.c8
    put("r_gcodes", c8)

    sR = np.zeros(V16, np.float16)
    sR[:V] = head.s_R
    put("r_rowscale", sR)

    A = np.zeros((V16, r_c + r_r), np.int8)
    A[:V, :r_c] = head.A_c
    A[:V, r_c:] = head.A_w
    put("a_codes", A)

    cols = []
    if r_c > 0:
        cols.append(head.s_Ac)
    if r_r > 0:
        cols.append(head.s_Aw)
    sA = np.zeros((V16, len(cols)), np.float16)
    for i, col in enumerate(cols):
        sA[:V, i] = col
    put("a_scales", sA)

    put("b_codes", np.concatenate([head.B_c.reshape(r_c, D), head.B_w.reshape(r_r, D)], 0))
    put("b_scales", np.concatenate([head.s_Bc.reshape(r_c, ng), head.s_Bw.reshape(r_r, ng)], 0))
    return buf


def unpack(buf: np.ndarray, V, D, r_c, r_r, g) -> dict:
    """Read every component back out of a packed buffer (inverse of ``pack``)."""
    L = layout(V, D, r_c, r_r, g)
    V16 = L["V16"]
    ng = D // g
    buf = np.asarray(buf, np.uint8)
    hdr = buf[:HEADER_BYTES]

    def get(name, dtype):
        off, size = L[name]
        return buf[off:off + size].view(dtype)

    nib = _tiles_to_nibbles(get("r_codes", np.uint8), V16, D)
    q4 = nib.astype(np.int8)
    q4[q4 >= 8] -= 16
    c8 = get("r_gcodes", np.uint8).reshape(V16, ng)
    s_R = get("r_rowscale", np.float16)
    A = get("a_codes", np.int8).reshape(V16, r_c + r_r)
    nA = int(r_c > 0) + int(r_r > 0)
    sA = get("a_scales", np.float16).reshape(V16, nA)
    B = get("b_codes", np.int8).reshape(r_c + r_r, D)
    sB = get("b_scales", np.float16).reshape(r_c + r_r, ng)
    return dict(
        magic=int(hdr[0:4].view(np.uint32)[0]), version=int(hdr[4:8].view(np.uint32)[0]),
        V=int(hdr[8:16].view(np.uint64)[0]), D=int(hdr[16:24].view(np.uint64)[0]),
        r_c=int(hdr[24:28].view(np.uint32)[0]), r_r=int(hdr[28:32].view(np.uint32)[0]),
        g=int(hdr[32:36].view(np.uint32)[0]),
        q4=q4[:V], c8=c8[:V], s_R=s_R[:V],
        A_c=A[:V, :r_c], A_w=A[:V, r_c:],
        s_Ac=sA[:V, 0] if r_c > 0 else np.zeros(V, np.float16),
        s_Aw=sA[:V, nA - 1] if r_r > 0 else np.zeros(V, np.float16),
        B_c=B[:r_c], B_w=B[r_c:], s_Bc=sB[:r_c], s_Bw=sB[r_c:],
        pad_rows_zero=bool(np.all(q4[V:] == 0) and np.all(c8[V:] == 0) and np.all(A[V:] == 0)),
    )


# ------------------------------------------------------------ number decode ---

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32; widen and convert exactly."""
    u = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_to_f64(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 to fp64, exact (subnormals and zero included)."""
    return np.asarray(x, np.float16).astype(np.float64)


# ------------------------------------------------------------ dequantise ---

def dequant_R(q4, c8, s_R, g):
    """SC4 residual: R_hat[v,k] = q4[v,k] * c8[v, k//g] * s_R[v] (exact in fp64)."""
    grp = np.repeat(c8.astype(np.float64), g, axis=1)              # [V, D]
    return q4.astype(np.float64) * grp * f16_to_f64(s_R)[:, None]


def dequant_rows(codes, row_scale):
    """Row-wise INT8: A_hat[v,j] = code[v,j] * s[v]."""
    return codes.astype(np.float64) * f16_to_f64(row_scale)[:, None]


def dequant_groups(codes, group_scale, g):
    """Group-wise INT8 along D: B_hat[j,k] = code[j,k] * s[j, k//g]."""
    return codes.astype(np.float64) * np.repeat(f16_to_f64(group_scale), g, axis=1)


def w_hat(head, v0=0, v1=None):
    """Rows v0..v1 of W_hat = R_hat + A_c_hat B_c_hat + A_w_hat B_w_hat (fp64)."""
    v1 = head.V if v1 is None else v1
    g = head.g
    W = dequant_R(head.q4[v0:v1], head.c8[v0:v1], head.s_R[v0:v1], g)
    if head.r_c:
        W += dequant_rows(head.A_c[v0:v1], head.s_Ac[v0:v1]) @ dequant_groups(head.B_c, head.s_Bc, g)
    if head.r_r:
        W += dequant_rows(head.A_w[v0:v1], head.s_Aw[v0:v1]) @ dequant_groups(head.B_w, head.s_Bw, g)
    return W


def logits(H_bits, head, rows=None, cols=None, v_chunk=8192):
    """Y_ref = H W_hat^T in fp64 (Algorithm 1, inference step).

    ``rows`` selects token rows of H, ``cols`` selects vocabulary rows of the
    head (both optional index arrays); W_hat is rebuilt in chunks of
    ``v_chunk`` vocabulary rows so the V x D fp64 matrix is never whole.
    """
    H = bf16_bits_to_f64(H_bits if rows is None else H_bits[rows])
    if cols is not None:
        cols = np.asarray(cols)
        return H @ _w_hat_rows(head, cols).T
    Y = np.empty((H.shape[0], head.V), np.float64)
    for v0 in range(0, head.V, v_chunk):
        v1 = min(head.V, v0 + v_chunk)
        Y[:, v0:v1] = H @ w_hat(head, v0, v1).T
    return Y


def _w_hat_rows(head, cols):
    g = head.g
    W = dequant_R(head.q4[cols], head.c8[cols], head.s_R[cols], g)
    if head.r_c:
        W += dequant_rows(head.A_c[cols], head.s_Ac[cols]) @ dequant_groups(head.B_c, head.s_Bc, g)
    if head.r_r:
        W += dequant_rows(head.A_w[cols], head.s_Aw[cols]) @ dequant_groups(head.B_w, head.s_Bw, g)
    return W


# ------------------------------------------------------- comparison heads ---
#
# The storage-matched heads the pages set beside ARCHead (ARCHead, results
# discussion of Table 7: a GPTQ-style INT4 head at 25.78% of the BF16 head's
# storage; of Table 8: a row-INT8 head, more accurate but about twice the
# storage).  The page gives their storage, not their bytes; ALT_FORMAT is the
# reading taken, in the same container as FORMAT.

ALT_FORMAT = """
Comparison heads, format field f of the header's flags word (bytes 36..39),
r_c = r_r = 0, same header and 256-byte section alignment as FORMAT; sections
not listed are empty.
  f = 1, group INT4 with fp16 group scales (symmetric, no zero point):
   r_codes    the INT4 tiles of FORMAT (same byte positions);
   r_gcodes   V16*ng fp16, row-major: v*ng + t = scale of row v, group t.
   W_hat[v,k] = q4[v,k] * s_G[v, k//g]
   storage: 4 bits per weight + 16 bits per group = (4 + 16/g)/16 of BF16.
  f = 2, row INT8:
   r_codes    nkt*nb tiles of 2048 B, k-tile major: tile (b, kt) starts at
              (kt*nb + b)*2048.  In tile (b, kt), byte 32*l + 8*s + p
              (l in [0,64), s in [0,4), p in [0,8)) holds the INT8 code of row
              v = 16*b + (l mod 16) at k = 128*kt + 32*s + 8*(l div 16) + P[p],
              P = (0, 1, 4, 5, 2, 3, 6, 7).
   r_rowscale V16 fp16: s[v].
   W_hat[v,k] = q8[v,k] * s[v]
   storage: 8 bits per weight + 16 bits per row = (8 + 16/D)/16 of BF16.
"""

ALT_PERM8 = (0, 1, 4, 5, 2, 3, 6, 7)


def alt_persistent_bytes(V, D, g, fmt):
    """Sum of numel x element size over a comparison head's stored tensors
    (V a multiple of 16)."""
    if fmt == 1:
        return V * D // 2 + 2 * V * (D // g)
    if fmt == 2:
        return V * D + 2 * V
    raise ValueError(fmt)


def _bytes_to_tiles8(q8):
    """[V16, D] int8 codes -> row-INT8 tile bytes (ALT_FORMAT f = 2).  Writing
    k = 128*kt + 32*s + 8*q + P[p] and v = 16*b + i, the byte order is
    (kt, b, q, i, s, p); lane l = 16*q + i."""
    V16, D = q8.shape
    t = q8.reshape(V16 // 16, 16, D // 128, 4, 4, 8)             # b i kt s q j
    t = t[..., list(ALT_PERM8)]                                    # byte p holds column P[p]
    t = t.transpose(2, 0, 4, 1, 3, 5)                              # kt b q i s p
    return np.ascontiguousarray(t).view(np.uint8).reshape(-1)


def _tiles8_to_bytes(raw, V16, D):
    """Inverse of ``_bytes_to_tiles8``."""
    t = np.asarray(raw, np.uint8).view(np.int8).reshape(D // 128, V16 // 16, 4, 16, 4, 8)   # kt b q i s p
    t = t.transpose(1, 3, 0, 4, 2, 5)                              # b i kt s q p
    out = np.empty_like(t)
    out[..., list(ALT_PERM8)] = t                                  # column P[p] from byte p
    return out.reshape(V16, D)


def _header(V, D, r_c, r_r, g, flags):
    hdr = np.zeros(HEADER_BYTES, np.uint8)
    hdr[0:4] = np.frombuffer(np.uint32(MAGIC).tobytes(), np.uint8)
    hdr[4:8] = np.frombuffer(np.uint32(FORMAT_VERSION).tobytes(), np.uint8)
    hdr[8:16] = np.frombuffer(np.uint64(V).tobytes(), np.uint8)
    hdr[16:24] = np.frombuffer(np.uint64(D).tobytes(), np.uint8)
    hdr[24:28] = np.frombuffer(np.uint32(r_c).tobytes(), np.uint8)
    hdr[28:32] = np.frombuffer(np.uint32(r_r).tobytes(), np.uint8)
    hdr[32:36] = np.frombuffer(np.uint32(g).tobytes(), np.uint8)
    hdr[36:40] = np.frombuffer(np.uint32(flags).tobytes(), np.uint8)
    return hdr


def pack_alt(head) -> np.ndarray:
    """Serialise a comparison head (attributes fmt, V, D, g, codes, scales) into
    ALT_FORMAT.  fmt 1: codes [V, D] in [-8, 7], scales [V, D/g] fp16; fmt 2:
    codes [V, D] in [-127, 127], scales [V] fp16."""
    V, D, g, fmt = head.V, head.D, head.g, head.fmt
    L = layout(V, D, 0, 0, g, fmt)
    V16 = L["V16"]
    buf = np.zeros(L["total_bytes"], np.uint8)
    buf[0:HEADER_BYTES] = _header(V, D, 0, 0, g, fmt)

    def put(name, arr):
        off, size = L[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert raw.size == size, (name, raw.size, size)
        buf[off:off + size] = raw

    q = np.zeros((V16, D), np.int8)
    q[:V] = head.codes
    if fmt == 1:
        if q.min() < -8 or q.max() > 7:
            raise ValueError("INT4 code out of range")
        put("r_codes", _nibbles_to_tiles(q.view(np.uint8) & 0xF))
        sg = np.zeros((V16, D // g), np.float16)
        sg[:V] = head.scales
        put("r_gcodes", sg)
    else:
        if q.min() < -127:
            raise ValueError("INT8 code out of range")
        put("r_codes", _bytes_to_tiles8(q))
        sr = np.zeros(V16, np.float16)
        sr[:V] = head.scales
        put("r_rowscale", sr)
    return buf


def unpack_alt(buf, V, D, g, fmt) -> dict:
    """Read a comparison head back out of its packed buffer."""
    L = layout(V, D, 0, 0, g, fmt)
    V16 = L["V16"]
    buf = np.asarray(buf, np.uint8)

    def get(name, dtype):
        off, size = L[name]
        return buf[off:off + size].view(dtype)

    hdr = buf[:HEADER_BYTES]
    out = dict(magic=int(hdr[0:4].view(np.uint32)[0]), flags=int(hdr[36:40].view(np.uint32)[0]))
    if fmt == 1:
        q = _tiles_to_nibbles(get("r_codes", np.uint8), V16, D).astype(np.int8)
        q[q >= 8] -= 16
        out.update(codes=q[:V], scales=get("r_gcodes", np.float16).reshape(V16, D // g)[:V])
    else:
        q = _tiles8_to_bytes(get("r_codes", np.uint8), V16, D)
        out.update(codes=q[:V], scales=get("r_rowscale", np.float16)[:V])
    return out


def w_hat_alt(head, v0=0, v1=None):
    """Rows v0..v1 of a comparison head's W_hat (fp64, exact)."""
    v1 = head.V if v1 is None else v1
    q = head.codes[v0:v1].astype(np.float64)
    if head.fmt == 1:
        return q * np.repeat(f16_to_f64(head.scales[v0:v1]), head.g, axis=1)
    return q * f16_to_f64(head.scales[v0:v1])[:, None]


def logits_alt(H_bits, head, rows=None, v_chunk=8192):
    """Y_ref = H W_hat^T of a comparison head in fp64."""
    H = bf16_bits_to_f64(H_bits if rows is None else H_bits[rows])
    Y = np.empty((H.shape[0], head.V), np.float64)
    for v0 in range(0, head.V, v_chunk):
        v1 = min(head.V, v0 + v_chunk)
        Y[:, v0:v1] = H @ w_hat_alt(head, v0, v1).T
    return Y


def quant_group_int4(M32, g):
    """Group-wise (g columns) symmetric INT4 with fp16 scales, the reading of
    the GPTQ-style head's storage with round-to-nearest codes:
    s = fp16(amax / 7), code = clamp(rint(x / s), -8, 7), 0 where s = 0
    (decisions in fp32).  Returns (codes int8 [n, D], scales fp16 [n, D/g])."""
    M32 = np.asarray(M32, np.float32)
    n, D = M32.shape
    G = M32.reshape(n * (D // g), g)
    s = (np.abs(G).max(axis=1) / np.float32(7)).astype(np.float16)
    s32 = s.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32 > 0, np.rint(G / np.where(s32 > 0, s32, np.float32(1))), 0)
    return np.clip(q, -8, 7).astype(np.int8).reshape(n, D), s.reshape(n, D // g)


# -------------------------------------------------------------- statistics ---

def row_argmax(Y):
    """Per-row argmax; exact ties go to the lowest vocabulary index."""
    return np.argmax(Y, axis=1)


def top2_gap(Y):
    """Per-row gap between the largest and second-largest logit."""
    part = np.partition(Y, Y.shape[1] - 2, axis=1)
    return part[:, -1] - part[:, -2]


def row_stats(Y, targets=None):
    """Per-row statistics that the logits' consumers need, in fp64.

    The pages assess a head by what the vocabulary distribution softmax(Y[n])
    gives downstream: perplexity and added cross-entropy (ARCHead, Abstract)
    and agreement of the top-ranked token (ARCHead, results discussion of
    Table 8).  Per row n of Y:
      max[n]    = max_v Y[n, v]
      argmax[n] = the smallest v with Y[n, v] = max[n]
      lse[n]    = log sum_v exp(Y[n, v])           (log of softmax's normaliser)
      ce[n]     = lse[n] - Y[n, targets[n]]        (-log softmax(Y[n])[target])
    lse is evaluated as max + log sum_v exp(Y - max), so rows with large
    logits do not overflow.
    """
    Y = np.asarray(Y, np.float64)
    m = Y.max(axis=1)
    out = {"max": m, "argmax": np.argmax(Y, axis=1),
           "lse": m + np.log(np.exp(Y - m[:, None]).sum(axis=1))}
    if targets is not None:
        t = np.asarray(targets, np.int64)
        out["ce"] = out["lse"] - Y[np.arange(Y.shape[0]), t]
    return out


def row_topk(Y, k):
    """The k largest entries of each row of Y with their column indices, what
    top-k agreement compares (ARCHead, results discussion of Table 8:
    top-1/5/10).  Order: larger value first, lower index first among equal
    values (a unique answer).  Returns (values [N, k], indices [N, k] int64)."""
    Y = np.asarray(Y)
    N, V = Y.shape
    idx = np.empty((N, k), np.int64)
    for n in range(N):
        order = np.lexsort((np.arange(V), -Y[n]))   # primary key -Y, then the index
        idx[n] = order[:k]
    return np.take_along_axis(Y, idx, axis=1), idx


# ------------------------------------------------------------- quantizers ---
#
# The packing step of Algorithm 1 (ARCHead, Algorithm 1 and the Sec. 3
# quantized-core sentence): the core factors are quantised (Q_b), the residual
# the quantised core leaves, R = W - Q(A_c) Q(B_c), goes to SC4, and the
# correction factors are stored with row-wise (A_w) and group-wise (B_w) INT8.
# The page fixes no rounding rule, scale formula or range; the readings here
# are symmetric absmax scaling with round-half-to-even:
#   INT8 (rows of A, or g-column groups of rows of B): s = fp16(amax / 127),
#     code = clamp(rint(x / s), -127, 127), 0 where s = 0;
#   SC4 (rows of R in g-column groups): with m_t the group's amax,
#     s_R = fp16(max_t m_t / (7 * 255)),
#     c8_t = clamp(ceil(m_t / (7 s_R)), 1, 255) (the smallest step that keeps
#     the group within [-7, 7], up to the fp16 rounding of s_R),
#     q4 = clamp(rint(r / (c8_t s_R)), -8, 7); s_R = 0 gives c8 = 0, q4 = 0.
# Every decision (the division and the rounding to an integer, the fp16
# rounding of a scale) is taken in fp32 from fp32 operands, the precision the
# GPU kernels use; the residual itself is accumulated in fp64 over the core
# rank in index order (each product is exact in fp64) and then rounded once
# to fp32.  E = W - W_d, the error the correction is fitted to, is returned as
# fp32(R) - fp32(SC4 dequantised R).

def quant_int8_rows(M32):
    """Row-wise symmetric INT8 of a float32 matrix: (codes int8, scales fp16)."""
    M32 = np.asarray(M32, np.float32)
    if M32.shape[1] == 0:
        return np.zeros(M32.shape, np.int8), np.zeros(M32.shape[0], np.float16)
    amax = np.abs(M32).max(axis=1)
    s = (amax / np.float32(127)).astype(np.float16)
    s32 = s.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32 > 0, np.rint(M32 / np.where(s32 > 0, s32, np.float32(1))), 0)
    return np.clip(q, -127, 127).astype(np.int8), s


def quant_int8_groups(M32, g):
    """Group-wise (g columns) symmetric INT8 of a float32 matrix:
    (codes int8 [n, D], scales fp16 [n, D/g])."""
    M32 = np.asarray(M32, np.float32)
    n, D = M32.shape
    q, s = quant_int8_rows(M32.reshape(n * (D // g), g))
    return q.reshape(n, D), s.reshape(n, D // g)


def quant_sc4(R32, g):
    """SC4 of a float32 residual: (q4 int8 in [-8, 7], c8 uint8 [V, D/g], s_R fp16)."""
    R32 = np.asarray(R32, np.float32)
    V, D = R32.shape
    ng = D // g
    m = np.abs(R32).reshape(V, ng, g).max(axis=2)                     # [V, ng]
    s_R = (m.max(axis=1) / np.float32(7 * 255)).astype(np.float16)
    sR32 = s_R.astype(np.float32)
    den = np.float32(7) * sR32                                         # exact
    ok = (sR32 > 0)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c8 = np.where(ok, np.clip(np.ceil(m / np.where(ok, den[:, None], np.float32(1))), 1, 255), 0)
    c8 = c8.astype(np.uint8)
    scale = np.repeat(c8.astype(np.float32) * sR32[:, None], g, axis=1)   # exact
    okk = scale > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        q4 = np.where(okk, np.clip(np.rint(R32 / np.where(okk, scale, np.float32(1))), -8, 7), 0)
    return q4.astype(np.int8), c8, s_R


def core_residual(W64, qa, sa, qb, sb, g):
    """R = W - Q(A_c) Q(B_c) in fp64, the core rank accumulated in index order."""
    acc = np.zeros_like(W64)
    a = qa.astype(np.float64) * f16_to_f64(sa)[:, None]                # [V, r_c], exact
    b = qb.astype(np.float64) * np.repeat(f16_to_f64(sb), g, axis=1)   # [r_c, D], exact
    for j in range(qa.shape[1]):
        acc = acc + a[:, j:j + 1] * b[j:j + 1, :]                      # exact products
    return W64 - acc


def quantize(W, A_c, B_c, A_w, B_w, g):
    """Quantise a dense head and its factors into the packed components.

    W: [V, D] as bf16 bit patterns (uint16) or float32; A_c [V, r_c], B_c
    [r_c, D], A_w [V, r_r], B_w [r_r, D]: float32.  Returns (head, E) where
    head has the attributes ``pack`` reads and E is float32 [V, D]."""
    from types import SimpleNamespace
    W = np.asarray(W)
    W64 = bf16_bits_to_f64(W) if W.dtype == np.uint16 else W.astype(np.float32).astype(np.float64)
    V, D = W64.shape
    r_c, r_r = A_c.shape[1], A_w.shape[1]
    qa, sa = quant_int8_rows(A_c)
    qb, sb = quant_int8_groups(B_c, g) if r_c else (np.zeros((0, D), np.int8), np.zeros((0, D // g), np.float16))
    R32 = core_residual(W64, qa, sa, qb, sb, g).astype(np.float32)
    q4, c8, s_R = quant_sc4(R32, g)
    deq = (q4.astype(np.float32) * np.repeat(c8.astype(np.float32) * s_R.astype(np.float32)[:, None], g, axis=1))
    E = R32 - deq
    qaw, saw = quant_int8_rows(A_w)
    qbw, sbw = quant_int8_groups(B_w, g) if r_r else (np.zeros((0, D), np.int8), np.zeros((0, D // g), np.float16))
    head = SimpleNamespace(V=V, D=D, r_c=r_c, r_r=r_r, g=g, q4=q4, c8=c8, s_R=s_R,
                           A_c=qa, s_Ac=sa, B_c=qb, s_Bc=sb, A_w=qaw, s_Aw=saw, B_w=qbw, s_Bw=sbw)
    return head, E


def logit_error(H_bits, head, W):
    """The logit error of Eq. 1 before the 1/N: sum over tokens and vocabulary
    of (H W^T - H W_hat^T)^2, and the reference energy sum of (H W^T)^2.
    H_bits [N, D] and W [V, D] are bf16 bit patterns; fp64 throughout."""
    H = bf16_bits_to_f64(H_bits)
    Yd = H @ bf16_bits_to_f64(W).T
    Yp = logits(H_bits, head)
    return float(np.sum((Yd - Yp) ** 2)), float(np.sum(Yd ** 2))


# ---------------------------------------------------------------- fitting ---
#
# The construction of Algorithm 1 (ARCHead, Sec. 3 and Algorithm 1): the core
# is a rank-r_c approximation of W (quantised, then the residual goes to SC4);
# the correction is fitted to the core error E = W - W_d in a damped
# activation metric.  Readings:
#   - damping as the Sec. 3 metric definition states it: C_lam = C + lam c_bar I
#     with C = H^T H / N and c_bar the mean diagonal of C (Algorithm 1's prose
#     writes C + lam I; the mean-diagonal scaling makes lam scale-free);
#   - T_p = Q Lam^p Q^T from the eigendecomposition C_lam = Q Lam Q^T, and
#     T_p^{-1} = Q Lam^{-p} Q^T;
#   - both low-rank approximations are randomized truncated SVDs (the Sec. 3
#     sentence names one for the correction; the core uses the same routine):
#     Y = M Omega, q rounds of re-orthonormalised power iteration, Q = qr(Y),
#     B = Q^T M, B = U S V^T, and the factors are A = Q U_r S_r, B = V_r^T
#     (the singular values go to the left factor);
#   - the correction's right factor is mapped back: A_w = left factor of
#     [E T_p]_r, B_w = (its right factor) T_p^{-1}.
# The Gaussian test matrices Omega are inputs, so the GPU path can use the
# same ones.

def damped_covariance(H, lam):
    """C_lam = H^T H / N + lam * mean(diag(H^T H / N)) * I  (fp64)."""
    H = np.asarray(H, np.float64)
    C = H.T @ H / H.shape[0]
    return C + lam * np.mean(np.diag(C)) * np.eye(C.shape[0])


def metric_transform(C_lam, p):
    """(T_p, T_p^{-1}) from the eigendecomposition of the damped covariance."""
    lam, Q = np.linalg.eigh(np.asarray(C_lam, np.float64))
    return (Q * lam ** p) @ Q.T, (Q * lam ** (-p)) @ Q.T


def rsvd(M, r, omega, q):
    """Randomized rank-r truncated SVD of M with test matrix omega [D, k >= r]
    and q power iterations: returns (A [V, r], B [r, D]) with A B ~ M."""
    M = np.asarray(M, np.float64)
    Y = M @ np.asarray(omega, np.float64)
    for _ in range(q):
        Qy = np.linalg.qr(Y)[0]
        Qz = np.linalg.qr(M.T @ Qy)[0]
        Y = M @ Qz
    Q = np.linalg.qr(Y)[0]
    U, S, Vt = np.linalg.svd(Q.T @ M, full_matrices=False)
    return (Q @ U[:, :r]) * S[:r], Vt[:r]


def metric_objective(Delta, T):
    """||Delta T||_F^2: at p = 1/2 the damped logit error of Eq. 1."""
    return float(np.sum((np.asarray(Delta, np.float64) @ T) ** 2))


def fit(W, H_bits, r_c, r_r, g, p, lam, omega_c, omega_r, q):
    """Algorithm 1 end to end.  W: [V, D] bf16 bits (uint16) or float32;
    H_bits: calibration hidden states [N, D] as bf16 bits.  Returns (head, f)
    where head is what ``pack`` reads and f holds the fp32 factors A_c, B_c,
    A_w, B_w, the core error E and the metric transforms."""
    W = np.asarray(W)
    W64 = bf16_bits_to_f64(W) if W.dtype == np.uint16 else W.astype(np.float32).astype(np.float64)
    V, D = W64.shape
    none = (np.zeros((V, 0), np.float32), np.zeros((0, D), np.float32))
    A_c, B_c = none
    if r_c:
        A_c, B_c = rsvd(W64, r_c, omega_c, q)
        A_c, B_c = A_c.astype(np.float32), B_c.astype(np.float32)
    _, E = quantize(W, A_c, B_c, *none, g)
    T, Tinv = metric_transform(damped_covariance(bf16_bits_to_f64(H_bits), lam), p)
    A_w, B_w = none
    if r_r:
        A_w, Bt = rsvd(E.astype(np.float64) @ T, r_r, omega_r, q)
        A_w, B_w = A_w.astype(np.float32), (Bt @ Tinv).astype(np.float32)
    head, _ = quantize(W, A_c, B_c, A_w, B_w, g)
    return head, dict(A_c=A_c, B_c=B_c, A_w=A_w, B_w=B_w, E=E, T=T, Tinv=Tinv)
