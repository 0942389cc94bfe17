"""Python binding of libarchead: the packed ARCHead LM-head forward on MI355X.

The functions below carry the names of the C entry points in
``include/archead.h`` and only marshal arguments: every step of the forward
runs in the library's HIP kernels.  Torch is used for device memory and the
current stream.  Importing the package fails loudly when ``libarchead.so`` has
not been built (``python compressed_output_head_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libarchead.so")

ARCHEAD_OK = 0
ARCHEAD_BF16, ARCHEAD_F32 = 1, 2
ARCHEAD_PATH_AUTO, ARCHEAD_PATH_DECODE, ARCHEAD_PATH_TILE = 0, 1, 2
# storage formats (archead_format): the method's head and the two comparison heads
ARCHEAD_FMT_ARCHEAD, ARCHEAD_FMT_GROUP_INT4, ARCHEAD_FMT_ROW_INT8 = 0, 1, 2
# main kernels (archead_main_kernel), by the names the profiler shows
KERNEL_NAMES = {0: "tile32_kernel", 1: "small_decode_kernel", 2: "decode_kernel", 3: "batch_kernel"}
STATUS = {0: "OK", 1: "E_NULL", 2: "E_DIMS", 3: "E_UNSUPPORTED", 4: "E_DTYPE", 5: "E_SHAPE",
          6: "E_ALIGN", 7: "E_WORKSPACE", 8: "E_HIP", 9: "E_VALUE", 10: "E_SIZE"}
EXPORTS = ("archead_pack_layout", "archead_workspace_bytes", "archead_workspace_bytes_path", "archead_main_kernel",
           "archead_pack",
           "archead_logits", "archead_logits_noalloc",
           "archead_logits_path", "archead_logits_events", "archead_stats_workspace_bytes",
           "archead_logits_stats", "archead_quantize", "archead_topk_workspace_bytes", "archead_logits_topk",
           "archead_fit_workspace_bytes", "archead_fit", "archead_logit_error_workspace_bytes",
           "archead_logit_error",
           "archead_status_string", "archead_format_version")


class ArcheadError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {archead_status_string(status)}")


class ArcheadDims(ctypes.Structure):
    _fields_ = [("V", ctypes.c_int64), ("D", ctypes.c_int64),
                ("r_c", ctypes.c_int32), ("r_r", ctypes.c_int32), ("g", ctypes.c_int32),
                ("format", ctypes.c_int32)]


class ArcheadSpan(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("bytes", ctypes.c_uint64)]


_SECTIONS = ("header", "r_codes", "r_gcodes", "r_rowscale", "a_codes", "a_scales", "b_codes", "b_scales")


class ArcheadLayout(ctypes.Structure):
    _fields_ = ([("format_version", ctypes.c_uint32), ("alignment", ctypes.c_uint32),
                 ("total_bytes", ctypes.c_uint64), ("payload_bytes", ctypes.c_uint64),
                 ("header_bytes", ctypes.c_uint64)]
                + [(n, ArcheadSpan) for n in _SECTIONS]
                + [("padded_rows", ctypes.c_int64)])


class ArcheadHostComponents(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q4", "c8", "s_R", "A_c", "A_w", "s_Ac", "s_Aw", "B_c", "B_w", "s_Bc", "s_Bw", "s_G", "q8")]


class ArcheadTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class ArcheadPackedHead(ctypes.Structure):
    _fields_ = [("dims", ArcheadDims), ("buffer", ctypes.c_void_p), ("buffer_bytes", ctypes.c_uint64),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64)]


class ArcheadRowStats(ctypes.Structure):
    _fields_ = [("row_max", ctypes.c_void_p), ("row_argmax", ctypes.c_void_p), ("row_lse", ctypes.c_void_p),
                ("row_ce", ctypes.c_void_p), ("targets", ctypes.c_void_p)]


class ArcheadDenseHead(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("W_stride", ctypes.c_int64), ("W_dtype", ctypes.c_int32),
                ("A_c", ctypes.c_void_p), ("B_c", ctypes.c_void_p), ("A_w", ctypes.c_void_p),
                ("B_w", ctypes.c_void_p)]


class ArcheadFitInputs(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("W_stride", ctypes.c_int64), ("W_dtype", ctypes.c_int32),
                ("H", ctypes.c_void_p), ("H_rows", ctypes.c_int64), ("H_stride", ctypes.c_int64),
                ("omega_c", ctypes.c_void_p), ("omega_r", ctypes.c_void_p), ("p", ctypes.c_float),
                ("lam", ctypes.c_float), ("oversample", ctypes.c_int32), ("power_iters", ctypes.c_int32)]


class ArcheadFitOutputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("A_c", "B_c", "A_w", "B_w", "E")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python compressed_output_head_amd/build.py`")
    # torch ships its own libamdhip64 (same soname).  Loading torch first makes
    # the dynamic linker bind libarchead to that one HIP runtime, so torch's
    # streams, events and allocations are valid handles for the library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.archead_pack_layout.argtypes = [P(ArcheadDims), P(ArcheadLayout)]
    lib.archead_workspace_bytes.argtypes = [P(ArcheadDims), ctypes.c_int64, P(ctypes.c_uint64)]
    lib.archead_workspace_bytes_path.argtypes = [P(ArcheadDims), ctypes.c_int64, ctypes.c_int, P(ctypes.c_uint64)]
    lib.archead_main_kernel.argtypes = [P(ArcheadDims), ctypes.c_int64, ctypes.c_int, P(ctypes.c_int)]
    lib.archead_pack.argtypes = [P(ArcheadDims), P(ArcheadHostComponents), ctypes.c_void_p, ctypes.c_uint64]
    lib.archead_logits.argtypes = [P(ArcheadTensor), P(ArcheadPackedHead), P(ArcheadTensor), ctypes.c_void_p]
    lib.archead_logits_noalloc.argtypes = [P(ArcheadTensor), P(ArcheadPackedHead), P(ArcheadTensor), ctypes.c_void_p]
    lib.archead_logits_path.argtypes = [P(ArcheadTensor), P(ArcheadPackedHead), P(ArcheadTensor),
                                        ctypes.c_int, ctypes.c_void_p]
    lib.archead_logits_events.argtypes = [P(ArcheadTensor), P(ArcheadPackedHead), P(ArcheadTensor),
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.archead_stats_workspace_bytes.argtypes = [P(ArcheadDims), ctypes.c_int64, P(ctypes.c_uint64)]
    lib.archead_logits_stats.argtypes = [P(ArcheadTensor), P(ArcheadPackedHead), P(ArcheadRowStats),
                                         ctypes.c_void_p]
    lib.archead_quantize.argtypes = [P(ArcheadDims), P(ArcheadDenseHead), ctypes.c_void_p, ctypes.c_uint64,
                                     P(ArcheadTensor), ctypes.c_void_p]
    lib.archead_topk_workspace_bytes.argtypes = [P(ArcheadDims), ctypes.c_int64, P(ctypes.c_uint64)]
    lib.archead_logits_topk.argtypes = [P(ArcheadTensor), P(ArcheadPackedHead), ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.archead_fit_workspace_bytes.argtypes = [P(ArcheadDims), ctypes.c_int32, P(ctypes.c_uint64)]
    lib.archead_fit.argtypes = [P(ArcheadDims), P(ArcheadFitInputs), ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                ctypes.c_uint64, P(ArcheadFitOutputs), ctypes.c_void_p]
    lib.archead_logit_error_workspace_bytes.argtypes = [P(ArcheadDims), ctypes.c_int64, P(ctypes.c_uint64)]
    lib.archead_logit_error.argtypes = [P(ArcheadTensor), P(ArcheadPackedHead), P(ArcheadTensor),
                                        P(ctypes.c_double), ctypes.c_void_p]
    lib.archead_status_string.argtypes = [ctypes.c_int]
    lib.archead_status_string.restype = ctypes.c_char_p
    lib.archead_format_version.argtypes = []
    for name in EXPORTS:
        if name not in ("archead_status_string",):
            getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def _dims(V, D, r_c, r_r, g, fmt=ARCHEAD_FMT_ARCHEAD) -> ArcheadDims:
    return ArcheadDims(int(V), int(D), int(r_c), int(r_r), int(g), int(fmt))


def _check(status: int, where: str):
    if status != ARCHEAD_OK:
        raise ArcheadError(status, where)


# ------------------------------------------------------------- host calls ---

def archead_status_string(status: int) -> str:
    return lib.archead_status_string(int(status)).decode()


def archead_format_version() -> int:
    return lib.archead_format_version()


def archead_pack_layout(V, D, r_c, r_r, g, fmt=ARCHEAD_FMT_ARCHEAD) -> dict:
    """Section offsets/sizes of the packed buffer (see include/archead.h)."""
    L = ArcheadLayout()
    _check(lib.archead_pack_layout(ctypes.byref(_dims(V, D, r_c, r_r, g, fmt)), ctypes.byref(L)),
           "archead_pack_layout")
    out = {n: (getattr(L, n).offset, getattr(L, n).bytes) for n in _SECTIONS}
    out.update(total_bytes=L.total_bytes, payload_bytes=L.payload_bytes, header_bytes=L.header_bytes,
               format_version=L.format_version, alignment=L.alignment, V16=L.padded_rows)
    return out


def archead_workspace_bytes(V, D, r_c, r_r, g, n_tokens: int, fmt=ARCHEAD_FMT_ARCHEAD) -> int:
    b = ctypes.c_uint64()
    _check(lib.archead_workspace_bytes(ctypes.byref(_dims(V, D, r_c, r_r, g, fmt)), int(n_tokens),
                                       ctypes.byref(b)), "archead_workspace_bytes")
    return b.value


def archead_workspace_bytes_path(V, D, r_c, r_r, g, n_tokens: int, path: int, fmt=ARCHEAD_FMT_ARCHEAD) -> int:
    b = ctypes.c_uint64()
    _check(lib.archead_workspace_bytes_path(ctypes.byref(_dims(V, D, r_c, r_r, g, fmt)), int(n_tokens), int(path),
                                            ctypes.byref(b)), "archead_workspace_bytes_path")
    return b.value


def archead_main_kernel(V, D, r_c, r_r, g, n_tokens: int, path: int = ARCHEAD_PATH_AUTO,
                        fmt=ARCHEAD_FMT_ARCHEAD) -> str:
    """Name of the main kernel a call of n_tokens rows on `path` launches."""
    k = ctypes.c_int()
    _check(lib.archead_main_kernel(ctypes.byref(_dims(V, D, r_c, r_r, g, fmt)), int(n_tokens), int(path),
                                   ctypes.byref(k)), "archead_main_kernel")
    return KERNEL_NAMES[k.value]


def archead_stats_workspace_bytes(V, D, r_c, r_r, g, n_tokens: int, fmt=ARCHEAD_FMT_ARCHEAD) -> int:
    b = ctypes.c_uint64()
    _check(lib.archead_stats_workspace_bytes(ctypes.byref(_dims(V, D, r_c, r_r, g, fmt)), int(n_tokens),
                                             ctypes.byref(b)), "archead_stats_workspace_bytes")
    return b.value


def archead_topk_workspace_bytes(V, D, r_c, r_r, g, n_tokens: int, fmt=ARCHEAD_FMT_ARCHEAD) -> int:
    out = ctypes.c_uint64(0)
    _check(lib.archead_topk_workspace_bytes(ctypes.byref(_dims(V, D, r_c, r_r, g, fmt)), int(n_tokens),
                                            ctypes.byref(out)), "archead_topk_workspace_bytes")
    return out.value


def _ptr(a: Optional[np.ndarray], dtype):
    if a is None or a.size == 0:
        return None, None
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def _head_dims(head):
    """(V, D, r_c, r_r, g, fmt) of an ARCHead (attributes V, D, r_c, r_r, g) or
    of a comparison head (attributes fmt, V, D, g; no factors)."""
    fmt = int(getattr(head, "fmt", ARCHEAD_FMT_ARCHEAD))
    if fmt == ARCHEAD_FMT_ARCHEAD:
        return head.V, head.D, head.r_c, head.r_r, head.g, fmt
    return head.V, head.D, 0, 0, head.g, fmt


def archead_pack(head) -> np.ndarray:
    """Serialise host components into a uint8 array: an ARCHead (attributes
    V, D, r_c, r_r, g, q4, c8, s_R, A_c, A_w, s_Ac, s_Aw, B_c, B_w, s_Bc, s_Bw)
    or a comparison head (attributes fmt, V, D, g, codes, scales: fmt 1 reads
    codes as q4 and scales as s_G, fmt 2 codes as q8 and scales as s_R)."""
    dims = _head_dims(head)
    d = _dims(*dims)
    L = archead_pack_layout(*dims)
    out = np.empty(L["total_bytes"], np.uint8)
    keep = []
    comp = ArcheadHostComponents()
    fmt = dims[5]
    if fmt == ARCHEAD_FMT_ARCHEAD:
        spec = [("q4", np.int8, head.q4), ("c8", np.uint8, head.c8), ("s_R", np.float16, head.s_R),
                ("A_c", np.int8, head.A_c), ("A_w", np.int8, head.A_w), ("s_Ac", np.float16, head.s_Ac),
                ("s_Aw", np.float16, head.s_Aw), ("B_c", np.int8, head.B_c), ("B_w", np.int8, head.B_w),
                ("s_Bc", np.float16, head.s_Bc), ("s_Bw", np.float16, head.s_Bw)]
    elif fmt == ARCHEAD_FMT_GROUP_INT4:
        spec = [("q4", np.int8, head.codes), ("s_G", np.float16, head.scales)]
    else:
        spec = [("q8", np.int8, head.codes), ("s_R", np.float16, head.scales)]
    for name, dt, val in spec:
        arr, p = _ptr(val, dt)
        keep.append(arr)
        setattr(comp, name, p)
    _check(lib.archead_pack(ctypes.byref(d), ctypes.byref(comp), out.ctypes.data, out.nbytes), "archead_pack")
    return out


# ----------------------------------------------------------- device calls ---

def _torch():
    import torch
    return torch


class PackedHead:
    """A packed head resident in device memory plus a reusable workspace."""

    def __init__(self, V, D, r_c, r_r, g, buffer, device=None, fmt=ARCHEAD_FMT_ARCHEAD):
        torch = _torch()
        self.V, self.D, self.r_c, self.r_r, self.g = int(V), int(D), int(r_c), int(r_r), int(g)
        self.fmt = int(fmt)
        self.layout = archead_pack_layout(V, D, r_c, r_r, g, fmt)
        if isinstance(buffer, np.ndarray):
            buffer = torch.from_numpy(buffer).to(device or "cuda")
        if buffer.dtype != torch.uint8 or buffer.numel() < self.layout["total_bytes"]:
            raise ValueError("packed buffer must be uint8 with at least layout total_bytes elements")
        self.buffer = buffer
        self.workspace = None

    @classmethod
    def from_components(cls, head, device="cuda") -> "PackedHead":
        V, D, r_c, r_r, g, fmt = _head_dims(head)
        return cls(V, D, r_c, r_r, g, archead_pack(head), device=device, fmt=fmt)

    @property
    def dims(self):
        return dict(V=self.V, D=self.D, r_c=self.r_c, r_r=self.r_r, g=self.g, fmt=self.fmt)

    def ensure_workspace(self, n_tokens: int, stats: bool = False, topk: bool = False, logit_error: bool = False,
                         path: int = ARCHEAD_PATH_AUTO):
        torch = _torch()
        if logit_error or topk or stats:
            size = archead_logit_error_workspace_bytes if logit_error else archead_topk_workspace_bytes if topk \
                else archead_stats_workspace_bytes
            need = size(self.V, self.D, self.r_c, self.r_r, self.g, n_tokens, fmt=self.fmt)
        else:
            need = archead_workspace_bytes_path(self.V, self.D, self.r_c, self.r_r, self.g, n_tokens, path,
                                                fmt=self.fmt)
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=self.buffer.device)
        return self.workspace

    def struct(self) -> ArcheadPackedHead:
        ws = self.workspace
        return ArcheadPackedHead(_dims(self.V, self.D, self.r_c, self.r_r, self.g, self.fmt),
                                 self.buffer.data_ptr(), self.buffer.numel(),
                                 ws.data_ptr() if ws is not None else None,
                                 ws.numel() if ws is not None else 0)


def _tensor(t) -> ArcheadTensor:
    torch = _torch()
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    code = {torch.bfloat16: ARCHEAD_BF16, torch.float32: ARCHEAD_F32}.get(t.dtype, 0)
    return ArcheadTensor(t.data_ptr(), t.shape[0], t.shape[1], t.stride(0), code)


def archead_logits_path(H, head: PackedHead, Y, path: int = ARCHEAD_PATH_AUTO, stream=None):
    """Y = H W_hat^T on the GPU.  H: bf16 [N, D]; Y: fp32 or bf16 [N, V] (written)."""
    torch = _torch()
    head.ensure_workspace(H.shape[0], path=path)
    if stream is None:
        stream = torch.cuda.current_stream(H.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    h, y, p = _tensor(H), _tensor(Y), head.struct()
    _check(lib.archead_logits_path(ctypes.byref(h), ctypes.byref(p), ctypes.byref(y), int(path),
                                   ctypes.c_void_p(stream)), "archead_logits")
    return Y


def archead_logits_events(H, head: PackedHead, Y, path: int, ev_begin, ev_end, stream=None):
    """archead_logits_path that also records two torch.cuda.Event objects
    around the main kernel (each must have been recorded once, so it exists)."""
    torch = _torch()
    head.ensure_workspace(H.shape[0], path=path)
    if stream is None:
        stream = torch.cuda.current_stream(H.device).cuda_stream
    h, y, p = _tensor(H), _tensor(Y), head.struct()
    _check(lib.archead_logits_events(ctypes.byref(h), ctypes.byref(p), ctypes.byref(y), int(path),
                                     ctypes.c_void_p(stream), ctypes.c_void_p(ev_begin.cuda_event),
                                     ctypes.c_void_p(ev_end.cuda_event)), "archead_logits_events")
    return Y


def archead_logits(H, head: PackedHead, Y, stream=None):
    return archead_logits_path(H, head, Y, ARCHEAD_PATH_AUTO, stream)


# workspace the library holds per GPU for archead_logits_noalloc
ARCHEAD_NOALLOC_SCRATCH_BYTES = 16 << 20


def archead_logits_noalloc(H, head: PackedHead, Y, stream=None):
    """archead_logits with the library's own per-GPU workspace: allocates
    nothing (head's workspace is neither allocated nor used)."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(H.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    h, y, p = _tensor(H), _tensor(Y), head.struct()
    _check(lib.archead_logits_noalloc(ctypes.byref(h), ctypes.byref(p), ctypes.byref(y), ctypes.c_void_p(stream)),
           "archead_logits_noalloc")
    return Y


def logits(H, head: PackedHead, out_dtype=None, path: int = ARCHEAD_PATH_AUTO):
    """Allocate Y and run the forward; returns Y (fp32 unless out_dtype says bf16)."""
    torch = _torch()
    Y = torch.empty((H.shape[0], head.V), dtype=out_dtype or torch.float32, device=H.device)
    return archead_logits_path(H, head, Y, path)


def archead_logits_stats(H, head: PackedHead, targets=None, stream=None, outputs=("max", "argmax", "lse", "ce")):
    """Per-row statistics of Y = H W_hat^T without writing Y: returns a dict of
    device tensors of N elements -- "max" and "lse" (fp32), "argmax" (int32),
    and "ce" (fp32, cross-entropy of ``targets``, an int32 device tensor of N
    elements) when targets are given."""
    torch = _torch()
    N = H.shape[0]
    head.ensure_workspace(N, stats=True)
    if stream is None:
        stream = torch.cuda.current_stream(H.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    out = {}
    for k in outputs:
        if k == "ce" and targets is None:
            continue
        out[k] = torch.empty(N, dtype=torch.int32 if k == "argmax" else torch.float32, device=H.device)
    if targets is not None and (targets.dtype != torch.int32 or targets.numel() != N or not targets.is_contiguous()):
        raise ValueError("targets must be a contiguous int32 tensor of N elements")
    st = ArcheadRowStats(*(out[k].data_ptr() if k in out else None for k in ("max", "argmax", "lse", "ce")),
                         targets.data_ptr() if targets is not None else None)
    h, p = _tensor(H), head.struct()
    _check(lib.archead_logits_stats(ctypes.byref(h), ctypes.byref(p), ctypes.byref(st), ctypes.c_void_p(stream)),
           "archead_logits_stats")
    return out


def archead_quantize(W, A_c, B_c, A_w, B_w, g: int, with_error: bool = False, stream=None):
    """Quantise a dense head on the GPU into a packed head (the packing step:
    INT8 factors, SC4 residual of the quantised core).  W: bf16 or fp32 [V, D]
    device tensor; A_c [V, r_c], B_c [r_c, D], A_w [V, r_r], B_w [r_r, D]:
    fp32 device tensors.  Returns (PackedHead, E) where E is the fp32 [V, D]
    error left after the residual codes when ``with_error``, else None."""
    torch = _torch()
    V, D = W.shape
    r_c, r_r = A_c.shape[1], A_w.shape[1]
    for name, t, shape in (("A_c", A_c, (V, r_c)), ("B_c", B_c, (r_c, D)), ("A_w", A_w, (V, r_r)),
                           ("B_w", B_w, (r_r, D))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {shape}")
    L = archead_pack_layout(V, D, r_c, r_r, g)
    buf = torch.empty(L["total_bytes"], dtype=torch.uint8, device=W.device)
    E = torch.empty((V, D), dtype=torch.float32, device=W.device) if with_error else None
    if stream is None:
        stream = torch.cuda.current_stream(W.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    w = _tensor(W)
    src = ArcheadDenseHead(w.data, w.row_stride, w.dtype,
                           *(t.data_ptr() if t.numel() else None for t in (A_c, B_c, A_w, B_w)))
    e = _tensor(E) if E is not None else None
    _check(lib.archead_quantize(ctypes.byref(_dims(V, D, r_c, r_r, g)), ctypes.byref(src),
                                ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                ctypes.byref(e) if e is not None else None, ctypes.c_void_p(stream)),
           "archead_quantize")
    return PackedHead(V, D, r_c, r_r, g, buf), E


def archead_logits_topk(H, head: PackedHead, k: int, stream=None):
    """The k largest logits of each row of Y = H W_hat^T and their indices:
    returns (values fp32 [N, k], indices int32 [N, k]) as device tensors,
    largest first, lower index first among equal values."""
    torch = _torch()
    N = H.shape[0]
    head.ensure_workspace(N, topk=True)
    if stream is None:
        stream = torch.cuda.current_stream(H.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    vals = torch.empty((N, k), dtype=torch.float32, device=H.device)
    idx = torch.empty((N, k), dtype=torch.int32, device=H.device)
    h, p = _tensor(H), head.struct()
    _check(lib.archead_logits_topk(ctypes.byref(h), ctypes.byref(p), int(k), ctypes.c_void_p(vals.data_ptr()),
                                   ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(stream)), "archead_logits_topk")
    return vals, idx


def archead_fit_workspace_bytes(V, D, r_c, r_r, g, oversample: int) -> int:
    out = ctypes.c_uint64(0)
    _check(lib.archead_fit_workspace_bytes(ctypes.byref(_dims(V, D, r_c, r_r, g)), int(oversample),
                                           ctypes.byref(out)), "archead_fit_workspace_bytes")
    return out.value


def archead_fit(W, H, omega_c, omega_r, r_c: int, r_r: int, g: int, p: float = 0.75, lam: float = 0.01,
                oversample: int = 8, power_iters: int = 2, outputs: bool = False, stream=None):
    """Build a packed head from a dense one on the GPU (the whole construction).
    W: bf16 or fp32 [V, D]; H: bf16 [N, D] calibration hidden states; omega_c
    [D, r_c + oversample] and omega_r [D, r_r + oversample]: fp32 Gaussian
    test matrices (device tensors).  Returns (PackedHead, factors) where
    factors is a dict of fp32 device tensors A_c, B_c, A_w, B_w, E when
    ``outputs``, else None.  The call waits for the stream."""
    torch = _torch()
    V, D = W.shape
    L = archead_pack_layout(V, D, r_c, r_r, g)
    buf = torch.empty(L["total_bytes"], dtype=torch.uint8, device=W.device)
    ws = torch.empty(max(archead_fit_workspace_bytes(V, D, r_c, r_r, g, oversample), 256), dtype=torch.uint8,
                     device=W.device)
    if stream is None:
        stream = torch.cuda.current_stream(W.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    for name, t, shape in (("omega_c", omega_c, (D, r_c + oversample)), ("omega_r", omega_r, (D, r_r + oversample))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {shape}")
    if H.dtype != torch.bfloat16 or H.dim() != 2 or H.shape[1] != D or H.stride(1) != 1:
        raise ValueError("H must be a bf16 [N, D] tensor with unit column stride")
    w = _tensor(W)
    inp = ArcheadFitInputs(w.data, w.row_stride, w.dtype, H.data_ptr(), H.shape[0], H.stride(0),
                           omega_c.data_ptr(), omega_r.data_ptr(), float(p), float(lam), int(oversample),
                           int(power_iters))
    f = None
    if outputs:
        f = {"A_c": torch.empty((V, r_c), dtype=torch.float32, device=W.device),
             "B_c": torch.empty((r_c, D), dtype=torch.float32, device=W.device),
             "A_w": torch.empty((V, r_r), dtype=torch.float32, device=W.device),
             "B_w": torch.empty((r_r, D), dtype=torch.float32, device=W.device),
             "E": torch.empty((V, D), dtype=torch.float32, device=W.device)}
        outs = ArcheadFitOutputs(*(f[k].data_ptr() if f[k].numel() else None for k in ("A_c", "B_c", "A_w", "B_w", "E")))
    _check(lib.archead_fit(ctypes.byref(_dims(V, D, r_c, r_r, g)), ctypes.byref(inp), ctypes.c_void_p(buf.data_ptr()),
                           buf.numel(), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                           ctypes.byref(outs) if outputs else None, ctypes.c_void_p(stream)), "archead_fit")
    return PackedHead(V, D, r_c, r_r, g, buf), f


def archead_logit_error_workspace_bytes(V, D, r_c, r_r, g, n_tokens: int, fmt=ARCHEAD_FMT_ARCHEAD) -> int:
    out = ctypes.c_uint64(0)
    _check(lib.archead_logit_error_workspace_bytes(ctypes.byref(_dims(V, D, r_c, r_r, g, fmt)), int(n_tokens),
                                                   ctypes.byref(out)), "archead_logit_error_workspace_bytes")
    return out.value


def archead_logit_error(H, head: PackedHead, W, stream=None):
    """(sum of squared logit differences against the dense bf16 head W, sum of
    squared dense logits) over the rows of H, as Python floats (the call waits)."""
    torch = _torch()
    head.ensure_workspace(H.shape[0], logit_error=True)
    if stream is None:
        stream = torch.cuda.current_stream(H.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    sums = (ctypes.c_double * 2)()
    h, p, w = _tensor(H), head.struct(), _tensor(W)
    _check(lib.archead_logit_error(ctypes.byref(h), ctypes.byref(p), ctypes.byref(w), sums, ctypes.c_void_p(stream)),
           "archead_logit_error")
    return sums[0], sums[1]
