/*
 * archead.h -- C ABI of the packed ARCHead LM-head forward for AMD MI355X (gfx950).
 *
 * Method: "ARCHead: Activation-Metric Residual Correction for Large Language
 * Model Output Heads" (arXiv:2608.02703).  The packed head stores
 *   - an SC4 residual: signed INT4 codes with quantised group scales
 *     (Sec. 3, quantized-core equation and the sentence after it),
 *   - a low-rank core A_c B_c held as quantised factors (same equation),
 *   - the activation-metric correction A_w (row-wise INT8) and B_w
 *     (group-wise INT8) (Sec. 3, packed-variant paragraph; Algorithm 1),
 * and inference evaluates  Y = H W_d^T + (H B_w^T) A_w^T  (Algorithm 1, last
 * step), with W_d = Q(A_c) Q(B_c) + SC4(R).  This library computes exactly that
 * forward from the packed bytes; it never forms the V x D matrix.  Around the
 * forward: per-row statistics and top-k of the logits, the logit error of
 * Eq. 1, and the construction itself (packing, and the full fit of Algorithm 1).
 *
 * Conventions for every entry point:
 *   - All functions return an archead_status (0 = ARCHEAD_OK).  They never
 *     abort, throw or print.  Arguments are checked on the host before any
 *     HIP call; on a non-zero status nothing has been enqueued.
 *   - The caller owns all memory.  The library allocates nothing on the
 *     device and keeps no pointer after a call returns, except that
 *     archead_fit and archead_logit_error create rocBLAS handles for the call
 *     (rocBLAS and rocSOLVER allocate their own scratch; archead_fit also a
 *     second stream) and wait for the stream before returning.
 *   - Device pointers must stay valid until the stream has passed the work
 *     enqueued by the call.  Calls on different streams need different
 *     workspaces; the library holds no global state and is re-entrant.
 *   - The comparison heads (archead_format other than ARCHEAD_FMT_ARCHEAD) are
 *     served by archead_pack_layout, archead_pack, archead_workspace_bytes(_path),
 *     archead_main_kernel and archead_logits(_path, _events); every other
 *     entry point gives E_UNSUPPORTED for them.
 */
#ifndef ARCHEAD_H
#define ARCHEAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ARCHEAD_API __attribute__((visibility("default")))
#else
#define ARCHEAD_API
#endif

#define ARCHEAD_FORMAT_VERSION 1
#define ARCHEAD_MAGIC 0x48435241u /* "ARCH" little-endian, first word of a packed buffer */
#define ARCHEAD_ALIGNMENT 256

typedef enum {
  ARCHEAD_OK = 0,
  ARCHEAD_E_NULL = 1,        /* a required pointer is NULL                        */
  ARCHEAD_E_DIMS = 2,        /* dims are invalid (V<1, D not a multiple of 128, D % g != 0, rank < 0,
                                unknown format, a comparison head with factors) */
  ARCHEAD_E_UNSUPPORTED = 3, /* valid but not implemented (g not in {32,64,128,256}, rank not a multiple of 8,
                                rank above 1024, a forced decode path the decode kernel does not take,
                                section offsets past 32 bits, a comparison head where only the
                                ARCHead format is served) */
  ARCHEAD_E_DTYPE = 4,       /* H is not bf16, or Y is neither fp32 nor bf16       */
  ARCHEAD_E_SHAPE = 5,       /* H.cols != D, Y.cols != V, Y.rows != H.rows, bad strides */
  ARCHEAD_E_ALIGN = 6,       /* buffer/workspace not 256-byte aligned, H rows not 16-byte aligned,
                                Y not aligned to its element size                 */
  ARCHEAD_E_WORKSPACE = 7,   /* workspace smaller than archead_workspace_bytes()   */
  ARCHEAD_E_HIP = 8,         /* a kernel launch reported an error                  */
  ARCHEAD_E_VALUE = 9,       /* archead_pack: an INT4 code outside [-8, 7]          */
  ARCHEAD_E_SIZE = 10        /* packed buffer smaller than archead_layout.total_bytes */
} archead_status;

typedef enum { ARCHEAD_BF16 = 1, ARCHEAD_F32 = 2 } archead_dtype;

typedef enum {
  ARCHEAD_PATH_AUTO = 0,   /* the decode path when it takes the call, else the tile path */
  ARCHEAD_PATH_DECODE = 1, /* one kernel that streams the head once for up to 64 tokens.
                              Up to 16 tokens: the few-token kernel when H (N + 1 rows of D + 8
                              halves) and Z (N (r_c + r_r) fp32) fit 152 KiB of
                              LDS and D/128 is a multiple of 4 (N <= 16 at
                              D = 4096, r <= 128; N <= 8 at D = 8192), else the k-tile-major kernel
                              when the converted H fits the 160 KiB of LDS of a
                              workgroup (N <= 16 at D = 4096, N <= 8 at D = 8192),
                              with N (r_c + r_r) <= 2048, round_up(r_c, 32) +
                              round_up(r_r, 32) <= 256 and D/g <= 128.
                              17 to 64 tokens: the batched kernel (accumulators
                              of all tokens for its vocabulary rows held over
                              the whole hidden dimension) when round_up(r_c, 32)
                              + round_up(r_r, 32) <= 128, D/g <= 64 and D is a
                              multiple of 512 */
  ARCHEAD_PATH_TILE = 2    /* LDS-tiled MFMA path (any N); needs the workspace    */
} archead_path;

/* Storage format of a packed head.  ARCHEAD_FMT_ARCHEAD is the method's own
 * head.  The other two are the storage-matched heads the pages set beside it
 * (results discussion of Table 7: a GPTQ-style INT4 head at 25.78% of the
 * BF16 head; of Table 8: a row-INT8 head at about twice ARCHead's storage);
 * they have no factors (r_c = r_r = 0). */
typedef enum {
  ARCHEAD_FMT_ARCHEAD = 0,    /* SC4 residual + quantised core + INT8 correction        */
  ARCHEAD_FMT_GROUP_INT4 = 1, /* W[v,k] = q4[v,k] * s_G[v, k/g], fp16 group scales       */
  ARCHEAD_FMT_ROW_INT8 = 2    /* W[v,k] = q8[v,k] * s[v], fp16 row scales                */
} archead_format;

/* Shape of a packed head (Algorithm 1 inputs: vocabulary V, hidden size D,
 * core rank r_c, correction rank r_r, group size g along D) and its storage
 * format (archead_format; 0 when the struct is zero-initialised). */
typedef struct {
  int64_t V, D;
  int32_t r_c, r_r, g;
  int32_t format;
} archead_dims;

typedef struct {
  uint64_t offset, bytes;
} archead_span;

/* Where every stored tensor lives inside the one contiguous packed buffer
 * (format version 1; each section starts on a 256-byte boundary):
 *   header      64 B: u32 magic 0x48435241, u32 version, u64 V, u64 D,
 *                      u32 r_c, u32 r_r, u32 g, u32 flags (the format), 24 zero bytes
 *   r_codes     SC4 codes in tiles of 16 rows x 128 columns (1024 B).  With
 *               V16 = V rounded up to 16 and nb = V16/16 row blocks, tile
 *               (b, kt) sits at (kt*nb + b)*1024 (k-tile major, so tiles read
 *               at the same time by neighbouring waves are adjacent); byte 16*l + 4*s + c
 *               (l < 64, s < 4, c < 4) holds row 16*b + l%16 at columns
 *               k = 128*kt + 32*s + 8*(l/16) + 2*c (low nibble) and k+1 (high
 *               nibble), two's complement.  Rows >= V are zero.
 *   r_gcodes    uint8 group codes [V16][D/g], row-major: byte v*(D/g) + t is row v, group t.
 *   r_rowscale  fp16 per-row residual scale s_R [V16].
 *   a_codes     int8 [V16][r_c + r_r], row v = A_c[v,:] then A_w[v,:].
 *   a_scales    fp16 [V16][n_A], n_A = (r_c>0) + (r_r>0): s_Ac[v] then s_Aw[v].
 *   b_codes     int8 [r_c + r_r][D], rows B_c then B_w.
 *   b_scales    fp16 [r_c + r_r][D/g], group scales of B_c then B_w.
 * Dequantisation: R[v,k] = q4 * c8[v,k/g] * s_R[v];  A[v,j] = code * s_A(part)[v];
 * B[j,k] = code * s_B[j,k/g].  W_hat = R + A_c B_c + A_w B_w.
 * The header's flags word holds the format.  The comparison heads use the
 * same container with r_c = r_r = 0 (sections not named are empty):
 *   ARCHEAD_FMT_GROUP_INT4: r_codes as above; r_gcodes holds fp16 group
 *     scales [V16][D/g] (byte 2*(v*(D/g) + t)).  W_hat[v,k] = q4 * s_G[v,k/g].
 *   ARCHEAD_FMT_ROW_INT8: r_codes holds INT8 tiles of 16 rows x 128 columns
 *     (2048 B), tile (b, kt) at (kt*nb + b)*2048; byte 32*l + 8*s + p holds
 *     row 16*b + l%16 at column 128*kt + 32*s + 8*(l/16) + P[p],
 *     P = {0,1,4,5,2,3,6,7}; r_rowscale holds fp16 s[v].  W_hat[v,k] = q8 * s[v].
 * payload_bytes is the sum of numel x element size over the seven stored
 * tensors (the persistent size of Sec. 3); total_bytes adds the header and
 * alignment padding. */
typedef struct {
  uint32_t format_version, alignment;
  uint64_t total_bytes, payload_bytes, header_bytes;
  archead_span header, r_codes, r_gcodes, r_rowscale, a_codes, a_scales, b_codes, b_scales;
  int64_t padded_rows; /* V16 */
} archead_layout;

/* Host-side components of one head, one code per element, row-major.  fp16
 * values are passed as their uint16 bit patterns.  Pointers for a part of rank
 * 0 may be NULL.
 *   q4   [V][D]   int8 in [-8, 7]      c8   [V][D/g] uint8     s_R  [V] fp16
 *   A_c  [V][r_c] int8   A_w [V][r_r] int8   s_Ac [V] fp16   s_Aw [V] fp16
 *   B_c  [r_c][D] int8   B_w [r_r][D] int8   s_Bc [r_c][D/g] fp16   s_Bw [r_r][D/g] fp16 */
typedef struct {
  const int8_t* q4;
  const uint8_t* c8;
  const uint16_t* s_R;
  const int8_t* A_c;
  const int8_t* A_w;
  const uint16_t* s_Ac;
  const uint16_t* s_Aw;
  const int8_t* B_c;
  const int8_t* B_w;
  const uint16_t* s_Bc;
  const uint16_t* s_Bw;
  /* comparison heads: ARCHEAD_FMT_GROUP_INT4 reads q4 and s_G [V][D/g] fp16;
   * ARCHEAD_FMT_ROW_INT8 reads q8 [V][D] int8 in [-127, 127] and s_R as the
   * row scales.  Unused fields may be NULL. */
  const uint16_t* s_G;
  const int8_t* q8;
} archead_host_components;

/* A 2-D device tensor: element (i, j) at data + (i*row_stride + j)*elem_size. */
typedef struct {
  void* data;
  int64_t rows, cols, row_stride; /* row_stride in elements, >= cols */
  int32_t dtype;                  /* archead_dtype */
} archead_tensor;

/* A packed head resident in device memory, plus the caller's device workspace. */
typedef struct {
  archead_dims dims;
  const void* buffer;       /* device, 256-byte aligned, laid out per archead_pack_layout */
  uint64_t buffer_bytes;    /* >= layout.total_bytes */
  void* workspace;          /* device, 256-byte aligned scratch for one call */
  uint64_t workspace_bytes; /* >= archead_workspace_bytes(dims, N) */
} archead_packed_head;

/* Layout of the packed buffer for `d`.  Pure host arithmetic: no allocation,
 * no HIP call.  E_NULL, E_DIMS. */
ARCHEAD_API int archead_pack_layout(const archead_dims* d, archead_layout* out);

/* Device workspace one archead_logits call with n_tokens rows of H needs on
 * the automatic path: when the few-token decode kernel takes the call, H
 * converted to fp16 (n_tokens D halves), its per-token scales and Z
 * (n_tokens (r_c + r_r) fp32), each section rounded up to 256 bytes; when the
 * k-tile-major decode kernel takes it, the partial sums of the
 * pre-projection (n_tokens (r_c + r_r) zst fp32, zst = ceil(D / 1024)
 * rounded up to a multiple of 4; 0 when r_c + r_r = 0, and the workspace
 * pointer may then be NULL); on the tile path the converted hidden states,
 * the low-rank pre-projection, per-token scales and 64 MiB for partial sums
 * of output tiles whose hidden dimension is split over several workgroups.
 * Pure host arithmetic.  E_NULL, E_DIMS, E_SHAPE (n_tokens < 0). */
ARCHEAD_API int archead_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes);

/* Same for a call with the path chosen by the caller (archead_path):
 * ARCHEAD_PATH_TILE always needs the tile path's workspace.  E_NULL, E_DIMS,
 * E_SHAPE, E_UNSUPPORTED (unknown path). */
ARCHEAD_API int archead_workspace_bytes_path(const archead_dims* d, int64_t n_tokens, int path, uint64_t* bytes);

/* The main kernel a successful archead_logits_path call of n_tokens rows
 * launches (after its pre-projection kernel):
 *   ARCHEAD_KERNEL_TILE           tile32_kernel, the LDS-tiled MFMA path
 *   ARCHEAD_KERNEL_DECODE_FEW     small_decode_kernel: up to 16 tokens whose
 *                                 fp16 rows and Z fit in 152 KiB of LDS (N <= 16
 *                                 at D = 4096, r <= 128; D a multiple of 512)
 *   ARCHEAD_KERNEL_DECODE_STREAM  decode_kernel: the k-tile-major streaming
 *                                 kernel for the other calls of up to 16 tokens
 *   ARCHEAD_KERNEL_DECODE_BATCH   batch_kernel: the batched streaming kernel
 *                                 for 17 to 64 tokens (r_c, r_r rounded up to
 *                                 32 sum to at most 128, D/g <= 64, D a
 *                                 multiple of 512)
 * Host only; lets a caller or profiler name the kernel it times.  E_NULL,
 * E_DIMS, E_SHAPE, E_UNSUPPORTED (unknown path, or a forced decode path the
 * call cannot take). */
enum archead_kernel {
  ARCHEAD_KERNEL_TILE = 0,
  ARCHEAD_KERNEL_DECODE_FEW = 1,
  ARCHEAD_KERNEL_DECODE_STREAM = 2,
  ARCHEAD_KERNEL_DECODE_BATCH = 3
};
ARCHEAD_API int archead_main_kernel(const archead_dims* d, int64_t n_tokens, int path, int* kernel);

/* Serialise host components into `dst` (host memory, dst_bytes >=
 * layout.total_bytes), writing every byte of the layout including padding,
 * in the format d->format names.  Host only; multithreaded.  E_NULL, E_DIMS,
 * E_SIZE, E_VALUE (an INT4 code outside [-8, 7], an INT8 code of -128). */
ARCHEAD_API int archead_pack(const archead_dims* d, const archead_host_components* src, void* dst,
                 uint64_t dst_bytes);

/* Dense inputs of the packing step (Algorithm 1 and the Sec. 3 quantized-core
 * sentence): the head W and the factor matrices, all device memory, row-major.
 *   W    [V][D]   bf16 or fp32 (W_dtype), row stride W_stride elements; W and
 *                 every row 16-byte aligned
 *   A_c  [V][r_c] fp32, B_c [r_c][D] fp32   the low-rank core (e.g. a truncated SVD of W)
 *   A_w  [V][r_r] fp32, B_w [r_r][D] fp32   the activation-metric correction
 * Factors of a part of rank 0 may be NULL. */
typedef struct {
  const void* W;
  int64_t W_stride;
  int32_t W_dtype; /* archead_dtype */
  const float* A_c;
  const float* B_c;
  const float* A_w;
  const float* B_w;
} archead_dense_head;

/* Quantise a dense head into a packed buffer on the GPU (the packing step of
 * Algorithm 1; ARCHead Sec. 3, quantized-core equation and packed-variant
 * paragraph).  The pages fix no rounding rule or scale formula; this uses
 * symmetric absmax scaling with round half to even, every decision in fp32:
 *   INT8 (rows of A_c and A_w; g-column groups of the rows of B_c and B_w):
 *     s = fp16(amax / 127), code = clamp(rint(x / s), -127, 127), 0 where s = 0;
 *   R = W - Q(A_c) Q(B_c), accumulated in fp64 over the core rank in index
 *     order and rounded once to fp32;
 *   SC4 of R (g-column groups t of row v, m_t = the group's amax):
 *     s_R = fp16(max_t m_t / 1785), c8_t = clamp(ceil(m_t / (7 s_R)), 1, 255),
 *     q4 = clamp(rint(R / (c8_t s_R)), -8, 7); a zero row gives s_R = c8 = q4 = 0.
 * packed: device, 256-byte aligned, packed_bytes >= archead_layout.total_bytes;
 *   every byte of the layout is written (padding rows and gaps are zero).
 * E: optional fp32 [V][D] device tensor (NULL: not written), rows 16-byte
 *   aligned; receives fp32(R) - SC4(R), the error left after the residual
 *   codes (what the correction A_w B_w is meant to absorb).
 * Enqueued on `stream` without synchronising; allocates nothing.
 * E_NULL, E_DIMS, E_UNSUPPORTED (g not in {32, 64, 128, 256}, D > 8192,
 * r_c > 1024, r_r > 65536), E_DTYPE, E_SHAPE, E_ALIGN, E_SIZE, E_HIP. */
ARCHEAD_API int archead_quantize(const archead_dims* d, const archead_dense_head* src, void* packed,
                                 uint64_t packed_bytes, archead_tensor* E, void* stream);

/* Inputs of the whole construction (Algorithm 1; Sec. 3), device memory:
 *   W        [V][D] bf16 or fp32 (W_dtype), row stride W_stride elements,
 *            4-byte aligned: the dense head
 *   H        [H_rows][D] bf16, row stride H_stride: calibration hidden states
 *   omega_c  fp32 row-major [D][r_c + oversample], omega_r [D][r_r + oversample]:
 *            the Gaussian test matrices of the two randomized SVDs (NULL for
 *            a part of rank 0)
 *   p, lambda   metric power and damping (lambda > 0)
 *   oversample  extra columns of the randomized SVDs; power_iters <= 16 rounds
 *               of power iteration. */
typedef struct {
  const void* W;
  int64_t W_stride;
  int32_t W_dtype;
  const void* H;
  int64_t H_rows, H_stride;
  const float* omega_c;
  const float* omega_r;
  float p, lambda;
  int32_t oversample, power_iters;
} archead_fit_inputs;

/* Optional copies of the fitted fp32 factors (row-major, contiguous) and of
 * the core error E = W - W_d [V][D]; each pointer may be NULL. */
typedef struct {
  float* A_c;
  float* B_c;
  float* A_w;
  float* B_w;
  float* E;
} archead_fit_outputs;

/* Device workspace archead_fit needs (two fp32 V x D arrays, four D x D, the
 * randomized SVDs' panels, 65 chunk products of D x k, small fp64 matrices and
 * the factors; k = max(r_c, r_r) + oversample).  Pure host arithmetic.
 * E_NULL, E_DIMS, E_SHAPE (k above V or D), E_UNSUPPORTED (k above 128, or
 * what archead_quantize does not take). */
ARCHEAD_API int archead_fit_workspace_bytes(const archead_dims* d, int32_t oversample, uint64_t* bytes);

/* Build a packed head from a dense one (Algorithm 1; Sec. 3 metric transform,
 * quantized-core equation and packed-variant paragraph):
 *   1. A_c B_c = rank-r_c randomized SVD of W (Y = W omega_c, power_iters
 *      rounds of power iteration with an orthonormal basis between them,
 *      Q = orth(Y), Q^T W = U S V^T, A_c = Q U_r S_r, B_c = V_r^T);
 *   2. the packing step of archead_quantize for the core: INT8 A_c, B_c, SC4 of
 *      R = W - Q(A_c) Q(B_c), and E = W - W_d;
 *   3. C_lam = H^T H / H_rows + lambda c_bar I (c_bar = mean diagonal of
 *      H^T H / H_rows), C_lam = Q Lam Q^T, T_p = Q Lam^p Q^T, T_p^{-1};
 *   4. A_w Bt = rank-r_r randomized SVD of E T_p (omega_r), B_w = Bt T_p^{-1};
 *   5. INT8 A_w (rows) and B_w (groups) into the same buffer.
 * Dense products run on rocBLAS in fp32 (E T_p is never formed: the
 * randomized SVD applies E and T_p in turn), orthonormal bases by Cholesky QR
 * twice with fp64 Gram matrices, the SVD of the k x D sketch from the fp64
 * eigenpairs of its Gram matrix, the eigendecomposition of C_lam on rocSOLVER
 * (fp32).  Step 3 runs on a second stream (default priority) created for the
 * call, beside steps 1-2; two rocBLAS handles are created for the call
 * (rocBLAS may allocate its own scratch).  k = max(r_c, r_r) + oversample
 * must be at most 128.  The call waits for both streams at the end to read
 * the solvers' status: ARCHEAD_E_VALUE if one failed or a Cholesky pivot was
 * not finite (or for a lambda that is not positive, or a non-finite p).
 * packed: as for archead_quantize.  E_NULL, E_DIMS, E_UNSUPPORTED, E_DTYPE,
 * E_SHAPE, E_ALIGN, E_SIZE, E_WORKSPACE, E_VALUE, E_HIP. */
ARCHEAD_API int archead_fit(const archead_dims* d, const archead_fit_inputs* in, void* packed,
                            uint64_t packed_bytes, void* workspace, uint64_t workspace_bytes,
                            const archead_fit_outputs* out, void* stream);

/* Device workspace archead_logit_error needs for n_tokens rows: the
 * forward's workspace for min(n_tokens, 256) rows rounded up to 256, two
 * fp32 blocks of min(n_tokens, 256) x V logits (each rounded up to 256),
 * 16 KiB of partial sums and 256 bytes (0 when n_tokens = 0).  Pure host
 * arithmetic.  E_NULL, E_DIMS, E_SHAPE. */
ARCHEAD_API int archead_logit_error_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes);

/* The logit error of a packed head against the dense head W it replaces, on
 * the N rows of H (ARCHead, Sec. 3, Eq. 1 before its 1/N):
 *   sums[0] = sum_{n,v} (H W^T - H W_hat^T)[n, v]^2,  sums[1] = sum_{n,v} (H W^T)[n, v]^2,
 * in fp64 from fp32 logits (host array of 2 doubles).  W: bf16 [V][D] device
 * tensor.  The packed logits come from the forward, the dense ones from a
 * rocBLAS bf16 product with fp32 accumulation, 256 tokens at a time in the
 * workspace (at least archead_logit_error_workspace_bytes).  Waits for the
 * stream.  H and head as for archead_logits.  E_NULL, E_DTYPE, E_SHAPE,
 * E_UNSUPPORTED, E_ALIGN, E_WORKSPACE, E_HIP. */
ARCHEAD_API int archead_logit_error(const archead_tensor* H, const archead_packed_head* head,
                                    const archead_tensor* W, double* sums, void* stream);

/* Y = H W_hat^T  (Algorithm 1, inference step).
 *   H: bf16 [N][D] device tensor; rows 16-byte aligned.
 *   Y: fp32 or bf16 [N][V] device tensor, written completely (every element
 *      once); bf16 output is rounded to nearest even from the fp32 result.
 *   stream: a hipStream_t (NULL = the default stream).
 * Enqueues the decode path (up to 64 tokens: a small pre-projection kernel,
 * then one kernel that streams the head) or the tile path (pre-projection
 * kernels, then the tile kernel) on `stream` and returns without
 * synchronising.  A comparison head (ARCHEAD_FMT_GROUP_INT4, _ROW_INT8) runs
 * on the batched streaming kernel only, 32 tokens per launch (the tile path
 * gives E_UNSUPPORTED); it needs D a multiple of 512 and D/g <= 64.
 * N = 0 is a no-op that returns ARCHEAD_OK.  Faults inside kernels surface at
 * the caller's next synchronisation with the stream. */
ARCHEAD_API int archead_logits(const archead_tensor* H, const archead_packed_head* head, archead_tensor* Y,
                   void* stream);

/* Y = H W_hat^T exactly as archead_logits (automatic path), for callers that
 * cannot allocate device memory or call hipMalloc (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * workspace comes from an array of ARCHEAD_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends; head->workspace
 * and head->workspace_bytes are ignored.  Calls whose workspace (without the
 * optional split-tile partial sums, which get whatever is left) exceeds it
 * give E_WORKSPACE before anything is enqueued: at D = 4096, r_c = r_r = 64
 * that is past about 1790 tokens (930 at D = 8192).  Allocates nothing and calls no allocating
 * routine; the first call on a device looks the array's address up.  Every
 * call on one GPU uses the same array and nothing in it needs to start at
 * zero: calls that overlap on one GPU (other streams, other threads) race and
 * give undefined results.  ARCHead-format heads only (E_UNSUPPORTED for a
 * comparison head).  Other arguments and errors as archead_logits. */
#define ARCHEAD_NOALLOC_SCRATCH_BYTES (16ull << 20)
ARCHEAD_API int archead_logits_noalloc(const archead_tensor* H, const archead_packed_head* head,
                                       archead_tensor* Y, void* stream);

/* Same as archead_logits with the path chosen by the caller (archead_path).
 * ARCHEAD_PATH_DECODE gives E_UNSUPPORTED for a call the decode kernel does
 * not take; ARCHEAD_PATH_TILE needs archead_workspace_bytes_path(.., TILE).
 * A decode-path call (automatic or forced) whose N rows of Y span 4 GiB or
 * more gives E_UNSUPPORTED (that kernel stores through 32-bit offsets).
 * Both paths compute the same Y up to fp32 summation order. */
ARCHEAD_API int archead_logits_path(const archead_tensor* H, const archead_packed_head* head,
                        archead_tensor* Y, int path, void* stream);

/* Same as archead_logits_path, and has the caller's events ev_begin and
 * ev_end (hipEvent_t handles, either may be NULL) record the start of the
 * main kernel (decode or tile, after either path's pre-projection kernels)
 * and the end of the forward's last kernel (the main kernel, or the tile
 * path's reduce kernel of split tiles; for a comparison head, from the first
 * to the last of its launches).  The launches themselves record them (AMD's
 * launch with start and stop events), so no marker is added to `stream` and
 * the span is the kernels' own.  For timing the dominant kernel on the stream
 * it runs on. */
ARCHEAD_API int archead_logits_events(const archead_tensor* H, const archead_packed_head* head,
                                      archead_tensor* Y, int path, void* stream, void* ev_begin,
                                      void* ev_end);

/* Per-row statistics of Y = H W_hat^T (the fp32 logits archead_logits
 * computes), without writing Y: what the pages' quality metrics are built
 * from (ARCHead, Abstract: perplexity and cross-entropy; results discussion
 * of Table 8: top-1 agreement).  Each output is a device array of N elements,
 * 4-byte aligned, or NULL (not written):
 *   row_max[n]    = max_v Y[n, v]                          fp32
 *   row_argmax[n] = the lowest v with Y[n, v] = row_max[n]  int32
 *   row_lse[n]    = log sum_v exp(Y[n, v])                  fp32
 *   row_ce[n]     = row_lse[n] - Y[n, targets[n]]           fp32; NaN where
 *                   targets[n] is outside [0, V); needs targets
 *   targets       = device int32 [N], or NULL when row_ce is NULL. */
typedef struct {
  float* row_max;
  int32_t* row_argmax;
  float* row_lse;
  float* row_ce;
  const int32_t* targets;
} archead_row_stats;

/* Device workspace one archead_logits_stats call with n_tokens rows needs:
 * archead_workspace_bytes plus 16 bytes per token and statistics piece
 * (max(64, ceil(V16 / 256)) pieces), plus Y in fp32 when n_tokens <= 16.
 * Pure host arithmetic.  E_NULL, E_DIMS. */
ARCHEAD_API int archead_stats_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes);

/* Enqueue the statistics of `out` for the N rows of H on `stream`; the same
 * argument rules as archead_logits for H and head (the workspace must hold
 * archead_stats_workspace_bytes).  The tile path reduces each 256-row
 * vocabulary tile of every token in its epilogue and never writes Y; up to
 * 16 tokens whose H and Z fit LDS run the decode kernel into the workspace
 * first.  Shapes neither path takes (section offsets past 32 bits) give
 * E_UNSUPPORTED.  E_NULL also when row_ce is set without targets. */
ARCHEAD_API int archead_logits_stats(const archead_tensor* H, const archead_packed_head* head,
                                     const archead_row_stats* out, void* stream);

/* Device workspace one archead_logits_topk call with n_tokens rows needs:
 * archead_workspace_bytes for min(n_tokens, 256) rows, rounded up to 256,
 * plus min(n_tokens, 256) x V fp32 logits rounded up to 256, plus twice
 * min(n_tokens, 256) x ceil(V / 4096) x 256 bytes rounded up to 256 of
 * first-stage candidates (0 when n_tokens = 0).  Pure host arithmetic.
 * E_NULL, E_DIMS, E_SHAPE. */
ARCHEAD_API int archead_topk_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes);

/* The k largest logits of each row of Y = H W_hat^T and their vocabulary
 * indices, what top-k agreement is measured on (ARCHead, results discussion
 * of Table 8: top-1/5/10).  Row n gets top_val[n*k + i] (fp32) and
 * top_idx[n*k + i] (int32) for i < k, largest value first; among equal values
 * the lower index comes first, so the result is unique.  Device arrays of
 * N*k elements, 4-byte aligned.  The forward runs on `stream` in chunks of
 * 256 tokens into fp32 logits held in the workspace (the logits are read back
 * once, not returned); the selection takes the k best of every 1024-element
 * span of a row, then the k best of those candidates.  1 <= k <= 16 (E_SHAPE below 1 or above V,
 * E_UNSUPPORTED above 16); H and head as for archead_logits, the workspace
 * at least archead_topk_workspace_bytes.  N = 0 is a no-op. */
ARCHEAD_API int archead_logits_topk(const archead_tensor* H, const archead_packed_head* head, int32_t k,
                                    float* top_val, int32_t* top_idx, void* stream);

/* Static string naming a status code. */
ARCHEAD_API const char* archead_status_string(int status);

/* ARCHEAD_FORMAT_VERSION the library was built for. */
ARCHEAD_API int archead_format_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ARCHEAD_H */
