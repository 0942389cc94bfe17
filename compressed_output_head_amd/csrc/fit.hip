// The construction of a packed head (ARCHead, Algorithm 1 and Sec. 3) on the
// GPU: a rank-r_c core of W by randomized SVD, quantised with the SC4
// residual of what it leaves (the packing kernels), then the correction
// fitted to the core error E = W - W_d in the damped activation metric:
//   C_lam = H^T H / N + lam c_bar I   (c_bar = mean diagonal of H^T H / N),
//   C_lam = Q Lam Q^T,  T_p = Q Lam^p Q^T,  T_p^{-1} = Q Lam^{-p} Q^T,
//   [E T_p]_r = A_w Bt (randomized SVD),  B_w = Bt T_p^{-1},
// and A_w, B_w quantised into the same buffer.  The randomized SVD of an
// M [V x D]: Y = M Omega, q rounds of power iteration with QR between them,
// Q = qr(Y), Q^T M = U S V^T, A = Q U_r S_r, B = V_r^T.  Dense products run
// on rocBLAS, QR / SVD / the symmetric eigendecomposition on rocSOLVER, in
// fp32; the conversions, damping and scalings are the kernels below.
//
// rocBLAS and rocSOLVER are column-major: a row-major [R][C] array with row
// stride ld is the column-major C x R matrix (its transpose) with leading
// dimension ld, which is how every row-major array below is passed.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>
#include <stdint.h>

#include <cmath>

#include "archead.h"
#include "device_common.h"
#include "quantize.h"

namespace {

using archead::QuantArgs;

constexpr int kFThreads = 256;
constexpr uint64_t up256(uint64_t x) { return (x + 255) / 256 * 256; }

// dst [rows][cols] fp32 contiguous from a bf16 or fp32 row-major source
__global__ __launch_bounds__(kFThreads) void to_f32_kernel(const void* src, int64_t ld, bool bf16, int64_t rows,
                                                           int64_t cols, float* dst) {
  const int64_t n = rows * cols, stride = (int64_t)gridDim.x * kFThreads;
  for (int64_t i = (int64_t)blockIdx.x * kFThreads + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / cols, c = i - r * cols;
    dst[i] = bf16 ? archead::bf16_to_f32(static_cast<const uint16_t*>(src)[r * ld + c])
                  : static_cast<const float*>(src)[r * ld + c];
  }
}

// C [n x n] += lam * mean(diag C) * I   (one workgroup)
__global__ __launch_bounds__(kFThreads) void damp_kernel(float* C, int n, float lam) {
  __shared__ double part[kFThreads];
  double acc = 0.0;
  for (int i = threadIdx.x; i < n; i += kFThreads) acc += (double)C[(int64_t)i * n + i];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kFThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const float add = (float)((double)lam * part[0] / n);
  for (int i = threadIdx.x; i < n; i += kFThreads) C[(int64_t)i * n + i] += add;
}

// dst[:, j] = src[:, j] * f(s[j]) for column-major n_rows x n_cols (ld = n_rows);
// f(x) = x^p with x clamped below at tiny (mode 0) or f(x) = x (mode 1)
__global__ __launch_bounds__(kFThreads) void scale_cols_kernel(const float* src, float* dst, int64_t n_rows,
                                                               int64_t n_cols, int64_t ld, const float* s, float p,
                                                               int mode) {
  const int64_t n = n_rows * n_cols, stride = (int64_t)gridDim.x * kFThreads;
  for (int64_t i = (int64_t)blockIdx.x * kFThreads + threadIdx.x; i < n; i += stride) {
    const int64_t j = i / n_rows, r = i - j * n_rows;
    const float x = s[j];
    const float f = mode == 1 ? x : powf(fmaxf(x, 1e-30f), p);
    dst[j * ld + r] = src[j * ld + r] * f;
  }
}

// dst row-major [r][D] from the first r rows of a column-major k x D array (ld k)
__global__ __launch_bounds__(kFThreads) void rows_from_colmajor_kernel(const float* src, int64_t k, int64_t r,
                                                                       int64_t D, float* dst) {
  const int64_t n = r * D, stride = (int64_t)gridDim.x * kFThreads;
  for (int64_t i = (int64_t)blockIdx.x * kFThreads + threadIdx.x; i < n; i += stride) {
    const int64_t j = i / D, d = i - j * D;
    dst[i] = src[d * k + j];
  }
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + kFThreads - 1) / kFThreads;
  return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

struct Status {
  int rc = ARCHEAD_OK;
  bool ok(rocblas_status st) {
    if (st != rocblas_status_success && rc == ARCHEAD_OK) rc = ARCHEAD_E_HIP;
    return rc == ARCHEAD_OK;
  }
  bool ok(hipError_t e) {
    if (e != hipSuccess && rc == ARCHEAD_OK) rc = ARCHEAD_E_HIP;
    return rc == ARCHEAD_OK;
  }
};

// Scratch of one randomized SVD (k = rank + oversampling columns).
struct RsvdBufs {
  float *Y, *Z, *tau, *Bm, *S, *U, *Vt, *work;
  rocblas_int* info;  // the SVD's status (a device int)
};

// Randomized rank-r SVD of the row-major M [V][D] (row stride ldm) with the
// row-major test matrix omega [D][k]: A row-major [V][r], B row-major [r][D].
void rsvd(Status& st, rocblas_handle h, hipStream_t s, const float* M, int64_t ldm, int V, int D, int r, int k,
          const float* omega, int q, const RsvdBufs& b, float* A, float* B) {
  const float one = 1.0f, zero = 0.0f;
  // Y (col-major V x k) = M Omega
  if (!st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_transpose, V, k, D, &one, M, (int)ldm,
                           omega, k, &zero, b.Y, V)))
    return;
  for (int it = 0; it < q; ++it) {
    if (!st.ok(rocsolver_sgeqrf(h, V, k, b.Y, V, b.tau)) || !st.ok(rocsolver_sorgqr(h, V, k, k, b.Y, V, b.tau)))
      return;
    // Z (D x k) = M^T Y
    if (!st.ok(rocblas_sgemm(h, rocblas_operation_none, rocblas_operation_none, D, k, V, &one, M, (int)ldm, b.Y, V,
                             &zero, b.Z, D)))
      return;
    if (!st.ok(rocsolver_sgeqrf(h, D, k, b.Z, D, b.tau)) || !st.ok(rocsolver_sorgqr(h, D, k, k, b.Z, D, b.tau)))
      return;
    // Y = M Z
    if (!st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, V, k, D, &one, M, (int)ldm, b.Z,
                             D, &zero, b.Y, V)))
      return;
  }
  if (!st.ok(rocsolver_sgeqrf(h, V, k, b.Y, V, b.tau)) || !st.ok(rocsolver_sorgqr(h, V, k, k, b.Y, V, b.tau)))
    return;
  // Bm (k x D) = Q^T M
  if (!st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_transpose, k, D, V, &one, b.Y, V, M,
                           (int)ldm, &zero, b.Bm, k)))
    return;
  if (!st.ok(rocsolver_sgesvd(h, rocblas_svect_singular, rocblas_svect_singular, k, D, b.Bm, k, b.S, b.U, k, b.Vt, k,
                              b.work, rocblas_outofplace, b.info)))
    return;
  // U[:, :r] *= S[:r]; A^T (r x V) = (U S)_r^T Q^T
  hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for((int64_t)k * r)), dim3(kFThreads), 0, s, b.U, b.U, (int64_t)k,
                     (int64_t)r, (int64_t)k, b.S, 0.0f, 1);
  if (!st.ok(hipGetLastError())) return;
  if (!st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_transpose, r, V, k, &one, b.U, k, b.Y, V,
                           &zero, A, r)))
    return;
  hipLaunchKernelGGL(rows_from_colmajor_kernel, dim3(grid_for((int64_t)r * D)), dim3(kFThreads), 0, s, b.Vt,
                     (int64_t)k, (int64_t)r, (int64_t)D, B);
  st.ok(hipGetLastError());
}

// Byte offsets of the fit's workspace (every piece 256-byte aligned).
struct FitLayout {
  uint64_t Wf, E, Y, Z, tau, Bm, S, U, Vt, work, info, C, Lam, M1, Tp, Ti, A_c, B_c, A_w, Bt, B_w, total;
};

FitLayout fit_layout(const archead_dims* d, int oversample) {
  const uint64_t V = (uint64_t)d->V, D = (uint64_t)d->D;
  const uint64_t k = (uint64_t)((d->r_c > d->r_r ? d->r_c : d->r_r) + oversample);
  FitLayout L{};
  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = o;
    o += up256(bytes);
    return at;
  };
  L.Wf = take(V * D * 4);
  L.E = take(V * D * 4);
  L.Y = take(V * k * 4);
  L.Z = take(D * k * 4);
  L.tau = take(k * 4);
  L.Bm = take(k * D * 4);
  L.S = take(k * 4);
  L.U = take(k * k * 4);
  L.Vt = take(k * D * 4);
  L.work = take((k > D ? k : D) * 4);
  L.info = take(16 * sizeof(rocblas_int));
  L.C = take(D * D * 4);
  L.Lam = take(D * 4);
  L.M1 = take(D * D * 4);
  L.Tp = take(D * D * 4);
  L.Ti = take(D * D * 4);
  L.A_c = take(V * (uint64_t)d->r_c * 4);
  L.B_c = take((uint64_t)d->r_c * D * 4);
  L.A_w = take(V * (uint64_t)d->r_r * 4);
  L.Bt = take((uint64_t)d->r_r * D * 4);
  L.B_w = take((uint64_t)d->r_r * D * 4);
  L.total = o;
  return L;
}

int check_fit(const archead_dims* d, int oversample, archead_layout* L) {
  int rc = archead_pack_layout(d, L);
  if (rc) return rc;
  if (d->format != ARCHEAD_FMT_ARCHEAD) return ARCHEAD_E_UNSUPPORTED;  // the fit writes an ARCHead-format head
  if (d->g != 32 && d->g != 64 && d->g != 128 && d->g != 256) return ARCHEAD_E_UNSUPPORTED;
  if (d->D > archead::kQuantMaxD || d->r_c > archead::kQuantMaxCoreRank) return ARCHEAD_E_UNSUPPORTED;
  if (oversample < 0) return ARCHEAD_E_SHAPE;
  const int64_t kmax = (int64_t)(d->r_c > d->r_r ? d->r_c : d->r_r) + oversample;
  if (kmax > d->V || kmax > d->D || d->V > INT32_MAX / 2) return ARCHEAD_E_SHAPE;
  return ARCHEAD_OK;
}

}  // namespace

extern "C" {

int archead_fit_workspace_bytes(const archead_dims* d, int32_t oversample, uint64_t* bytes) {
  if (!d || !bytes) return ARCHEAD_E_NULL;
  archead_layout L;
  const int rc = check_fit(d, oversample, &L);
  if (rc) return rc;
  *bytes = fit_layout(d, oversample).total;
  return ARCHEAD_OK;
}

int archead_fit(const archead_dims* d, const archead_fit_inputs* in, void* packed, uint64_t packed_bytes,
                void* workspace, uint64_t workspace_bytes, const archead_fit_outputs* out, void* stream) {
  if (!d || !in || !packed || !workspace || !in->W || !in->H) return ARCHEAD_E_NULL;
  archead_layout PL;
  int rc = check_fit(d, in->oversample, &PL);
  if (rc) return rc;
  if ((d->r_c > 0 && !in->omega_c) || (d->r_r > 0 && !in->omega_r)) return ARCHEAD_E_NULL;
  if (in->W_dtype != ARCHEAD_BF16 && in->W_dtype != ARCHEAD_F32) return ARCHEAD_E_DTYPE;
  if (in->W_stride < d->D || in->H_stride < d->D || in->H_rows < 1 || in->H_rows > INT32_MAX) return ARCHEAD_E_SHAPE;
  if (in->power_iters < 0 || in->power_iters > 16) return ARCHEAD_E_SHAPE;
  if (!(in->lambda > 0.0f) || !std::isfinite(in->lambda) || !std::isfinite(in->p)) return ARCHEAD_E_VALUE;
  if ((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(workspace)) % ARCHEAD_ALIGNMENT)
    return ARCHEAD_E_ALIGN;
  if (reinterpret_cast<uintptr_t>(in->H) % 2 || reinterpret_cast<uintptr_t>(in->W) % 4) return ARCHEAD_E_ALIGN;
  if (packed_bytes < PL.total_bytes) return ARCHEAD_E_SIZE;
  const FitLayout FL = fit_layout(d, in->oversample);
  if (workspace_bytes < FL.total) return ARCHEAD_E_WORKSPACE;

  const int V = (int)d->V, D = (int)d->D, r_c = d->r_c, r_r = d->r_r, k_c = r_c + in->oversample,
            k_r = r_r + in->oversample, N = (int)in->H_rows, q = in->power_iters;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  auto F = [&](uint64_t off) { return reinterpret_cast<float*>(ws + off); };
  RsvdBufs b{F(FL.Y), F(FL.Z), F(FL.tau), F(FL.Bm), F(FL.S), F(FL.U), F(FL.Vt), F(FL.work),
             reinterpret_cast<rocblas_int*>(ws + FL.info)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return ARCHEAD_E_HIP;
  Status st;
  const float one = 1.0f, zero = 0.0f;
  st.ok(rocblas_set_stream(h, s)) && st.ok(rocblas_set_pointer_mode(h, rocblas_pointer_mode_host));
  do {
    if (!st.ok(hipMemsetAsync(b.info, 0, 16 * sizeof(rocblas_int), s))) break;
    // W as contiguous fp32
    hipLaunchKernelGGL(to_f32_kernel, dim3(grid_for((int64_t)V * D)), dim3(kFThreads), 0, s, in->W, in->W_stride,
                       in->W_dtype == ARCHEAD_BF16, (int64_t)V, (int64_t)D, F(FL.Wf));
    if (!st.ok(hipGetLastError())) break;
    // the core: rank-r_c randomized SVD of W, quantised with the SC4 residual; E = W - W_d
    if (r_c > 0) {
      rsvd(st, h, s, F(FL.Wf), D, V, D, r_c, k_c, in->omega_c, q, b, F(FL.A_c), F(FL.B_c));
      if (st.rc) break;
    }
    const QuantArgs qa = archead::quant_args(d, PL, packed, F(FL.Wf), D, false, F(FL.E), D);
    if (!st.ok(archead::launch_quantize_core(qa, F(FL.A_c), F(FL.B_c), PL.total_bytes, s))) break;
    if (r_r > 0) {
      // C_lam = H^T H / N + lam c_bar I  (bf16 inputs, fp32 products and sums)
      const float invN = 1.0f / (float)N;
      if (!st.ok(rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_transpose, D, D, N, &invN, in->H,
                                 rocblas_datatype_bf16_r, (int)in->H_stride, in->H, rocblas_datatype_bf16_r,
                                 (int)in->H_stride, &zero, F(FL.C), rocblas_datatype_f32_r, D, F(FL.C),
                                 rocblas_datatype_f32_r, D, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                                 0)))
        break;
      hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(kFThreads), 0, s, F(FL.C), D, in->lambda);
      if (!st.ok(hipGetLastError())) break;
      // C_lam = Q Lam Q^T (eigenvectors overwrite C)
      if (!st.ok(rocsolver_ssyevd(h, rocblas_evect_original, rocblas_fill_upper, D, F(FL.C), D, F(FL.Lam), b.work,
                                  b.info + 2)))
        break;
      // T_p = (Q Lam^p) Q^T and T_p^{-1} = (Q Lam^{-p}) Q^T (symmetric)
      const float pw[2] = {in->p, -in->p};
      const uint64_t dst[2] = {FL.Tp, FL.Ti};
      for (int t = 0; t < 2 && !st.rc; ++t) {
        hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for((int64_t)D * D)), dim3(kFThreads), 0, s, F(FL.C),
                           F(FL.M1), (int64_t)D, (int64_t)D, (int64_t)D, F(FL.Lam), pw[t], 0);
        if (!st.ok(hipGetLastError())) break;
        st.ok(rocblas_sgemm(h, rocblas_operation_none, rocblas_operation_transpose, D, D, D, &one, F(FL.M1), D,
                            F(FL.C), D, &zero, F(dst[t]), D));
      }
      if (st.rc) break;
      // E T_p (row-major [V][D], into the W slot) = column-major T_p^T E^T
      if (!st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, D, V, D, &one, F(FL.Tp), D,
                               F(FL.E), D, &zero, F(FL.Wf), D)))
        break;
      RsvdBufs br = b;
      br.info = b.info + 1;
      rsvd(st, h, s, F(FL.Wf), D, V, D, r_r, k_r, in->omega_r, q, br, F(FL.A_w), F(FL.Bt));
      if (st.rc) break;
      // B_w = Bt T_p^{-1}: column-major B_w^T (D x r_r) = T_p^{-T} Bt^T
      if (!st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, D, r_r, D, &one, F(FL.Ti), D,
                               F(FL.Bt), D, &zero, F(FL.B_w), D)))
        break;
      if (!st.ok(archead::launch_quantize_corr(qa, F(FL.A_w), F(FL.B_w), s))) break;
    }
    if (out) {
      struct {
        float* dst;
        uint64_t off, n;
      } cp[5] = {{out->A_c, FL.A_c, (uint64_t)V * r_c},
                 {out->B_c, FL.B_c, (uint64_t)r_c * D},
                 {out->A_w, FL.A_w, (uint64_t)V * r_r},
                 {out->B_w, FL.B_w, (uint64_t)r_r * D},
                 {out->E, FL.E, (uint64_t)V * D}};
      for (auto& c : cp)
        if (c.dst && c.n && !st.ok(hipMemcpyAsync(c.dst, F(c.off), c.n * 4, hipMemcpyDeviceToDevice, s))) break;
    }
    // the solvers report failures in device ints; wait and read them
    rocblas_int info[16];
    if (!st.ok(hipMemcpyAsync(info, b.info, sizeof(info), hipMemcpyDeviceToHost, s)) ||
        !st.ok(hipStreamSynchronize(s)))
      break;
    for (int i = 0; i < 16; ++i)
      if (info[i] != 0 && st.rc == ARCHEAD_OK) st.rc = ARCHEAD_E_VALUE;
  } while (false);
  // rocSOLVER's scratch belongs to the handle: nothing may still run on the
  // stream when it is destroyed (an error can leave work enqueued)
  if (hipStreamSynchronize(s) != hipSuccess && st.rc == ARCHEAD_OK) st.rc = ARCHEAD_E_HIP;
  rocblas_destroy_handle(h);
  return st.rc;
}

}  // extern "C"
