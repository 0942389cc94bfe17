// The construction of a packed head (ARCHead, Algorithm 1 and Sec. 3) on the
// GPU: a rank-r_c core of W by randomized SVD, quantised with the SC4
// residual of what it leaves (the packing kernels), then the correction
// fitted to the core error E = W - W_d in the damped activation metric:
//   C_lam = H^T H / N + lam c_bar I   (c_bar = mean diagonal of H^T H / N),
//   C_lam = Q Lam Q^T,  T_p = Q Lam^p Q^T,  T_p^{-1} = Q Lam^{-p} Q^T,
//   [E T_p]_r = A_w Bt (randomized SVD),  B_w = Bt T_p^{-1},
// and A_w, B_w quantised into the same buffer.  The randomized SVD of an
// M [V x D]: Y = M Omega, q rounds of power iteration with an orthonormal
// basis between them, Q = orth(Y), Q^T M = U S V^T, A = Q U_r S_r, B = V_r^T.
//
// How it runs (fp32 data, fp64 where a small matrix is factorised):
//   - M = E T_p is never formed: the randomized SVD only needs M X = E (T_p X),
//     M^T Y = T_p^T (E^T Y) and Q^T M = (Q^T E) T_p, which are thin products;
//   - products with a reduction over the V rows (E^T Y, Q^T E) are split
//     over row chunks (strided-batched rocBLAS) and the chunk sums added in a
//     fixed order, so they fill the GPU instead of a handful of tiles;
//   - orth() is CholeskyQR2: the Gram matrix of the panel in fp64, its
//     Cholesky factor R and R^{-1} in one workgroup, the panel times R^{-1},
//     twice (the second pass restores orthogonality to fp32 level);
//     directions whose Cholesky pivot vanishes are dropped (zero columns);
//   - the SVD of the k x D sketch Q^T M comes from the fp64 eigenpairs of its
//     k x k Gram matrix: Q^T M = U S V^T with U S^2 U^T = (Q^T M)(Q^T M)^T and
//     V_r^T = S_r^{-1} U_r^T Q^T M;
//   - the covariance, its eigendecomposition (rocSOLVER) and T_p, T_p^{-1}
//     depend on H only and run on a second stream beside the core's
//     randomized SVD and packing; the correction waits for both.
//
// rocBLAS and rocSOLVER are column-major: a row-major [R][C] array with row
// stride ld is the column-major C x R matrix (its transpose) with leading
// dimension ld, which is how every row-major array below is passed.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>
#include <stdint.h>

#include <cmath>
#include <utility>

#include "archead.h"
#include "device_common.h"
#include "quantize.h"

namespace {

using archead::QuantArgs;

constexpr int kFThreads = 256;
constexpr int kFitMaxK = 128;      // rank + oversample of either randomized SVD
constexpr int kSplit = 64;         // row chunks of a reduction over V rows
constexpr int kGramChunks = 256;   // row chunks of a Gram matrix
constexpr int kGramRows = 32;      // rows per LDS tile of the Gram kernel
constexpr int kTri = kFitMaxK * (kFitMaxK + 1) / 2;
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

// dst[:, j] = src[:, j] * max(s[j], tiny)^p for column-major n_rows x n_cols
// (ld = n_rows); one workgroup per column at a time, the power once per thread
__global__ __launch_bounds__(kFThreads) void scale_cols_kernel(const float* src, float* dst, int64_t n_rows,
                                                               int64_t n_cols, int64_t ld, const float* s, float p) {
  for (int64_t j = blockIdx.x; j < n_cols; j += gridDim.x) {
    const float f = powf(fmaxf(s[j], 1e-30f), p);
    for (int64_t r = threadIdx.x; r < n_rows; r += kFThreads) dst[j * ld + r] = src[j * ld + r] * f;
  }
}

// out = sum over S chunk products P_i (each D x k column-major, contiguous),
// added in chunk order; out column-major D x k, or its transpose k x D (out_t)
__global__ __launch_bounds__(kFThreads) void sum_parts_kernel(const float* part, int S, int64_t D, int k, float* out,
                                                              bool out_t) {
  const int64_t n = D * k, stride = (int64_t)gridDim.x * kFThreads;
  for (int64_t e = (int64_t)blockIdx.x * kFThreads + threadIdx.x; e < n; e += stride) {
    float acc = 0.0f;
    for (int i = 0; i < S; ++i) acc += part[(int64_t)i * n + e];
    const int64_t d = e % D, j = e / D;
    out[out_t ? j + (int64_t)k * d : e] = acc;
  }
}

// Partial Gram matrices in fp64 of the m x k panel X (element (i, j) at
// X[i*rs + j*cs]): part[c][a*k + b] = sum over the rows of chunk c of
// X[i,a] X[i,b].  Grid (chunks, ceil(k*k/256)): one entry per thread.  Each
// product of two fp32 values is exact in fp64.
__global__ __launch_bounds__(kFThreads) void gram_kernel(const float* X, int64_t rs, int64_t cs, int64_t m, int k,
                                                         int64_t rows_per_chunk, double* part) {
  __shared__ float tile[kGramRows * kFitMaxK];
  const int e = (int)blockIdx.y * kFThreads + (int)threadIdx.x;
  const bool live = e < k * k;
  const int a = live ? e / k : 0, b = live ? e - a * k : 0;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < m ? r0 + rows_per_chunk : m;
  double acc = 0.0;
  for (int64_t t0 = r0; t0 < r1; t0 += kGramRows) {
    const int64_t nr = r1 - t0 < kGramRows ? r1 - t0 : kGramRows;
    __syncthreads();
    for (int idx = threadIdx.x; idx < kGramRows * k; idx += kFThreads) {
      const int i = idx % kGramRows, j = idx / kGramRows;
      tile[i * k + j] = i < nr ? X[(t0 + i) * rs + (int64_t)j * cs] : 0.0f;
    }
    __syncthreads();
    if (live)
      for (int i = 0; i < kGramRows; ++i) acc += (double)tile[i * k + a] * (double)tile[i * k + b];
  }
  if (live) part[(int64_t)blockIdx.x * k * k + e] = acc;
}

// G[e] = sum over chunks of part[c][e], in chunk order
__global__ __launch_bounds__(kFThreads) void gram_reduce_kernel(const double* part, int chunks, int k, double* G) {
  const int e = (int)blockIdx.x * kFThreads + (int)threadIdx.x;
  if (e >= k * k) return;
  double acc = 0.0;
  for (int c = 0; c < chunks; ++c) acc += part[(int64_t)c * k * k + e];
  G[e] = acc;
}

__device__ __forceinline__ int tri(int i, int l) { return l * (l + 1) / 2 + i; }  // (i, l), i <= l

// One workgroup: the Cholesky factor G = R^T R (R upper) of the k x k Gram
// matrix and Rinv = R^{-1} (fp32, column-major, ld k).  A pivot that is not
// positive or below 1e-14 of its original diagonal drops its direction (row
// and column of R^{-1} zero); a non-finite pivot sets *info.
__global__ __launch_bounds__(kFThreads) void chol_inv_kernel(const double* G, int k, float* Rinv, int* info) {
  __shared__ double R[kTri], X[kTri];
  __shared__ int drop[kFitMaxK];
  __shared__ double piv;
  const int tid = threadIdx.x;
  for (int e = tid; e < k * k; e += kFThreads) {
    const int i = e / k, l = e - i * k;
    if (i <= l) R[tri(i, l)] = G[e];
  }
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    if (tid == 0) {
      const double d = R[tri(j, j)];
      const double g = G[j * k + j];
      if (!std::isfinite(d) || !std::isfinite(g)) *info = 1;
      const bool ok = std::isfinite(d) && d > 0.0 && d > 1e-14 * g;
      drop[j] = !ok;
      piv = ok ? sqrt(d) : 0.0;
    }
    __syncthreads();
    const bool dj = drop[j];
    const double pj = piv;
    for (int l = j + tid; l < k; l += kFThreads) R[tri(j, l)] = dj ? 0.0 : (l == j ? pj : R[tri(j, l)] / pj);
    __syncthreads();
    const int w = k - j - 1;
    if (!dj)
      for (int idx = tid; idx < w * w; idx += kFThreads) {
        const int i = j + 1 + idx / w, l = j + 1 + idx % w;
        if (i <= l) R[tri(i, l)] -= R[tri(j, i)] * R[tri(j, l)];
      }
    __syncthreads();
  }
  // rows of X = R^{-1} from the last up: X[i][l] = (delta_il - sum_{t>i} R[i][t] X[t][l]) / R[i][i]
  for (int i = k - 1; i >= 0; --i) {
    for (int l = i + tid; l < k; l += kFThreads) {
      double v = 0.0;
      if (!drop[i]) {
        double s = l == i ? 1.0 : 0.0;
        for (int t = i + 1; t <= l; ++t) s -= R[tri(i, t)] * X[tri(t, l)];
        v = s / R[tri(i, i)];
      }
      X[tri(i, l)] = v;
    }
    __syncthreads();
  }
  for (int e = tid; e < k * k; e += kFThreads) {
    const int l = e / k, i = e - l * k;  // column-major: (i, l) at i + l*k
    Rinv[e] = i <= l ? (float)X[tri(i, l)] : 0.0f;
  }
}

// From the ascending fp64 eigenpairs (column-major vectors, ld k) of the
// sketch's Gram matrix: US[:, i] = u_i s_i and UinvS[:, i] = u_i / s_i for
// the r largest (s_i = sqrt(lambda_i)); components with s_i <= 1e-6 s_max are
// zero in both.
__global__ __launch_bounds__(kFThreads) void svd_factors_kernel(const double* vec, const double* lam, int k, int r,
                                                                float* US, float* UinvS) {
  const double smax = sqrt(fmax(lam[k - 1], 0.0));
  for (int e = threadIdx.x; e < k * r; e += kFThreads) {
    const int i = e / k, a = e - i * k;
    const int src = k - 1 - i;
    const double s = sqrt(fmax(lam[src], 0.0));
    const bool keep = smax > 0.0 && s > 1e-6 * smax;
    const double u = vec[(int64_t)src * k + a];
    US[e] = keep ? (float)(u * s) : 0.0f;
    UinvS[e] = keep ? (float)(u / s) : 0.0f;
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
  float *Y, *Y2;        // V x k panels (column-major, ld V)
  float *Z, *Z2, *X;    // D x k panels (column-major, ld D)
  float *Bm, *Bm2;      // k x D sketches (column-major, ld k)
  float *part;          // (kSplit + 1) chunk products of D x k
  double *gpart, *G;    // Gram partials and the Gram matrix (k x k)
  double *lam, *ework;  // eigenvalues and rocSOLVER's off-diagonal scratch (k)
  float *Rinv, *US, *UinvS;
  int* info;  // device ints: [0] the Gram eigensolver, [1] a non-finite Cholesky pivot
};

// The operator of a randomized SVD: M = E, or M = E T (T column-major D x D).
struct Op {
  const float* E;
  int64_t ld;  // row stride of the row-major E [V][D]
  const float* T;
};

const float kOne = 1.0f, kZero = 0.0f;

// out = E^T Y (column-major D x k) or its transpose (k x D, out_t) with Y
// column-major V x k (ld V): chunk products over row ranges of E, then their
// sum in chunk order.
void tall_tn(Status& st, rocblas_handle h, hipStream_t s, const float* E, int64_t ld, int V, int D, const float* Y,
             int k, float* part, float* out, bool out_t) {
  const int c = V / kSplit;
  int S = 0;
  if (c > 0) {
    if (!st.ok(rocblas_sgemm_strided_batched(h, rocblas_operation_none, rocblas_operation_none, D, k, c, &kOne, E,
                                             (int)ld, (rocblas_stride)c * ld, Y, V, (rocblas_stride)c, &kZero, part,
                                             D, (rocblas_stride)D * k, kSplit)))
      return;
    S = kSplit;
  }
  const int rem = V - S * c;
  if (rem > 0) {
    if (!st.ok(rocblas_sgemm(h, rocblas_operation_none, rocblas_operation_none, D, k, rem, &kOne,
                             E + (int64_t)S * c * ld, (int)ld, Y + (int64_t)S * c, V, &kZero,
                             part + (int64_t)S * D * k, D)))
      return;
    ++S;
  }
  hipLaunchKernelGGL(sum_parts_kernel, dim3(grid_for((int64_t)D * k)), dim3(kFThreads), 0, s, part, S, (int64_t)D,
                     k, out, out_t);
  st.ok(hipGetLastError());
}

// Y (column-major V x k) = M X; X column-major D x k (ld D), or the row-major
// D x k test matrix (x_rowmajor, ld k).
void op_apply(Status& st, rocblas_handle h, const Op& M, int V, int D, int k, const float* X, bool x_rowmajor,
              float* tmp, float* Y) {
  const rocblas_operation ox = x_rowmajor ? rocblas_operation_transpose : rocblas_operation_none;
  const int ldx = x_rowmajor ? k : D;
  if (M.T) {  // tmp = T X
    if (!st.ok(rocblas_sgemm(h, rocblas_operation_none, ox, D, k, D, &kOne, M.T, D, X, ldx, &kZero, tmp, D))) return;
    X = tmp;
  }
  st.ok(rocblas_sgemm(h, rocblas_operation_transpose, M.T ? rocblas_operation_none : ox, V, k, D, &kOne, M.E,
                      (int)M.ld, X, M.T ? D : ldx, &kZero, Y, V));
}

// Z (column-major D x k) = M^T Y
void op_apply_t(Status& st, rocblas_handle h, hipStream_t s, const Op& M, int V, int D, int k, const float* Y,
                const RsvdBufs& b, float* tmp, float* Z) {
  tall_tn(st, h, s, M.E, M.ld, V, D, Y, k, b.part, M.T ? tmp : Z, false);
  if (M.T && !st.rc)
    st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, D, k, D, &kOne, M.T, D, tmp, D,
                        &kZero, Z, D));
}

// Gram matrix b.G (fp64 k x k) of the m x k panel X (element (i, j) at X[i*rs + j*cs])
void gram(Status& st, hipStream_t s, const float* X, int64_t rs, int64_t cs, int64_t m, int k, const RsvdBufs& b) {
  const int64_t per = (m + kGramChunks - 1) / kGramChunks;
  const int chunks = (int)((m + per - 1) / per);
  hipLaunchKernelGGL(gram_kernel, dim3((unsigned)chunks, (unsigned)((k * k + kFThreads - 1) / kFThreads)),
                     dim3(kFThreads), 0, s, X, rs, cs, m, k, per, b.gpart);
  if (!st.ok(hipGetLastError())) return;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3((unsigned)((k * k + kFThreads - 1) / kFThreads)), dim3(kFThreads), 0,
                     s, b.gpart, chunks, k, b.G);
  st.ok(hipGetLastError());
}

// An orthonormal basis of the column-major m x k panel P (ld m) by
// CholeskyQR2; P and P2 swap so that P holds the result.
void orth(Status& st, rocblas_handle h, hipStream_t s, float*& P, float*& P2, int m, int k, const RsvdBufs& b) {
  for (int pass = 0; pass < 2 && !st.rc; ++pass) {
    gram(st, s, P, 1, m, m, k, b);
    if (st.rc) return;
    hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(kFThreads), 0, s, b.G, k, b.Rinv, b.info + 1);
    if (!st.ok(hipGetLastError())) return;
    if (!st.ok(rocblas_sgemm(h, rocblas_operation_none, rocblas_operation_none, m, k, k, &kOne, P, m, b.Rinv, k,
                             &kZero, P2, m)))
      return;
    std::swap(P, P2);
  }
}

// Randomized rank-r SVD of M [V][D] with the row-major test matrix omega
// [D][k]: A row-major [V][r], B row-major [r][D].
void rsvd(Status& st, rocblas_handle h, hipStream_t s, const Op& M, int V, int D, int r, int k, const float* omega,
          int q, RsvdBufs b, float* A, float* B) {
  op_apply(st, h, M, V, D, k, omega, true, b.X, b.Y);  // Y = M Omega
  for (int it = 0; it < q && !st.rc; ++it) {
    orth(st, h, s, b.Y, b.Y2, V, k, b);
    if (st.rc) return;
    op_apply_t(st, h, s, M, V, D, k, b.Y, b, b.X, b.Z);  // Z = M^T Y
    orth(st, h, s, b.Z, b.Z2, D, k, b);
    if (st.rc) return;
    op_apply(st, h, M, V, D, k, b.Z, false, b.X, b.Y);  // Y = M Z
  }
  if (st.rc) return;
  orth(st, h, s, b.Y, b.Y2, V, k, b);
  if (st.rc) return;
  // Bm (k x D) = Q^T M = (Q^T E) T
  tall_tn(st, h, s, M.E, M.ld, V, D, b.Y, k, b.part, M.T ? b.Bm2 : b.Bm, true);
  if (st.rc) return;
  if (M.T && !st.ok(rocblas_sgemm(h, rocblas_operation_none, rocblas_operation_none, k, D, D, &kOne, b.Bm2, k, M.T,
                                  D, &kZero, b.Bm, k)))
    return;
  // Bm = U S V^T from the eigenpairs of Bm Bm^T (the panel Bm^T: D rows, element (d, j) at Bm[j + k d])
  gram(st, s, b.Bm, k, 1, D, k, b);
  if (st.rc) return;
  if (!st.ok(rocsolver_dsyevd(h, rocblas_evect_original, rocblas_fill_upper, k, b.G, k, b.lam, b.ework, b.info)))
    return;
  hipLaunchKernelGGL(svd_factors_kernel, dim3(1), dim3(kFThreads), 0, s, b.G, b.lam, k, r, b.US, b.UinvS);
  if (!st.ok(hipGetLastError())) return;
  // A^T (r x V) = (U S)_r^T Q^T;  B^T (D x r) = Bm^T (U S^{-1})_r
  if (!st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_transpose, r, V, k, &kOne, b.US, k, b.Y,
                           V, &kZero, A, r)))
    return;
  st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, D, r, k, &kOne, b.Bm, k, b.UinvS, k,
                      &kZero, B, D));
}

// Byte offsets of the fit's workspace (every piece 256-byte aligned).
struct FitLayout {
  uint64_t Wf, E, Y, Y2, Z, Z2, X, Bm, Bm2, part, gpart, G, lam, ework, Rinv, US, UinvS, info, C, Lam, work, M1, Tp,
      Ti, A_c, B_c, A_w, Bt, B_w, total;
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
  L.Y2 = take(V * k * 4);
  L.Z = take(D * k * 4);
  L.Z2 = take(D * k * 4);
  L.X = take(D * k * 4);
  L.Bm = take(k * D * 4);
  L.Bm2 = take(k * D * 4);
  L.part = take((uint64_t)(kSplit + 1) * D * k * 4);
  L.gpart = take((uint64_t)kGramChunks * k * k * 8);
  L.G = take(k * k * 8);
  L.lam = take(k * 8);
  L.ework = take(k * 8);
  L.Rinv = take(k * k * 4);
  L.US = take(k * k * 4);
  L.UinvS = take(k * k * 4);
  L.info = take(16 * sizeof(rocblas_int));
  L.C = take(D * D * 4);
  L.Lam = take(D * 4);
  L.work = take(D * 4);
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
  if (kmax > kFitMaxK) return ARCHEAD_E_UNSUPPORTED;  // the small factorisations run in one workgroup's LDS
  return ARCHEAD_OK;
}

// Resources of one call that must be released on every path.
struct FitRes {
  rocblas_handle h = nullptr, h2 = nullptr;
  hipStream_t s2 = nullptr;
  hipEvent_t e_in = nullptr, e_cov = nullptr;
  ~FitRes() {
    // rocSOLVER's scratch belongs to the handles: nothing may still run on
    // their streams when they are destroyed
    if (s2) (void)hipStreamSynchronize(s2);
    if (h2) rocblas_destroy_handle(h2);
    if (h) rocblas_destroy_handle(h);
    if (e_in) (void)hipEventDestroy(e_in);
    if (e_cov) (void)hipEventDestroy(e_cov);
    if (s2) (void)hipStreamDestroy(s2);
  }
};

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
  auto F64 = [&](uint64_t off) { return reinterpret_cast<double*>(ws + off); };
  rocblas_int* info = reinterpret_cast<rocblas_int*>(ws + FL.info);
  // info: [0, 1] the core's randomized SVD, [2, 3] the correction's, [4] the covariance eigensolver
  RsvdBufs b{F(FL.Y),     F(FL.Y2),     F(FL.Z),    F(FL.Z2),      F(FL.X),     F(FL.Bm),   F(FL.Bm2),
             F(FL.part),  F64(FL.gpart), F64(FL.G), F64(FL.lam),   F64(FL.ework), F(FL.Rinv), F(FL.US),
             F(FL.UinvS), info};
  hipStream_t s = static_cast<hipStream_t>(stream);
  Status st;
  {
    FitRes res;
    if (!st.ok(hipStreamCreateWithFlags(&res.s2, hipStreamNonBlocking)) ||
        !st.ok(hipEventCreateWithFlags(&res.e_in, hipEventDisableTiming)) ||
        !st.ok(hipEventCreateWithFlags(&res.e_cov, hipEventDisableTiming)))
      return st.rc;
    if (rocblas_create_handle(&res.h) != rocblas_status_success ||
        rocblas_create_handle(&res.h2) != rocblas_status_success)
      return ARCHEAD_E_HIP;
    rocblas_handle h = res.h, h2 = res.h2;
    hipStream_t s2 = res.s2;
    do {
      if (!st.ok(rocblas_set_stream(h, s)) || !st.ok(rocblas_set_pointer_mode(h, rocblas_pointer_mode_host)) ||
          !st.ok(rocblas_set_stream(h2, s2)) || !st.ok(rocblas_set_pointer_mode(h2, rocblas_pointer_mode_host)))
        break;
      if (!st.ok(hipMemsetAsync(info, 0, 16 * sizeof(rocblas_int), s))) break;
      // the second stream starts after the caller's work and the status reset
      if (!st.ok(hipEventRecord(res.e_in, s)) || !st.ok(hipStreamWaitEvent(s2, res.e_in, 0))) break;
      if (r_r > 0) {
        // second stream: C_lam = H^T H / N + lam c_bar I (bf16 inputs, fp32
        // products and sums), C_lam = Q Lam Q^T, T_p and T_p^{-1}
        const float invN = 1.0f / (float)N;
        if (!st.ok(rocblas_gemm_ex(h2, rocblas_operation_none, rocblas_operation_transpose, D, D, N, &invN, in->H,
                                   rocblas_datatype_bf16_r, (int)in->H_stride, in->H, rocblas_datatype_bf16_r,
                                   (int)in->H_stride, &kZero, F(FL.C), rocblas_datatype_f32_r, D, F(FL.C),
                                   rocblas_datatype_f32_r, D, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                                   0)))
          break;
        hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(kFThreads), 0, s2, F(FL.C), D, in->lambda);
        if (!st.ok(hipGetLastError())) break;
        // eigenvectors overwrite C
        if (!st.ok(rocsolver_ssyevd(h2, rocblas_evect_original, rocblas_fill_upper, D, F(FL.C), D, F(FL.Lam),
                                    F(FL.work), info + 4)))
          break;
        // T_p = (Q Lam^p) Q^T and T_p^{-1} = (Q Lam^{-p}) Q^T
        const float pw[2] = {in->p, -in->p};
        const uint64_t dst[2] = {FL.Tp, FL.Ti};
        for (int t = 0; t < 2 && !st.rc; ++t) {
          hipLaunchKernelGGL(scale_cols_kernel, dim3((unsigned)(D < 8192 ? D : 8192)), dim3(kFThreads), 0, s2, F(FL.C),
                             F(FL.M1), (int64_t)D, (int64_t)D, (int64_t)D, F(FL.Lam), pw[t]);
          if (!st.ok(hipGetLastError())) break;
          st.ok(rocblas_sgemm(h2, rocblas_operation_none, rocblas_operation_transpose, D, D, D, &kOne, F(FL.M1), D,
                              F(FL.C), D, &kZero, F(dst[t]), D));
        }
        if (st.rc) break;
      }
      if (!st.ok(hipEventRecord(res.e_cov, s2))) break;
      // first stream: W as contiguous fp32, the core's randomized SVD, the packing step for the core
      hipLaunchKernelGGL(to_f32_kernel, dim3(grid_for((int64_t)V * D)), dim3(kFThreads), 0, s, in->W,
                         in->W_stride, in->W_dtype == ARCHEAD_BF16, (int64_t)V, (int64_t)D, F(FL.Wf));
      if (!st.ok(hipGetLastError())) break;
      if (r_c > 0) {
        rsvd(st, h, s, Op{F(FL.Wf), D, nullptr}, V, D, r_c, k_c, in->omega_c, q, b, F(FL.A_c), F(FL.B_c));
        if (st.rc) break;
      }
      const QuantArgs qa = archead::quant_args(d, PL, packed, F(FL.Wf), D, false, F(FL.E), D);
      if (!st.ok(archead::launch_quantize_core(qa, F(FL.A_c), F(FL.B_c), PL.total_bytes, s))) break;
      if (!st.ok(hipStreamWaitEvent(s, res.e_cov, 0))) break;
      if (r_r > 0) {
        // the correction: randomized SVD of E T_p (never formed), B_w = Bt T_p^{-1}
        RsvdBufs br = b;
        br.info = info + 2;
        rsvd(st, h, s, Op{F(FL.E), D, F(FL.Tp)}, V, D, r_r, k_r, in->omega_r, q, br, F(FL.A_w), F(FL.Bt));
        if (st.rc) break;
        // column-major B_w^T (D x r_r) = T_p^{-T} Bt^T
        if (!st.ok(rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, D, r_r, D, &kOne,
                                 F(FL.Ti), D, F(FL.Bt), D, &kZero, F(FL.B_w), D)))
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
      rocblas_int hinfo[16];
      if (!st.ok(hipMemcpyAsync(hinfo, info, sizeof(hinfo), hipMemcpyDeviceToHost, s)) ||
          !st.ok(hipStreamSynchronize(s)))
        break;
      for (int i = 0; i < 16; ++i)
        if (hinfo[i] != 0 && st.rc == ARCHEAD_OK) st.rc = ARCHEAD_E_VALUE;
    } while (false);
    // an error can leave work enqueued on either stream
    if (hipStreamSynchronize(s) != hipSuccess && st.rc == ARCHEAD_OK) st.rc = ARCHEAD_E_HIP;
    if (hipStreamSynchronize(s2) != hipSuccess && st.rc == ARCHEAD_OK) st.rc = ARCHEAD_E_HIP;
  }
  return st.rc;
}

}  // extern "C"
