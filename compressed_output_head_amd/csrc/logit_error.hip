// Logit error of a packed head against the dense head it replaces, the
// quantity of Eq. 1 (ARCHead, Sec. 3): sum over tokens n and vocabulary v of
// (H W^T - H W_hat^T)[n, v]^2, with the reference energy sum (H W^T)^2.  Per
// chunk of 256 tokens the packed logits come from the forward and the dense
// ones from a rocBLAS bf16 product (fp32 accumulation), both fp32 in the
// workspace; a reduction kernel sums the squares in fp64 per workgroup and a
// second one adds the workgroups' partial sums in a fixed order.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include "archead.h"

namespace {

constexpr int kLeThreads = 256;
constexpr int kLeBlocks = 1024;         // partial sums per chunk
constexpr int64_t kLeChunkRows = 256;   // tokens per chunk

constexpr uint64_t up256(uint64_t x) { return (x + 255) / 256 * 256; }

// part[b] = (sum (yd - yp)^2, sum yd^2) over a grid-strided share of n elements
__global__ __launch_bounds__(kLeThreads) void sq_partial_kernel(const float* yd, const float* yp, int64_t n,
                                                                double* part) {
  __shared__ double s0[kLeThreads], s1[kLeThreads];
  double a = 0.0, b = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * kLeThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kLeThreads) {
    const double d = (double)yd[i] - (double)yp[i];
    a += d * d;
    b += (double)yd[i] * (double)yd[i];
  }
  s0[threadIdx.x] = a;
  s1[threadIdx.x] = b;
  __syncthreads();
  for (int w = kLeThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s0[threadIdx.x] += s0[threadIdx.x + w];
      s1[threadIdx.x] += s1[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = s0[0];
    part[2 * blockIdx.x + 1] = s1[0];
  }
}

// acc += sum of the nb partial pairs (one workgroup; acc is zeroed when first)
__global__ __launch_bounds__(kLeThreads) void sq_total_kernel(const double* part, int nb, double* acc, int first) {
  __shared__ double s0[kLeThreads], s1[kLeThreads];
  double a = 0.0, b = 0.0;
  for (int i = threadIdx.x; i < nb; i += kLeThreads) {
    a += part[2 * i];
    b += part[2 * i + 1];
  }
  s0[threadIdx.x] = a;
  s1[threadIdx.x] = b;
  __syncthreads();
  for (int w = kLeThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s0[threadIdx.x] += s0[threadIdx.x + w];
      s1[threadIdx.x] += s1[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    acc[0] = (first ? 0.0 : acc[0]) + s0[0];
    acc[1] = (first ? 0.0 : acc[1]) + s1[0];
  }
}

int le_layout(const archead_dims* d, int64_t n_tokens, uint64_t* fwd, uint64_t* ybytes, uint64_t* total) {
  const int64_t rows = n_tokens < kLeChunkRows ? n_tokens : kLeChunkRows;
  int rc = archead_workspace_bytes(d, rows, fwd);
  if (rc) return rc;
  *fwd = up256(*fwd);
  *ybytes = up256((uint64_t)rows * (uint64_t)d->V * 4);
  *total = rows > 0 ? *fwd + 2 * *ybytes + up256(kLeBlocks * 16) + 256 : 0;
  return ARCHEAD_OK;
}

}  // namespace

extern "C" {

int archead_logit_error_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes) {
  if (!d || !bytes) return ARCHEAD_E_NULL;
  if (n_tokens < 0) return ARCHEAD_E_SHAPE;
  uint64_t fwd = 0, yb = 0;
  return le_layout(d, n_tokens, &fwd, &yb, bytes);
}

int archead_logit_error(const archead_tensor* H, const archead_packed_head* head, const archead_tensor* W,
                        double* sums, void* stream) {
  if (!H || !head || !W || !sums) return ARCHEAD_E_NULL;
  const archead_dims* d = &head->dims;
  const int64_t N = H->rows;
  if (N < 0) return ARCHEAD_E_SHAPE;
  uint64_t fwd = 0, yb = 0, need = 0;
  int rc = le_layout(d, N, &fwd, &yb, &need);
  if (rc) return rc;
  if (W->dtype != ARCHEAD_BF16 || H->dtype != ARCHEAD_BF16) return ARCHEAD_E_DTYPE;
  if (W->rows != d->V || W->cols != d->D || W->row_stride < d->D) return ARCHEAD_E_SHAPE;
  if (d->V > INT32_MAX || W->row_stride > INT32_MAX || H->row_stride > INT32_MAX) return ARCHEAD_E_UNSUPPORTED;
  if (N == 0) {
    sums[0] = sums[1] = 0.0;
    return ARCHEAD_OK;
  }
  if (!W->data || !head->workspace) return ARCHEAD_E_NULL;
  if (reinterpret_cast<uintptr_t>(W->data) % 2) return ARCHEAD_E_ALIGN;
  if (reinterpret_cast<uintptr_t>(head->workspace) % ARCHEAD_ALIGNMENT) return ARCHEAD_E_ALIGN;
  if (head->workspace_bytes < need) return ARCHEAD_E_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(head->workspace);
  float* Yp = reinterpret_cast<float*>(ws + fwd);
  float* Yd = reinterpret_cast<float*>(ws + fwd + yb);
  double* part = reinterpret_cast<double*>(ws + fwd + 2 * yb);
  double* acc = reinterpret_cast<double*>(ws + fwd + 2 * yb + up256(kLeBlocks * 16));
  hipStream_t s = static_cast<hipStream_t>(stream);
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return ARCHEAD_E_HIP;
  rc = ARCHEAD_OK;
  if (rocblas_set_stream(h, s) != rocblas_status_success ||
      rocblas_set_pointer_mode(h, rocblas_pointer_mode_host) != rocblas_status_success)
    rc = ARCHEAD_E_HIP;
  const float one = 1.0f, zero = 0.0f;
  for (int64_t t0 = 0; t0 < N && rc == ARCHEAD_OK; t0 += kLeChunkRows) {
    const int64_t rows = N - t0 < kLeChunkRows ? N - t0 : kLeChunkRows;
    archead_tensor Hc = *H;
    Hc.rows = rows;
    if (H->data) Hc.data = static_cast<uint8_t*>(H->data) + (uint64_t)t0 * (uint64_t)H->row_stride * 2;
    archead_packed_head P = *head;
    P.workspace_bytes = fwd;
    archead_tensor Yt{Yp, rows, d->V, d->V, ARCHEAD_F32};
    rc = archead_logits(&Hc, &P, &Yt, stream);  // validates H and the head
    if (rc) break;
    // dense logits, row-major [rows][V] = column-major W H^T (V x rows)
    if (rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, (int)d->V, (int)rows, (int)d->D, &one,
                        W->data, rocblas_datatype_bf16_r, (int)W->row_stride, Hc.data, rocblas_datatype_bf16_r,
                        (int)H->row_stride, &zero, Yd, rocblas_datatype_f32_r, (int)d->V, Yd, rocblas_datatype_f32_r,
                        (int)d->V, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success) {
      rc = ARCHEAD_E_HIP;
      break;
    }
    hipLaunchKernelGGL(sq_partial_kernel, dim3(kLeBlocks), dim3(kLeThreads), 0, s, Yd, Yp, rows * d->V, part);
    hipLaunchKernelGGL(sq_total_kernel, dim3(1), dim3(kLeThreads), 0, s, part, kLeBlocks, acc, t0 == 0 ? 1 : 0);
    if (hipGetLastError() != hipSuccess) rc = ARCHEAD_E_HIP;
  }
  if (rc == ARCHEAD_OK && hipMemcpyAsync(sums, acc, 16, hipMemcpyDeviceToHost, s) != hipSuccess) rc = ARCHEAD_E_HIP;
  // the handle's scratch must outlive everything enqueued with it, also after an error
  if (hipStreamSynchronize(s) != hipSuccess && rc == ARCHEAD_OK) rc = ARCHEAD_E_HIP;
  rocblas_destroy_handle(h);
  return rc;
}

}  // extern "C"
