// The k largest logits of every row of Y = H W_hat^T with their vocabulary
// indices: the quantity behind the pages' top-k agreement figures (ARCHead,
// results discussion of Table 8: top-1/5/10).  The forward runs in chunks of
// tokens into fp32 logits held in the caller's workspace; one workgroup per
// row then selects the k largest.  Order: larger value first, and among equal
// values the lower index first, so the result is unique.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "archead.h"

namespace {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkMax = 16;             // largest k
constexpr int64_t kTkChunkRows = 256;  // tokens per forward chunk

constexpr uint64_t up256(uint64_t x) { return (x + 255) / 256 * 256; }

// a before b: larger value, then lower index
__device__ __forceinline__ bool tk_before(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// One workgroup per row of Y [rows][V] (row stride V).  Each thread keeps the
// K best of the elements it reads (indices tid, tid + 256, ... in increasing
// order, so a later equal value never displaces an earlier one) as a sorted
// register list; then k rounds pick the best head among the 256 lists.
template <int K>
__global__ __launch_bounds__(kTkThreads) void topk_rows_kernel(const float* Y, int64_t V, int k, float* out_val,
                                                               int32_t* out_idx, int64_t out_ld) {
  __shared__ float sv[kTkWaves];
  __shared__ int si[kTkWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* y = Y + row * V;
  float val[K];
  int idx[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    val[i] = -INFINITY;
    idx[i] = INT32_MAX;
  }
  for (int64_t v = tid; v < V; v += kTkThreads) {
    const float x = y[v];
    if (x > val[K - 1] || (idx[K - 1] == INT32_MAX && x == -INFINITY)) {
      val[K - 1] = x;
      idx[K - 1] = (int)v;
#pragma unroll
      for (int i = K - 1; i > 0; --i) {
        if (tk_before(val[i], idx[i], val[i - 1], idx[i - 1])) {
          const float tv = val[i];
          val[i] = val[i - 1];
          val[i - 1] = tv;
          const int ti = idx[i];
          idx[i] = idx[i - 1];
          idx[i - 1] = ti;
        }
      }
    }
  }
  for (int r = 0; r < k; ++r) {
    float bv = val[0];
    int bi = idx[0];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (tk_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      sv[wave] = bv;
      si[wave] = bi;
    }
    __syncthreads();
    bv = sv[0];
    bi = si[0];
#pragma unroll
    for (int w = 1; w < kTkWaves; ++w)
      if (tk_before(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    __syncthreads();  // sv/si are rewritten in the next round
    if (tid == 0) {
      out_val[row * out_ld + r] = bv;
      out_idx[row * out_ld + r] = bi;
    }
    if (idx[0] == bi) {  // the owner of the winning element pops it (indices are unique)
#pragma unroll
      for (int i = 0; i < K - 1; ++i) {
        val[i] = val[i + 1];
        idx[i] = idx[i + 1];
      }
      val[K - 1] = -INFINITY;
      idx[K - 1] = INT32_MAX;
    }
  }
}

hipError_t launch_topk(const float* Y, int64_t rows, int64_t V, int k, float* out_val, int32_t* out_idx,
                       int64_t out_ld, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (k <= 4)
    hipLaunchKernelGGL((topk_rows_kernel<4>), dim3((unsigned)rows), dim3(kTkThreads), 0, s, Y, V, k, out_val,
                       out_idx, out_ld);
  else
    hipLaunchKernelGGL((topk_rows_kernel<kTkMax>), dim3((unsigned)rows), dim3(kTkThreads), 0, s, Y, V, k, out_val,
                       out_idx, out_ld);
  return hipGetLastError();
}

int topk_layout(const archead_dims* d, int64_t n_tokens, uint64_t* fwd_bytes, uint64_t* total) {
  const int64_t rows = n_tokens < kTkChunkRows ? n_tokens : kTkChunkRows;
  int rc = archead_workspace_bytes(d, rows, fwd_bytes);
  if (rc) return rc;
  *fwd_bytes = up256(*fwd_bytes);
  *total = rows > 0 ? *fwd_bytes + up256((uint64_t)rows * (uint64_t)d->V * 4) : 0;
  return ARCHEAD_OK;
}

}  // namespace

extern "C" {

int archead_topk_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes) {
  if (!d || !bytes) return ARCHEAD_E_NULL;
  if (n_tokens < 0) return ARCHEAD_E_SHAPE;
  uint64_t fwd = 0;
  return topk_layout(d, n_tokens, &fwd, bytes);
}

int archead_logits_topk(const archead_tensor* H, const archead_packed_head* head, int32_t k, float* top_val,
                        int32_t* top_idx, void* stream) {
  if (!H || !head) return ARCHEAD_E_NULL;
  const archead_dims* d = &head->dims;
  const int64_t N = H->rows;
  if (N < 0) return ARCHEAD_E_SHAPE;
  uint64_t fwd = 0, need = 0;
  int rc = topk_layout(d, N, &fwd, &need);
  if (rc) return rc;
  if (k < 1 || k > kTkMax) return k < 1 ? ARCHEAD_E_SHAPE : ARCHEAD_E_UNSUPPORTED;
  if (k > d->V) return ARCHEAD_E_SHAPE;
  if (N == 0) return ARCHEAD_OK;
  if (!top_val || !top_idx || !head->workspace) return ARCHEAD_E_NULL;
  if ((reinterpret_cast<uintptr_t>(top_val) | reinterpret_cast<uintptr_t>(top_idx)) % 4) return ARCHEAD_E_ALIGN;
  if (reinterpret_cast<uintptr_t>(head->workspace) % ARCHEAD_ALIGNMENT) return ARCHEAD_E_ALIGN;
  if (head->workspace_bytes < need) return ARCHEAD_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* Yc = reinterpret_cast<float*>(static_cast<uint8_t*>(head->workspace) + fwd);
  for (int64_t t0 = 0; t0 < N; t0 += kTkChunkRows) {
    const int64_t rows = N - t0 < kTkChunkRows ? N - t0 : kTkChunkRows;
    archead_tensor Hc = *H;
    Hc.rows = rows;
    if (H->data) Hc.data = static_cast<uint8_t*>(H->data) + (uint64_t)t0 * (uint64_t)H->row_stride * 2;
    archead_packed_head P = *head;
    P.workspace_bytes = fwd;
    archead_tensor Yt{Yc, rows, d->V, d->V, ARCHEAD_F32};
    rc = archead_logits(&Hc, &P, &Yt, stream);
    if (rc) return rc;
    if (launch_topk(Yc, rows, d->V, k, top_val + t0 * k, top_idx + t0 * k, k, s) != hipSuccess)
      return ARCHEAD_E_HIP;
  }
  return ARCHEAD_OK;
}

}  // extern "C"
