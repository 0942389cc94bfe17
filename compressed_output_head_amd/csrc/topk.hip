// The k largest logits of every row of Y = H W_hat^T with their vocabulary
// indices: the quantity behind the pages' top-k agreement figures (ARCHead,
// results discussion of Table 8: top-1/5/10).  The forward runs in chunks of
// tokens into fp32 logits held in the caller's workspace; the selection then
// takes the k best of every 1024-element span of a row (one wave each) and
// the k best of those candidates (one workgroup per row).  Order:
// larger value first, and among equal values the lower index first, so the
// result is unique.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "archead.h"

namespace {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkMax = 16;             // largest k
constexpr int64_t kTkChunkRows = 256;  // tokens per forward chunk
constexpr int kTkPer = 16;                              // first stage: elements per lane
constexpr int64_t kTkWaveSpan = 64 * kTkPer;            // elements per wave
constexpr int64_t kTkPiece = kTkWaves * kTkWaveSpan;    // elements per first-stage workgroup

constexpr uint64_t up256(uint64_t x) { return (x + 255) / 256 * 256; }

// a before b: larger value, then lower index
__device__ __forceinline__ bool tk_before(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Insert (x, xi) into a thread's sorted list of the K best so far.
template <int K>
__device__ __forceinline__ void tk_insert(float (&val)[K], int (&idx)[K], float x, int xi) {
  if (!tk_before(x, xi, val[K - 1], idx[K - 1])) return;
  val[K - 1] = x;
  idx[K - 1] = xi;
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

// k rounds over the workgroup's 256 sorted lists: each round the best head
// wins, is written to ov[r], oi[r] and is popped by its owner (an index sits
// in one list only).
template <int K>
__device__ __forceinline__ void tk_select(float (&val)[K], int (&idx)[K], int k, float* ov, int32_t* oi) {
  __shared__ float sv[kTkWaves];
  __shared__ int si[kTkWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r = 0; r < k; ++r) {
    float bv = val[0];
    int bi = idx[0];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float xv = __shfl_xor(bv, off);
      const int xi = __shfl_xor(bi, off);
      if (tk_before(xv, xi, bv, bi)) {
        bv = xv;
        bi = xi;
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
      ov[r] = bv;
      oi[r] = bi;
    }
    if (idx[0] == bi) {
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

template <int K>
__device__ __forceinline__ void tk_clear(float (&val)[K], int (&idx)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) {
    val[i] = -INFINITY;
    idx[i] = INT32_MAX;
  }
}

// Stage 1: wave w of workgroup (p, row) takes the kTkWaveSpan elements of
// one row of Y [rows][V] from (p waves + w) kTkWaveSpan on, kTkPer per lane
// (64 apart, all loads in flight together), and writes its k best to
// cand[((row P + p) waves + w) k + r]: k rounds of a shuffle reduction over
// the lanes' best remaining element; the winner's lane marks it taken.
// Elements past V never win (index INT32_MAX); with fewer than k elements the
// remaining outputs are (-inf, INT32_MAX) and lose every merge.
__global__ __launch_bounds__(kTkThreads) void topk_piece_kernel(const float* Y, int64_t V, int k, float* cv,
                                                                int32_t* ci) {
  const int P = gridDim.x, p = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.y;
  const float* y = Y + row * V;
  const int64_t base = ((int64_t)p * kTkWaves + wave) * kTkWaveSpan + lane;
  float x[kTkPer];
#pragma unroll
  for (int e = 0; e < kTkPer; ++e) {
    const int64_t v = base + 64 * e;
    x[e] = v < V ? y[v] : -INFINITY;
  }
  uint32_t taken = 0u;
  const int64_t o = ((row * P + p) * kTkWaves + wave) * k;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = INT32_MAX;
#pragma unroll
    for (int e = 0; e < kTkPer; ++e) {
      const int64_t v = base + 64 * e;
      const int vi = v < V ? (int)v : INT32_MAX;
      if (!((taken >> e) & 1u) && tk_before(x[e], vi, bv, bi)) {
        bv = x[e];
        bi = vi;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float xv = __shfl_xor(bv, off);
      const int xi = __shfl_xor(bi, off);
      if (tk_before(xv, xi, bv, bi)) {
        bv = xv;
        bi = xi;
      }
    }
    if (lane == 0) {
      cv[o + r] = bv;
      ci[o + r] = bi;
    }
    if (bi != INT32_MAX && (bi - base) % 64 == 0 && bi >= base) taken |= 1u << (int)((bi - base) / 64);
  }
}

// Stage 2: one workgroup per row merges the row's n = P waves k candidates.
template <int K>
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(const float* cv, const int32_t* ci, int n, int k,
                                                                float* out_val, int32_t* out_idx, int64_t out_ld) {
  const int64_t row = blockIdx.x;
  float val[K];
  int idx[K];
  tk_clear(val, idx);
  for (int c = threadIdx.x; c < n; c += kTkThreads) tk_insert(val, idx, cv[row * n + c], ci[row * n + c]);
  tk_select(val, idx, k, out_val + row * out_ld, out_idx + row * out_ld);
}

int64_t tk_pieces(int64_t V) { return (V + kTkPiece - 1) / kTkPiece; }

// candidate bytes of the first stage for a chunk of `rows` rows
uint64_t tk_cand_bytes(int64_t rows, int64_t V) {
  return up256((uint64_t)rows * (uint64_t)tk_pieces(V) * kTkWaves * kTkMax * 4) * 2;
}

template <int K>
hipError_t launch_topk_k(const float* Y, int64_t rows, int64_t V, int k, float* cv, int32_t* ci, float* out_val,
                         int32_t* out_idx, int64_t out_ld, hipStream_t s) {
  const int P = (int)tk_pieces(V);
  hipLaunchKernelGGL(topk_piece_kernel, dim3((unsigned)P, (unsigned)rows), dim3(kTkThreads), 0, s, Y, V, k, cv, ci);
  hipLaunchKernelGGL((topk_merge_kernel<K>), dim3((unsigned)rows), dim3(kTkThreads), 0, s, cv, ci,
                     P * kTkWaves * k, k, out_val, out_idx, out_ld);
  return hipGetLastError();
}

hipError_t launch_topk(const float* Y, int64_t rows, int64_t V, int k, float* cv, int32_t* ci, float* out_val,
                       int32_t* out_idx, int64_t out_ld, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return k <= 4 ? launch_topk_k<4>(Y, rows, V, k, cv, ci, out_val, out_idx, out_ld, s)
                : launch_topk_k<kTkMax>(Y, rows, V, k, cv, ci, out_val, out_idx, out_ld, s);
}

int topk_layout(const archead_dims* d, int64_t n_tokens, uint64_t* fwd_bytes, uint64_t* total) {
  const int64_t rows = n_tokens < kTkChunkRows ? n_tokens : kTkChunkRows;
  int rc = archead_workspace_bytes(d, rows, fwd_bytes);
  if (rc) return rc;
  *fwd_bytes = up256(*fwd_bytes);
  *total = rows > 0 ? *fwd_bytes + up256((uint64_t)rows * (uint64_t)d->V * 4) + tk_cand_bytes(rows, d->V) : 0;
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
  const uint64_t ybytes = up256((uint64_t)(N < kTkChunkRows ? N : kTkChunkRows) * (uint64_t)d->V * 4);
  const int64_t crow = N < kTkChunkRows ? N : kTkChunkRows;
  float* cv = reinterpret_cast<float*>(static_cast<uint8_t*>(head->workspace) + fwd + ybytes);
  int32_t* ci = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(head->workspace) + fwd + ybytes +
                                           tk_cand_bytes(crow, d->V) / 2);
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
    if (launch_topk(Yc, rows, d->V, k, cv, ci, top_val + t0 * k, top_idx + t0 * k, k, s) != hipSuccess)
      return ARCHEAD_E_HIP;
  }
  return ARCHEAD_OK;
}

}  // extern "C"
