// The k largest logits of every row of Y = H W_hat^T with their vocabulary
// indices: the quantity behind the pages' top-k agreement figures (ARCHead,
// results discussion of Table 8: top-1/5/10).  The forward runs in chunks of
// tokens into fp32 logits held in the caller's workspace; the selection then
// runs in four steps over spans of 1024 elements of a row (one wave each):
//   1. the largest key of every span (one kernel over all spans);
//   2. per row, tau = the k-th largest span key (counting repeats);
//   3. from every span whose largest key is at least tau, its elements with
//      keys >= tau (or its k best, when it has more than k of them);
//   4. the k best of those candidates
// (steps 2-4 in one workgroup per row).
// Step 3 skips no element of the result: k spans have keys >= tau, so the
// row's k-th best key is >= tau, and a span holding any of the k best has a
// largest key >= that one.  Usually only about k of the row's spans qualify
// and only about k elements reach tau, so a row is read about once and a
// handful of candidates is ranked.
//
// Order: larger value first, and among equal values the lower index first,
// so the result is unique.  Values are compared through an order-preserving
// 32-bit key (-0 counts as +0; NaN ranks below -inf); the values returned are
// the stored bits of the chosen elements.  Wave-wide maxima use DPP row
// shifts and broadcasts (a few VALU instructions) instead of LDS shuffles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "archead.h"

namespace {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkMax = 16;             // largest k
constexpr int64_t kTkChunkRows = 256;  // tokens per forward chunk
constexpr int kTkPer = 16;                              // elements per lane of a span
constexpr int64_t kTkWaveSpan = 64 * kTkPer;            // elements per span (one wave)
constexpr int64_t kTkPiece = kTkWaves * kTkWaveSpan;    // elements per workgroup of step 1
constexpr int kTkSpansPerLane = 16;                     // step 2: spans per row <= 1024 (V <= 2^20)
constexpr uint32_t kTkNoIdx = 0x7fffffffu;              // index of padding past V

constexpr uint64_t up256(uint64_t x) { return (x + 255) / 256 * 256; }

// Order-preserving key of a float: larger value, larger key; -0 and +0 share
// one key; every NaN maps to 0, below -inf (0x007fffff).
__device__ __forceinline__ uint32_t tk_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// x = max(x, x of the DPP-selected lane); lanes without a source keep x
template <int ctrl, int row_mask>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t x) {
  const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, ctrl, row_mask, 0xf, false);
  return x > y ? x : y;
}

// Maximum over the 64 lanes (all active), returned to every lane: prefix
// maxima within rows of 16 (row_shr 1, 2, 4, 8), then row 0's into row 1
// and row 2's into row 3 (row_bcast15), then rows 0-1 into rows 2-3
// (row_bcast31); lane 63 ends with the maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = dpp_max_step<0x111, 0xf>(x);
  x = dpp_max_step<0x112, 0xf>(x);
  x = dpp_max_step<0x114, 0xf>(x);
  x = dpp_max_step<0x118, 0xf>(x);
  x = dpp_max_step<0x142, 0xa>(x);
  x = dpp_max_step<0x143, 0xc>(x);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }

// The wave's best (key, index) pair among one offer per lane: the largest
// key, then the lowest index.  Returns the offering lane (the lowest such
// lane if several offer the same pair).
__device__ __forceinline__ int wave_best(uint32_t key, uint32_t idx, uint32_t& bkey, uint32_t& bidx) {
  bkey = wave_max_u32(key);
  bidx = wave_min_u32(key == bkey ? idx : 0xffffffffu);
  const uint64_t m = __ballot(key == bkey && idx == bidx);
  return (int)__builtin_ctzll(m);
}

// (ka, ia) before (kb, ib)
__device__ __forceinline__ bool tk_before(uint32_t ka, uint32_t ia, uint32_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Step 1: wave w of workgroup (p, row) writes the largest key of its span
// (p waves + w) of one row of Y [rows][V] to skey[row n + p waves + w], n =
// spans per row (elements past V count as key 0).
__global__ __launch_bounds__(kTkThreads) void topk_spanmax_kernel(const float* Y, int64_t V, uint32_t* skey) {
  const int P = gridDim.x, p = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.y;
  const float* y = Y + row * V;
  const int64_t base = ((int64_t)p * kTkWaves + wave) * kTkWaveSpan + lane;
  float x[kTkPer];
#pragma unroll
  for (int e = 0; e < kTkPer; ++e) {
    const int64_t v = base + 64 * e;
    x[e] = v < V ? y[v] : __builtin_nanf("");
  }
  uint32_t m = 0u;
#pragma unroll
  for (int e = 0; e < kTkPer; ++e) m = max(m, tk_key(x[e]));
  m = wave_max_u32(m);
  if (lane == 0) skey[row * ((int64_t)P * kTkWaves) + (int64_t)p * kTkWaves + wave] = m;
}

// Insert (key, idx, value) into a lane's list of the K best so far, best first.
template <int K>
__device__ __forceinline__ void tk_insert(uint32_t (&lk)[K], uint32_t (&li)[K], float (&lv)[K], uint32_t key,
                                          uint32_t idx, float v) {
  if (!tk_before(key, idx, lk[K - 1], li[K - 1])) return;
  lk[K - 1] = key;
  li[K - 1] = idx;
  lv[K - 1] = v;
#pragma unroll
  for (int i = K - 1; i > 0; --i) {
    if (tk_before(lk[i], li[i], lk[i - 1], li[i - 1])) {
      const uint32_t tk = lk[i], ti = li[i];
      const float tv = lv[i];
      lk[i] = lk[i - 1];
      li[i] = li[i - 1];
      lv[i] = lv[i - 1];
      lk[i - 1] = tk;
      li[i - 1] = ti;
      lv[i - 1] = tv;
    }
  }
}

constexpr int kTkRowThreads = 1024;  // steps 2-4: one workgroup of 16 waves per row
constexpr int kTkRowWaves = kTkRowThreads / 64;

// LDS of steps 2-4: the active spans' indices [n], then the candidates'
// values [n k] and indices [n k]
__host__ __device__ inline uint32_t tk_row_lds(int n, int k) { return (uint32_t)n * 4u * (1u + 2u * (uint32_t)k); }

// Steps 2-4 for one row (one workgroup):
//   2. wave 0: tau = the k-th largest of the row's n span keys, repeats
//      counted (0 when n < k): k rounds, each finds the largest remaining key
//      and one lane that holds it drops it; then the list of spans with keys
//      >= tau;
//   3. each wave takes listed spans w, w + 16, ...  A span with at most k
//      elements of key >= tau hands all of them on (every element of the
//      result has such a key); a span with more hands on its k best: k
//      rounds in which each lane offers its best element not yet taken (the
//      lowest index among equal keys: a lane's elements run in index order),
//      the wave picks the best offer and the offering lane marks it taken.
//      Candidates go to LDS at places taken by an LDS counter;
//   4. wave 0 ranks the candidates: with at most 64 (the usual case) each
//      lane counts the candidates before its own and the k first ranks are
//      written; with more, every lane keeps a sorted list of its K best and k
//      rounds take the best list head.  The order of the candidates in LDS
//      does not matter: (key, index) pairs are distinct.
template <int K>
__global__ __launch_bounds__(kTkRowThreads) void topk_row_kernel(const float* Y, int64_t V, int n, int k,
                                                                 const uint32_t* skey, float* out_val,
                                                                 int32_t* out_idx, int64_t out_ld) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* s_list = reinterpret_cast<uint32_t*>(smem);
  float* c_val = reinterpret_cast<float*>(smem + 4u * (uint32_t)n);
  uint32_t* c_idx = reinterpret_cast<uint32_t*>(smem + 4u * (uint32_t)n * (1u + (uint32_t)k));
  __shared__ int s_count, s_ncand;
  __shared__ uint32_t s_tau;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  if (wave == 0) {
    uint32_t x[kTkSpansPerLane];
#pragma unroll
    for (int e = 0; e < kTkSpansPerLane; ++e) {
      const int c = lane + 64 * e;
      x[e] = c < n ? skey[row * n + c] : 0u;
    }
    uint32_t taken = 0u, t = 0u;
    for (int r = 0; r < k; ++r) {
      uint32_t bk = 0u;
      int be = -1;
#pragma unroll
      for (int e = 0; e < kTkSpansPerLane; ++e)
        if (lane + 64 * e < n && !((taken >> e) & 1u) && (be < 0 || x[e] > bk)) {
          bk = x[e];
          be = e;
        }
      t = wave_max_u32(be < 0 ? 0u : bk);
      const uint64_t m = __ballot(be >= 0 && bk == t);
      if (m && lane == (int)__builtin_ctzll(m)) taken |= 1u << be;
    }
    if (k > n) t = 0u;
    int count = 0;
#pragma unroll
    for (int e = 0; e < kTkSpansPerLane; ++e) {
      const bool on = lane + 64 * e < n && x[e] >= t;
      const uint64_t m = __ballot(on);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (on) s_list[count + below] = (uint32_t)(lane + 64 * e);
      count += __builtin_popcountll(m);
    }
    if (lane == 0) {
      s_count = count;
      s_tau = t;
      s_ncand = 0;
    }
  }
  __syncthreads();
  const int count = s_count;
  const uint32_t t = s_tau;
  const float* y = Y + row * V;
  for (int a = wave; a < count; a += kTkRowWaves) {  // wave-uniform
    const int64_t base = (int64_t)s_list[a] * kTkWaveSpan + lane;
    float x[kTkPer];
    uint32_t kx[kTkPer];
    uint64_t on[kTkPer];
    int above = 0;
#pragma unroll
    for (int e = 0; e < kTkPer; ++e) {
      const int64_t v = base + 64 * e;
      x[e] = v < V ? y[v] : __builtin_nanf("");
      kx[e] = tk_key(x[e]);
      on[e] = __ballot(v < V && kx[e] >= t);
      above += __builtin_popcountll(on[e]);
    }
    if (above <= k) {  // every element with a key >= tau
      int slot = 0;
      if (lane == 0) slot = atomicAdd(&s_ncand, above);
      slot = __shfl(slot, 0);
#pragma unroll
      for (int e = 0; e < kTkPer; ++e) {
        const int below =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(on[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)on[e], 0u));
        if ((on[e] >> lane) & 1u) {
          c_val[slot + below] = x[e];
          c_idx[slot + below] = (uint32_t)(base + 64 * e);
        }
        slot += __builtin_popcountll(on[e]);
      }
      continue;
    }
    int slot = 0;  // the span's k best
    if (lane == 0) slot = atomicAdd(&s_ncand, k);
    slot = __shfl(slot, 0);
    uint32_t taken = 0u;
    for (int r = 0; r < k; ++r) {
      uint32_t bk = 0u, bi = 0xffffffffu;
      int be = 0;
#pragma unroll
      for (int e = 0; e < kTkPer; ++e) {
        const int64_t v = base + 64 * e;
        const uint32_t vi = v < V ? (uint32_t)v : kTkNoIdx;
        if (!((taken >> e) & 1u) && tk_before(kx[e], vi, bk, bi)) {
          bk = kx[e];
          bi = vi;
          be = e;
        }
      }
      uint32_t wk, wi;
      const int wl = wave_best(bk, bi, wk, wi);
      float xv = 0.0f;
#pragma unroll
      for (int e = 0; e < kTkPer; ++e) xv = e == be ? x[e] : xv;
      const float val = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(xv), wl));
      if (lane == 0) {
        c_val[slot + r] = val;
        c_idx[slot + r] = wi;
      }
      if (lane == wl) taken |= 1u << be;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const int nc = s_ncand;
  if (nc <= 64) {
    // rank of the lane's candidate among all of them
    const bool mine = lane < nc;
    const float v = mine ? c_val[lane] : 0.0f;
    const uint32_t key = mine ? tk_key(v) : 0u, idx = mine ? c_idx[lane] : 0xffffffffu;
    int rank = 0;
    for (int c = 0; c < nc; ++c) rank += tk_before(tk_key(c_val[c]), c_idx[c], key, idx) ? 1 : 0;
    if (mine && rank < k) {
      out_val[row * out_ld + rank] = v;
      out_idx[row * out_ld + rank] = (int32_t)idx;
    }
    return;
  }
  uint32_t lk[K], li[K];
  float lv[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    lk[i] = 0u;
    li[i] = 0xffffffffu;
    lv[i] = 0.0f;
  }
  for (int c = lane; c < nc; c += 64) tk_insert(lk, li, lv, tk_key(c_val[c]), c_idx[c], c_val[c]);
  for (int r = 0; r < k; ++r) {
    uint32_t wk, wi;
    const int wl = wave_best(lk[0], li[0], wk, wi);
    const float val = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(lv[0]), wl));
    if (lane == 0) {
      out_val[row * out_ld + r] = val;
      out_idx[row * out_ld + r] = (int32_t)wi;
    }
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < K - 1; ++i) {
        lk[i] = lk[i + 1];
        li[i] = li[i + 1];
        lv[i] = lv[i + 1];
      }
      lk[K - 1] = 0u;
      li[K - 1] = 0xffffffffu;
    }
  }
}

int64_t tk_pieces(int64_t V) { return (V + kTkPiece - 1) / kTkPiece; }

// Selection scratch of a chunk of `rows` rows: the span keys.
uint64_t tk_scratch_bytes(int64_t rows, int64_t V) {
  return up256((uint64_t)rows * (uint64_t)tk_pieces(V) * kTkWaves * 4);
}

template <int K>
hipError_t launch_topk_k(const float* Y, int64_t rows, int64_t V, int k, uint8_t* scratch, float* out_val,
                         int32_t* out_idx, int64_t out_ld, hipStream_t s) {
  const int P = (int)tk_pieces(V), n = P * kTkWaves;
  uint32_t* skey = reinterpret_cast<uint32_t*>(scratch);
  hipLaunchKernelGGL(topk_spanmax_kernel, dim3((unsigned)P, (unsigned)rows), dim3(kTkThreads), 0, s, Y, V, skey);
  hipLaunchKernelGGL((topk_row_kernel<K>), dim3((unsigned)rows), dim3(kTkRowThreads), tk_row_lds(n, k), s, Y, V, n, k,
                     skey, out_val, out_idx, out_ld);
  return hipGetLastError();
}

hipError_t launch_topk(const float* Y, int64_t rows, int64_t V, int k, uint8_t* scratch, float* out_val,
                       int32_t* out_idx, int64_t out_ld, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return k <= 4 ? launch_topk_k<4>(Y, rows, V, k, scratch, out_val, out_idx, out_ld, s)
                : launch_topk_k<kTkMax>(Y, rows, V, k, scratch, out_val, out_idx, out_ld, s);
}

int topk_layout(const archead_dims* d, int64_t n_tokens, uint64_t* fwd_bytes, uint64_t* total) {
  const int64_t rows = n_tokens < kTkChunkRows ? n_tokens : kTkChunkRows;
  int rc = archead_workspace_bytes(d, rows, fwd_bytes);
  if (rc) return rc;
  *fwd_bytes = up256(*fwd_bytes);
  *total = rows > 0 ? *fwd_bytes + up256((uint64_t)rows * (uint64_t)d->V * 4) + tk_scratch_bytes(rows, d->V) : 0;
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
  if (tk_pieces(d->V) * kTkWaves > 64 * kTkSpansPerLane) return ARCHEAD_E_UNSUPPORTED;  // V > 2^20
  if (N == 0) return ARCHEAD_OK;
  if (!top_val || !top_idx || !head->workspace) return ARCHEAD_E_NULL;
  if ((reinterpret_cast<uintptr_t>(top_val) | reinterpret_cast<uintptr_t>(top_idx)) % 4) return ARCHEAD_E_ALIGN;
  if (reinterpret_cast<uintptr_t>(head->workspace) % ARCHEAD_ALIGNMENT) return ARCHEAD_E_ALIGN;
  if (head->workspace_bytes < need) return ARCHEAD_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* Yc = reinterpret_cast<float*>(static_cast<uint8_t*>(head->workspace) + fwd);
  const uint64_t ybytes = up256((uint64_t)(N < kTkChunkRows ? N : kTkChunkRows) * (uint64_t)d->V * 4);
  uint8_t* scratch = static_cast<uint8_t*>(head->workspace) + fwd + ybytes;  // sized for the largest chunk
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
    if (launch_topk(Yc, rows, d->V, k, scratch, top_val + t0 * k, top_idx + t0 * k, k, s) != hipSuccess)
      return ARCHEAD_E_HIP;
  }
  return ARCHEAD_OK;
}

}  // extern "C"
