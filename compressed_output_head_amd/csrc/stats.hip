// Row statistics of the logits (archead_logits_stats): per token the maximum,
// the lowest index attaining it, log-sum-exp and the cross-entropy of a
// target -- the quantities the pages' quality metrics are built from
// (ARCHead, Abstract: perplexity and cross-entropy; results discussion of
// Table 8: top-1 agreement).
//
// The tile kernel produces them piecewise in its epilogue, one piece per
// (token, 256-row vocabulary tile), and never writes Y.  For the few-token
// decode path Y (at most 16 rows) is written to the workspace and
// rowstats_y_kernel cuts each row into kStatChunks pieces.  stats_reduce
// merges a token's pieces in a fixed order, so the results do not depend on
// scheduling.
#include "internal.h"
#include "rowstat.h"

namespace archead {

namespace {

constexpr int kStatThreads = 256;

// Merge the kStatThreads values of `r` held by the workgroup's threads into
// thread 0, in a fixed tree order.
__device__ RowStat block_merge(RowStat r, f4* sbuf) {
  const int tid = threadIdx.x;
  sbuf[tid] = stat_pack(r);
  __syncthreads();
  for (int half = kStatThreads / 2; half > 0; half >>= 1) {
    if (tid < half) sbuf[tid] = stat_pack(stat_merge(stat_unpack(sbuf[tid]), stat_unpack(sbuf[tid + half])));
    __syncthreads();
  }
  return stat_unpack(sbuf[0]);
}

// Workgroup (c, n): piece c of token n's row of Y, the columns
// [c * w, min(V, (c + 1) * w)) with w = ceil(V / kStatChunks).
__global__ __launch_bounds__(kStatThreads) void rowstats_y_kernel(const FwdArgs a, const float* Y, int64_t y_stride) {
  __shared__ f4 sbuf[kStatThreads];
  const int c = blockIdx.x;
  const int64_t n = blockIdx.y;
  const int64_t w = (a.V + kStatChunks - 1) / kStatChunks;
  const int64_t v0 = c * w, v1 = v0 + w < a.V ? v0 + w : a.V;
  const int tgt = a.targets ? a.targets[n] : -1;
  RowStat r = stat_empty();
  for (int64_t v = v0 + threadIdx.x; v < v1; v += kStatThreads) stat_add(r, Y[n * y_stride + v], (int)v, tgt);
  r = block_merge(r, sbuf);
  if (threadIdx.x == 0) reinterpret_cast<f4*>(a.st_part)[n * a.st_nparts + c] = stat_pack(r);
}

// Workgroup n: token n's a.st_nparts pieces, thread t taking pieces t,
// t + 256, ... in order, then the tree.
__global__ __launch_bounds__(kStatThreads) void stats_reduce_kernel(const FwdArgs a, float* row_max,
                                                                    int32_t* row_argmax, float* row_lse,
                                                                    float* row_ce) {
  __shared__ f4 sbuf[kStatThreads];
  const int64_t n = blockIdx.x;
  const f4* part = reinterpret_cast<const f4*>(a.st_part) + n * a.st_nparts;
  RowStat r = stat_empty();
  for (int64_t p = threadIdx.x; p < a.st_nparts; p += kStatThreads) r = stat_merge(r, stat_unpack(part[p]));
  r = block_merge(r, sbuf);
  if (threadIdx.x == 0) {
    const float lse = r.m + __logf(r.s);
    if (row_max) row_max[n] = r.m;
    if (row_argmax) row_argmax[n] = r.idx;
    if (row_lse) row_lse[n] = lse;
    if (row_ce) row_ce[n] = r.yt == -INFINITY ? __builtin_nanf("") : lse - r.yt;
  }
}

}  // namespace

hipError_t launch_rowstats_y(const FwdArgs& a, const float* Y, int64_t y_stride, hipStream_t s) {
  hipLaunchKernelGGL(rowstats_y_kernel, dim3(kStatChunks, (unsigned)a.N), dim3(kStatThreads), 0, s, a, Y, y_stride);
  return hipGetLastError();
}

hipError_t launch_stats_reduce(const FwdArgs& a, float* row_max, int32_t* row_argmax, float* row_lse,
                               float* row_ce, hipStream_t s) {
  hipLaunchKernelGGL(stats_reduce_kernel, dim3((unsigned)a.N), dim3(kStatThreads), 0, s, a, row_max, row_argmax,
                     row_lse, row_ce);
  return hipGetLastError();
}

}  // namespace archead
