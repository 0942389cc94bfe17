// Per-row logit statistics, combined in pieces: the running maximum, the sum
// of exp(y - max) over the logits seen, the lowest index attaining the
// maximum and the logit of the row's target (if seen).  Two pieces merge
// exactly as the definitions require (ARCHead, Abstract: perplexity and
// cross-entropy; results discussion of Table 8: top-1 agreement), so any
// split of a row's vocabulary into pieces, merged in a fixed order, gives
//   max, argmax, lse = max + log(sum), ce = lse - y[target].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace archead {

struct RowStat {
  float m;    // running maximum (-inf: nothing seen)
  float s;    // sum of exp(y - m)
  int idx;    // lowest index attaining m (INT32_MAX: nothing seen)
  float yt;   // the target's logit (-inf: not seen)
};

__device__ __forceinline__ RowStat stat_empty() { return RowStat{-INFINITY, 0.0f, INT32_MAX, -INFINITY}; }

// one logit y at vocabulary index v of a row whose target is tgt
__device__ __forceinline__ void stat_add(RowStat& r, float y, int v, int tgt) {
  if (v == tgt) r.yt = y;
  if (y > r.m) {
    r.s = r.s * __expf(r.m - y) + 1.0f;  // exp(-inf) = 0 for the first logit
    r.m = y;
    r.idx = v;
  } else {
    r.s += __expf(y - r.m);
    if (y == r.m && v < r.idx) r.idx = v;
  }
}

// The 16 logits one lane holds in a 32 x 32 result tile: y[4 j + e] at
// vocabulary index v0 + 8 j + e.  One maximum per block; the index of the
// maximum and the target's logit are looked for only in the rare blocks that
// can change them.
__device__ __forceinline__ void stat_add16(RowStat& r, const float (&y)[16], int v0, int tgt) {
  float bm = y[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) bm = fmaxf(bm, y[i]);
  if (bm >= r.m) {
    int bi = INT32_MAX;
#pragma unroll
    for (int i = 15; i >= 0; --i) bi = y[i] == bm ? v0 + 8 * (i >> 2) + (i & 3) : bi;
    r.idx = bm > r.m ? bi : (bi < r.idx ? bi : r.idx);
  }
  const float M = fmaxf(r.m, bm);
  float s = r.m == -INFINITY ? 0.0f : r.s * __expf(r.m - M);
#pragma unroll
  for (int i = 0; i < 16; ++i) s += __expf(y[i] - M);
  r.m = M;
  r.s = s;
  const unsigned d = (unsigned)(tgt - v0);
  if (d < 28u && (d & 4u) == 0u) {
    const int ti = (int)(d >> 3) * 4 + (int)(d & 3u);
#pragma unroll
    for (int i = 0; i < 16; ++i) r.yt = i == ti ? y[i] : r.yt;
  }
}

__device__ __forceinline__ RowStat stat_merge(const RowStat& a, const RowStat& b) {
  RowStat r;
  r.m = fmaxf(a.m, b.m);
  const float sa = a.m == -INFINITY ? 0.0f : a.s * __expf(a.m - r.m);
  const float sb = b.m == -INFINITY ? 0.0f : b.s * __expf(b.m - r.m);
  r.s = sa + sb;
  r.idx = a.m > b.m ? a.idx : b.m > a.m ? b.idx : (a.idx < b.idx ? a.idx : b.idx);
  r.yt = fmaxf(a.yt, b.yt);
  return r;
}

__device__ __forceinline__ f4 stat_pack(const RowStat& r) { return f4{r.m, r.s, __int_as_float(r.idx), r.yt}; }
__device__ __forceinline__ RowStat stat_unpack(const f4& p) {
  return RowStat{p[0], p[1], __float_as_int(p[2]), p[3]};
}

__device__ __forceinline__ RowStat stat_shfl_xor(const RowStat& r, int mask) {
  return RowStat{__shfl_xor(r.m, mask), __shfl_xor(r.s, mask), __shfl_xor(r.idx, mask), __shfl_xor(r.yt, mask)};
}

}  // namespace archead
