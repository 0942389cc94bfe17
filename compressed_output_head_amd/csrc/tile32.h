// The large-N tile kernel on the 32 x 32 x 16 MFMA and its host-side launch
// helpers, shared by the translation units that instantiate it (Y output in
// tile.hip, row statistics in tile_stats.hip).
#pragma once

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "rowstat.h"

namespace archead {

namespace {

// ---------------------------------------------------------------------------
// Tile kernel on the 32 x 32 x 16 MFMA: 32 TT tokens x 256 vocabulary rows
// per workgroup (TT = 2, 4 or 8 token tiles), eight waves (two per SIMD).
// Each wave takes all the workgroup's tokens and one 32-row vocabulary block
// (TT result tiles of 32 x 32, 16 TT fp32 accumulators per lane).  The hidden
// dimension advances 16 KS columns (KS MFMA steps) per stage.
//
//   H (32-row layout, written by the prep kernel): an LDS ring of 4 stages of
//     TT token tiles x KS steps x 1 KB fragments, filled by buffer loads
//     straight into LDS four stages ahead; one barrier per stage.
//   W: lane l of a wave reads, for 32-row vocabulary block CB, row l%16 of
//     packed block 2 CB + (l/16)%2 at packed lane (l%16) + 16 q, q = l/32 in
//     the first half of a k-tile and l/32 + 2 in the second; the 16 bytes give
//     its four 8-column runs of that half, one per MFMA step.  These loads run
//     four stages ahead in a register ring.  Step t of half h thus covers runs
//     R = 4 t + 2 h + l/32, the order the prep kernel gives H.
//   Group codes: the workgroup's 256 rows of codes are copied to LDS once.
// Each MFMA step's operands (TT H fragments from LDS, the W fragment unpacked
// to exact fp16 integers q4 * c8) are fetched while the previous step's MFMAs
// run, and the next stage's first step is fetched right after the barrier
// that publishes it.  Every global read goes through a buffer resource: a
// wave-uniform offset plus a small per-lane one.
// TT (a template parameter): 32-token tiles per workgroup, 2, 4 or 8
constexpr int kT32CB = 8;     // 32-row vocabulary blocks per workgroup
constexpr int kT32Waves = 8;  // one wave per vocabulary block; every wave takes all the tokens
constexpr int kT32Threads = 64 * kT32Waves;
constexpr int kT32WCB = 1;    // vocabulary blocks per wave
constexpr int kT32Ahead = 4;  // stages between a load's issue and its stage (H: 4 LDS slots, W: 4 register slots)
constexpr int kT32MaxCodes = 64;  // group codes per row the workgroup can hold in LDS
// LDS row stride of the group codes: an odd number of dwords, so the 32 rows
// one wave reads at a time fall in 32 different banks
__host__ __device__ constexpr int t32_code_stride(int ng) { return 4 * (((ng + 3) / 4) | 1); }
// MFMA steps (of 16 columns) per stage: the LDS ring holds 4 stages of TT KS
// 1 KB H fragments, so smaller token tiles take longer stages and keep more
// of the head in flight
__host__ __device__ constexpr int t32_ks(int tt) { return tt <= 4 ? 8 : 4; }
constexpr int kT32Group = 4;  // token tiles that walk the vocabulary together
constexpr int kEpiChunk = 2;  // low-rank rank steps whose loads are issued together
constexpr int kEpiLdsSteps = 8;  // up to 128 padded ranks: Z of the workgroup fits the H ring
constexpr int kXcds = 8;


// Workgroup barrier for the LDS ring: this wave's copies up to the last n
// vector-memory operations and all its LDS reads are complete, then every
// wave meets.  Buffer-to-LDS copies land in LDS when their vmcnt retires, so
// after the barrier every wave's copies are visible.  No fence is emitted (a
// fence would wait for every copy in flight); the empty asm statements with a
// memory clobber keep the compiler from moving memory accesses across.
template <int n>
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | (n & 0xF) | (((n >> 4) & 3) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}


// f(integral_constant<I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

struct Acc4 {  // low-rank accumulators of one wave's vocabulary blocks
  f16x v[kT32WCB];
};

struct T32Grid {
  int ntiles, ncb, ttiles, vtiles;
};
__host__ __device__ inline T32Grid t32_grid(const FwdArgs& a, int tt) {
  T32Grid t;
  t.ntiles = (int)(a.n32 >> 5);
  t.ncb = (int)((a.nb + 1) >> 1);
  t.ttiles = (t.ntiles + tt - 1) / tt;
  t.vtiles = (t.ncb + kT32CB - 1) / kT32CB;
  return t;
}

// Tile L of the walk order: groups of kT32Group token tiles walk the
// vocabulary together (the last group may be narrower).
__host__ __device__ inline void t32_tile(const T32Grid& G, int L, int& vt, int& ttile) {
  const int groups = G.ttiles / kT32Group, span = kT32Group * G.vtiles;
  if (L < groups * span) {
    const int rr = L % span;
    vt = rr / kT32Group;
    ttile = (L / span) * kT32Group + rr % kT32Group;
  } else {
    const int w = G.ttiles - groups * kT32Group, rr = L - groups * span;
    vt = rr / w;
    ttile = groups * kT32Group + rr % w;
  }
}

// Tiles full .. (all tiles - 1) of the walk order (the last, partly filled
// round of workgroups) are each split into s parts of the hidden dimension:
// workgroup full + s j + p computes part p of tile full + j and writes fp32
// partial sums, which t32_reduce_kernel adds up in part order.
struct T32Split {
  int full, s;
};

// One 16-byte buffer-to-LDS copy per lane.  Kept out of the kernel template:
// called from inside it directly, the builtin makes the host pass reject the
// template's instantiation without a diagnostic, and no launch stub is made.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rs, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 0);
}

// GC: group codes per k-tile and row that one stage needs: 0 -> one (g >= 128),
// 1 -> two (g = 64), 2 -> four (g = 32)
// The H ring is four separate LDS arrays, one per slot, chosen at compile
// time: with one array the compiler cannot tell the slot being filled by
// buffer-to-LDS copies from the slot being read, and makes every read wait
// for all copies in flight.  T32_SLOT(S) names slot S (S a constant).
#define T32_SLOT(S) (*((S) == 0 ? &sH0 : (S) == 1 ? &sH1 : (S) == 2 ? &sH2 : &sH3))

// ST: instead of storing Y, each workgroup reduces its 256 logits of every
// token to a row-statistics piece, written to a.st_part[token][vt].
template <int GC, int TT, bool ST>
__global__ __launch_bounds__(kT32Threads, 1) void tile32_kernel(const FwdArgs a, const T32Split sp) {
  constexpr int kT32TT = TT, kT32MT = TT;     // token tiles per workgroup and per wave
  constexpr int KS = t32_ks(TT);              // MFMA steps per stage
  constexpr int kLK = KS == 8 ? 3 : 2;        // log2(KS)
  constexpr int kSPT = 8 / KS;                // stages per 128-column k-tile
  constexpr int kT32HOps = TT * KS / kT32Waves;  // H copies per wave and stage
  constexpr int kWOps = kT32WCB * KS / 4;        // W loads per wave and stage
  static_assert(kT32HOps >= 1 && TT * KS == kT32HOps * kT32Waves, "TT must be 2, 4 or 8");
  __shared__ h8 sH0[kT32TT][KS][64], sH1[kT32TT][KS][64], sH2[kT32TT][KS][64], sH3[kT32TT][KS][64];
  extern __shared__ __align__(16) uint8_t sCode[];  // [256 rows][t32_code_stride(ng)], sized at launch
  __shared__ float sTok[kT32TT * 32][2];  // hscale, zscale of the workgroup's tokens
  __shared__ int sTgt[ST ? kT32TT * 32 : 1];  // targets of the workgroup's tokens (statistics)
  __shared__ __align__(16) float sVR[kT32CB * 32], sVC[kT32CB * 32], sVW[kT32CB * 32];  // s_R, s_Ac, s_Aw
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = 0, wn = wave;  // wave row 0: every wave takes all the tokens
  const int g = lane >> 5, c32 = lane & 31;
  const T32Grid G = t32_grid(a, TT);

  // Workgroups are dealt to the XCDs round robin.  Those that take whole
  // tiles are renumbered so each XCD owns one contiguous range of the walk
  // order, so the workgroups resident on one XCD share a few H row sets and
  // packed vocabulary tiles in its L2.  The rest take one part of the hidden
  // dimension of a split tile.
  const int b = blockIdx.x;
  const bool split = b >= sp.full;
  int L, part = 0;
  if (!split) {
    const int per = sp.full / kXcds, rem = sp.full % kXcds, x = b % kXcds;
    L = x * per + (x < rem ? x : rem) + b / kXcds;
  } else {
    const int q = b - sp.full, j = q / sp.s;
    L = sp.full + j;
    part = q - j * sp.s;
  }
  int vt, ttile;
  t32_tile(G, L, vt, ttile);
  const int tt0 = ttile * kT32TT;           // first 32-token tile
  const int cb0 = vt * kT32CB + wn * kT32WCB;  // first vocabulary block of this wave
  // stages of 16 KS columns: all of them (at least 2), or this part's share
  // of whole k-tiles (at least 4 stages: the host splits a tile in at most a
  // quarter as many parts as it has stages)
  int kb = 0, nS = (int)(a.D / (16 * KS));
  if (split) {
    const int nu = nS / kSPT;
    kb = kSPT * (part * nu / sp.s);
    nS = kSPT * ((part + 1) * nu / sp.s) - kb;
  }

  // H: the TT KS fragments of a stage (TT token tiles x KS MFMA steps) are
  // spread over the waves, fragment f = kT32Waves i + wave being token tile
  // f / KS, step f % KS.  Token tiles past the last re-read the last one:
  // their rows are never stored.
  const __amdgpu_buffer_rsrc_t hrs = buffer_rsrc(a.hf, (uint32_t)(a.n32 * a.D * 2));
  const uint32_t lane16 = (uint32_t)lane * 16u;
  const uint32_t hT = (uint32_t)a.nkt * 8192u;  // bytes per token tile
  uint32_t hoff[kT32HOps];
#pragma unroll
  for (int i = 0; i < kT32HOps; ++i) {
    const int f = kT32Waves * i + wave, tt = f >> kLK;
    hoff[i] = (uint32_t)(tt0 + tt < G.ntiles ? tt0 + tt : G.ntiles - 1) * hT + (uint32_t)(f & (KS - 1)) * 1024u +
              (uint32_t)kb * (KS * 1024u);
  }
  auto load_h = [&](int ks, auto S_) {
    constexpr int S = decltype(S_)::value;
#pragma unroll
    for (int i = 0; i < kT32HOps; ++i) {
      const int f = kT32Waves * i + wave;
      lds_copy16(hrs, &T32_SLOT(S)[f >> kLK][f & (KS - 1)][0], lane16, hoff[i] + (uint32_t)ks * (KS * 1024u));
    }
  };

  // W: per-lane byte offsets of this lane's row in each of its blocks (a
  // block past the end re-reads the last one; its results are never stored)
  const uint32_t tstride = (uint32_t)a.nb * 1024u;  // bytes per k-tile
  const uint32_t wkb = (uint32_t)(kb / kSPT) * tstride;  // the part's first k-tile
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(a.r_codes + wkb, (uint32_t)(a.nb * 16 * (a.D / 2)) - wkb);
  uint32_t wvoff[kT32WCB];
#pragma unroll
  for (int cb = 0; cb < kT32WCB; ++cb) {
    const int CB = cb0 + cb < G.ncb ? cb0 + cb : G.ncb - 1;
    int b = 2 * CB + ((lane >> 4) & 1);
    if (b >= a.nb) b = (int)a.nb - 1;
    wvoff[cb] = (uint32_t)b * 1024u + (uint32_t)(lane & 15) * 16u + (uint32_t)g * 256u;
  }
  // one 16-byte load per half k-tile (4 MFMA steps): one per stage of 64
  // columns, two per stage of 128
  u4 wr[kT32Ahead][kT32WCB][KS / 4];
  auto load_w = [&](int ks, auto S_) {
    constexpr int S = decltype(S_)::value;
#pragma unroll
    for (int h = 0; h < KS / 4; ++h) {
      const uint32_t soff = (uint32_t)(ks / kSPT) * tstride + 512u * (uint32_t)(kSPT == 2 ? (ks & 1) : h);
#pragma unroll
      for (int cb = 0; cb < kT32WCB; ++cb)
        wr[S][cb][h] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wvoff[cb], soff, 0));
    }
  };

  // Low-rank operands.  With at most kEpiLdsSteps rank steps (the common
  // case) Z of the workgroup's token tiles is copied into the H ring during
  // the last four stages, one slot per stage, and this lane's A codes are
  // loaded with the prologue.
  const int r = a.r_c + a.r_r;
  const int csteps = a.rc32 / 16, esteps = (a.rc32 + a.rr32) / 16;
  const bool zlds = esteps <= kEpiLdsSteps;
  const int zper = 2 * esteps;  // 1 KB Z fragments per token tile (hi, lo per step)
  const int8_t* arow[kT32WCB];
#pragma unroll
  for (int cb = 0; cb < kT32WCB; ++cb) {
    const int CB = cb0 + cb < G.ncb ? cb0 + cb : G.ncb - 1;
    int64_t v = 32 * (int64_t)CB + c32;
    if (v >= 16 * a.nb) v = 16 * a.nb - 1;
    arow[cb] = a.a_codes + v * r;
  }
  // A codes of this lane's row in block cb for rank step s (zero past the part's rank)
  auto a_code = [&](int cb, int s) {
    const bool part_c = s < csteps;
    const int sl = part_c ? s : s - csteps;
    const int col = 32 * (sl >> 1) + 16 * g + 8 * (sl & 1);  // rank order of the 32-row Z layout
    u2 raw = {0u, 0u};
    if (col < (part_c ? a.r_c : a.r_r)) raw = *reinterpret_cast<const u2*>(arow[cb] + (part_c ? 0 : a.r_c) + col);
    return raw;
  };
  u2 ac[kT32WCB][kEpiLdsSteps];
#pragma unroll
  for (int cb = 0; cb < kT32WCB; ++cb)
#pragma unroll
    for (int s = 0; s < kEpiLdsSteps; ++s) ac[cb][s] = zlds && s < esteps ? a_code(cb, s) : u2{0u, 0u};
  // Entry j of the copy sequence into slot j % 4: H stage j for j < nS; past
  // the last stage, Z of the workgroup (or the last stage again when Z is
  // read from memory in the epilogue).  Token tile tt's Z fragment rem sits
  // at z = tt * 2^zsh + rem (2^zsh the power of two >= zper, at most 16, so
  // all TT tiles fit the ring's 4 KS TT >= 16 TT positions): slot
  // z / (KS TT), the position z % (KS TT) an H fragment would take.  Positions past a tile's
  // fragments repeat one of them.  The source is a uniform select, so every
  // copy has the same form as an H copy.
  const __amdgpu_buffer_rsrc_t zrs = buffer_rsrc(a.zf, (uint32_t)(a.n32 * (a.rc32 + a.rr32) * 4));
  const int zsh = zper <= 1 ? 0 : 32 - __builtin_clz((unsigned)(zper - 1));
  auto load_slot = [&](int j, auto S_) {
    constexpr int S = decltype(S_)::value;
    const bool zsrc = j >= nS && zlds;
    const int jh = j < nS ? j : nS - 1;
#pragma unroll
    for (int i = 0; i < kT32HOps; ++i) {
      const int f = kT32Waves * i + wave;
      const int z = KS * kT32TT * S + f;
      int tt = z >> zsh, rem = z & ((1 << zsh) - 1);
      if (tt > kT32TT - 1) tt = kT32TT - 1;
      if (rem > zper - 1) rem = zper - 1;  // zper = 0: negative, read past the end as zero
      const int T = tt0 + tt < G.ntiles ? tt0 + tt : G.ntiles - 1;  // padding tiles are never stored
      const uint32_t off = zsrc ? (uint32_t)(T * zper + rem) * 1024u : hoff[i] + (uint32_t)jh * (KS * 1024u);
      lds_copy16(zsrc ? zrs : hrs, &T32_SLOT(S)[f >> kLK][f & (KS - 1)][0], lane16, off);
    }
  };

  // prologue: the workgroup's group codes into registers (row tid / 2, half
  // tid % 2 of its ng codes: dwords when rows are dword aligned, else bytes),
  // then the first kT32Ahead stages of W and H in flight; the codes go on to
  // LDS as soon as they arrive.  Rows past the end read as zero.
  const int ng = a.ng, cstride = t32_code_stride(ng);
  const int crow_ = tid >> 1, chalf = tid & 1;
  uint32_t craw[kT32MaxCodes / 8];
  const bool cdw = (ng & 3) == 0;
  {
    const __amdgpu_buffer_rsrc_t crs = buffer_rsrc(a.r_gcodes, (uint32_t)(a.nb * 16 * ng));
    const uint32_t rbase = ((uint32_t)vt * (kT32CB * 32) + (uint32_t)crow_) * (uint32_t)ng;
    if (cdw) {
#pragma unroll
      for (int j = 0; j < kT32MaxCodes / 8; ++j) {
        const int d = 2 * j + chalf;  // dword of the row
        craw[j] = 4 * d < ng ? __builtin_amdgcn_raw_buffer_load_b32(crs, rbase + 4u * (uint32_t)d, 0, 0) : 0u;
      }
    } else {  // fewer than 4 codes per row, or a count that is not a multiple of 4: bytes
#pragma unroll
      for (int j = 0; j < kT32MaxCodes / 8; ++j) {
        const int c = 2 * j + chalf;
        craw[j] = c < ng ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(crs, rbase + (uint32_t)c, 0, 0) : 0u;
      }
    }
  }
  load_w(0, std::integral_constant<int, 0>{});
  load_h(0, std::integral_constant<int, 0>{});
  load_w(1, std::integral_constant<int, 1>{});
  load_h(1, std::integral_constant<int, 1>{});
  load_w(std::min(2, nS - 1), std::integral_constant<int, 2>{});
  load_slot(2, std::integral_constant<int, 2>{});
  load_w(std::min(3, nS - 1), std::integral_constant<int, 3>{});
  load_slot(3, std::integral_constant<int, 3>{});
  if (cdw) {
#pragma unroll
    for (int j = 0; j < kT32MaxCodes / 8; ++j) {
      const int d = 2 * j + chalf;
      if (4 * d < ng) *reinterpret_cast<uint32_t*>(&sCode[crow_ * cstride + 4 * d]) = craw[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kT32MaxCodes / 8; ++j) {
      const int c = 2 * j + chalf;
      if (c < ng) sCode[crow_ * cstride + c] = (uint8_t)craw[j];
    }
  }
  if (tid < kT32TT * 32) {
    const int64_t tok = std::min<int64_t>(32 * (int64_t)tt0 + tid, a.n32 - 1);
    sTok[tid][0] = a.hscale[tok];
    sTok[tid][1] = part == 0 ? a.zscale[tok] : 0.0f;  // the low-rank term goes with part 0 only
    if constexpr (ST) sTgt[tid] = a.targets && 32 * (int64_t)tt0 + tid < a.N ? a.targets[32 * (int64_t)tt0 + tid] : -1;
  }
  static_assert(kT32Threads >= kT32CB * 32, "one thread per vocabulary row of the workgroup");
  if (tid < kT32CB * 32) {
    const int64_t v = std::min<int64_t>(32 * (int64_t)vt * kT32CB + tid, 16 * a.nb - 1);
    sVR[tid] = f16_to_f32(a.r_rowscale[v]);
    sVC[tid] = a.r_c > 0 ? f16_to_f32(a.a_scales[v * a.nA]) : 0.0f;
    sVW[tid] = a.r_r > 0 ? f16_to_f32(a.a_scales[v * a.nA + a.nA - 1]) : 0.0f;
  }

  // group codes of this lane's rows for one stage: the code of MFMA step t
  // of a half k-tile is byte (GC == 2 ? t : GC == 1 ? t / 2 : 0)
  const int lg = __builtin_ctz((unsigned)a.g);
  uint32_t crow[kT32WCB];
#pragma unroll
  for (int cb = 0; cb < kT32WCB; ++cb)
    crow[cb] = (uint32_t)(32 * (wn * kT32WCB + cb) + 16 * ((lane >> 4) & 1) + (lane & 15)) * (uint32_t)cstride;
  uint32_t cd[2][kT32WCB];
  auto read_codes = [&](int ks, uint32_t(&dst)[kT32WCB]) {
    const int kt = (kb + ks) / kSPT;
#pragma unroll
    for (int cb = 0; cb < kT32WCB; ++cb) {
      if constexpr (GC == 2)
        dst[cb] = *reinterpret_cast<const uint32_t*>(&sCode[crow[cb] + 4 * kt]);
      else if constexpr (GC == 1)
        dst[cb] = *reinterpret_cast<const uint16_t*>(&sCode[crow[cb] + 2 * kt]);
      else
        dst[cb] = sCode[crow[cb] + ((kKTile * kt) >> lg)];
    }
  };

  f16x acc[kT32MT][kT32WCB];
#pragma unroll
  for (int m = 0; m < kT32MT; ++m)
#pragma unroll
    for (int cb = 0; cb < kT32WCB; ++cb) acc[m][cb] = f16x{};

  // operands of one MFMA step, double buffered by step parity
  h8 av[2][kT32MT], bw[2][kT32WCB];
  auto fetch = [&](auto S_, auto T_, auto P_) {
    constexpr int S = decltype(S_)::value, T = decltype(T_)::value, P = decltype(P_)::value;
#pragma unroll
    for (int m = 0; m < kT32MT; ++m) av[P][m] = T32_SLOT(S)[kT32MT * wm + m][T][lane];
#pragma unroll
    for (int cb = 0; cb < kT32WCB; ++cb) {
      const uint32_t c = cd[S & 1][cb];
      constexpr int t = T & 3;  // step of the half k-tile
      const uint32_t code = GC == 2 ? (c >> (8 * t)) & 0xffu : GC == 1 ? (c >> (8 * (t >> 1))) & 0xffu : c;
      bw[P][cb] = unpack_q4_scaled(wr[S][cb][T >> 2][t], (_Float16)(float)code);
    }
  };
  auto mma = [&](auto P_) {
    constexpr int P = decltype(P_)::value;
#pragma unroll
    for (int m = 0; m < kT32MT; ++m)
#pragma unroll
      for (int cb = 0; cb < kT32WCB; ++cb) acc[m][cb] = mfma32(bw[P][cb], av[P][m], acc[m][cb]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // stage 0 complete: wait past the loads of stages 1..3, then publish every
  // wave's copies and the codes
  stage_barrier<3 * (kWOps + kT32HOps)>();
  read_codes(0, cd[0]);
  fetch(I0{}, I0{}, I0{});

  // One stage; S = ks mod 4 is its ring slot (H in LDS, W in registers) at
  // compile time.  The loads of stage ks + 4 go into the slot this stage
  // frees: W once the last step is unpacked, H after the barrier that ends
  // every wave's reads of it.  Past the last stage the H slot receives Z
  // instead (or the last stage again), and W repeats the last stage, which
  // keeps the count of operations in flight the same.
  auto stage = [&](int ks, auto S_) {
    constexpr int S = decltype(S_)::value;
    constexpr std::integral_constant<int, S> Sc{};
    constexpr std::integral_constant<int, (S + 1) & 3> Sn{};
    const int kn = ks + kT32Ahead < nS ? ks + kT32Ahead : nS - 1;
    // each MFMA step is its own scheduling region, so that no unpacking of
    // registers still being loaded is hoisted into it; step t's operands are
    // fetched while step t - 1 runs
    static_for<1, KS>([&](auto T_) {
      constexpr int T = decltype(T_)::value;
      fetch(Sc, T_, std::integral_constant<int, T & 1>{});
      if constexpr (T == 1) read_codes(ks + 1 < nS ? ks + 1 : ks, cd[(S + 1) & 1]);
      if constexpr (T == KS - 1) load_w(kn, Sc);  // the slot's last step is unpacked
      mma(std::integral_constant<int, (T - 1) & 1>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    // stage ks + 1 is complete once this wave has at most the loads of the
    // three stages after it (W of ks + 4 included) in flight
    stage_barrier<3 * kWOps + 2 * kT32HOps>();
    load_slot(ks + kT32Ahead, Sc);
    fetch(Sn, I0{}, I0{});  // past the last stage: harmless reads, never used
    mma(std::integral_constant<int, (KS - 1) & 1>{});
    __builtin_amdgcn_sched_barrier(0);
  };
  int ks = 0;
  for (; ks + 4 <= nS; ks += 4) {
    stage(ks, I0{});
    stage(ks + 1, I1{});
    stage(ks + 2, I2{});
    stage(ks + 3, I3{});
  }
  if constexpr (KS == 4) {
    if (ks < nS) {  // nS is even: two stages remain
      stage(ks, I0{});
      stage(ks + 1, I1{});
    }
  } else {  // one to three stages remain
    if (ks < nS) stage(ks, I0{});
    if (ks + 1 < nS) stage(ks + 1, I1{});
    if (ks + 2 < nS) stage(ks + 2, I2{});
  }
  __builtin_amdgcn_s_waitcnt(0);

  // Epilogue.  Result tile (m, cb): element v of lane l is vocabulary row
  // 32 CB + 8 (v/4) + 4 (l/32) + v%4 and token 32 T + l%32, so each lane holds
  // runs of 4 consecutive logits of one token.  The low-rank term (Z hi/lo
  // against exact INT8 A codes, 16 ranks per MFMA step, one accumulator per
  // part) is added with the scales, and each run is stored at once.
  const bool vec = ((uintptr_t)a.Y & 15) == 0 && (a.Y_stride & 3) == 0;
  // statistics pieces of this lane's token in each token tile
  RowStat st[ST ? kT32MT : 1];
#pragma unroll
  for (int m = 0; m < (ST ? kT32MT : 1); ++m) st[m] = stat_empty();
  // Combine the pieces: lanes l and l + 32 (the two row halves of a token),
  // then the waves in order of their vocabulary blocks, through the H ring
  // once every wave is done with the Z it holds.
  auto finish_stats = [&]() {
    if constexpr (ST) {
      if (split) return;
#pragma unroll
      for (int m = 0; m < kT32MT; ++m) st[m] = stat_merge(st[m], stat_shfl_xor(st[m], 32));
      __syncthreads();
      f4* const sP = reinterpret_cast<f4*>(&sH0[0][0][0]);  // [kT32Waves][32 TT]
      static_assert(sizeof(sH0) >= sizeof(f4) * kT32Waves * kT32TT * 32, "statistics pieces fit one ring slot");
      if (g == 0) {
#pragma unroll
        for (int m = 0; m < kT32MT; ++m) sP[wave * (kT32TT * 32) + 32 * m + c32] = stat_pack(st[m]);
      }
      __syncthreads();
      if (tid < kT32TT * 32) {
        RowStat t = stat_unpack(sP[tid]);
        for (int w = 1; w < kT32Waves; ++w) t = stat_merge(t, stat_unpack(sP[w * (kT32TT * 32) + tid]));
        const int64_t tok = 32 * (int64_t)tt0 + tid;
        if (tok < a.N) reinterpret_cast<f4*>(a.st_part)[tok * a.st_nparts + vt] = stat_pack(t);
      }
    }
  };
  // a split tile's partial sums: [32 TT tokens][kT32CB * 32 rows] fp32
  float* const ypart = a.part + (size_t)(split ? b - sp.full : 0) * (kT32TT * 32 * kT32CB * 32);
  auto store = [&](int m, int cb, const f16x& am, const f16x& pc, const f16x& pw) {
    const int tl = 32 * (kT32MT * wm + m) + c32;  // token within the workgroup
    const int64_t tok = 32 * (int64_t)tt0 + tl;
    if (tok >= a.N || cb0 + cb >= G.ncb) return;
    const float hs = sTok[tl][0], zs = sTok[tl][1];
    const int64_t row = tok * a.Y_stride;
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
      const int lr = 32 * (kT32WCB * wn + cb) + 8 * vg + 4 * g;  // vocabulary row within the workgroup
      const int64_t voc0 = 32 * (int64_t)vt * kT32CB + lr;
      const f4 sr = *reinterpret_cast<const f4*>(&sVR[lr]);
      const f4 sc = *reinterpret_cast<const f4*>(&sVC[lr]);
      const f4 sw = *reinterpret_cast<const f4*>(&sVW[lr]);
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * vg + e;
        y[e] = hs * (sr[e] * am[v]);
        if (r > 0) y[e] = fmaf(zs, fmaf(sw[e], pw[v], sc[e] * pc[v]), y[e]);
      }
      if (ST && !split) {
        if constexpr (ST) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (voc0 + e < a.V) stat_add(st[m], y[e], (int)(voc0 + e), sTgt[tl]);
        }
      } else if (split) {  // tile-local fp32 partial sums
        *reinterpret_cast<f4*>(ypart + tl * (kT32CB * 32) + lr) = f4{y[0], y[1], y[2], y[3]};
      } else if (vec && voc0 + 3 < a.V) {
        if (a.y_bf16)
          *reinterpret_cast<u2*>(reinterpret_cast<uint16_t*>(a.Y) + row + voc0) = pack_bf16x4(y[0], y[1], y[2], y[3]);
        else
          *reinterpret_cast<f4*>(reinterpret_cast<float*>(a.Y) + row + voc0) = f4{y[0], y[1], y[2], y[3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (voc0 + e < a.V) {
            if (a.y_bf16)
              reinterpret_cast<uint16_t*>(a.Y)[row + voc0 + e] = f32_to_bf16(y[e]);
            else
              reinterpret_cast<float*>(a.Y)[row + voc0 + e] = y[e];
          }
        }
      }
    }
  };

  // Whole workgroup tile in range (every token and vocabulary row exists),
  // aligned rows and an output span within 32-bit offsets: a straight-line
  // epilogue with the split between the two low-rank parts fixed at compile
  // time (csteps is even), the row scales in registers and buffer stores at
  // uniform offsets.
  // Z fragment rem of the workgroup's token tile tt from the ring (rem past
  // the tile's fragments reads a copy or an old H fragment; its A codes are 0)
  auto zfrag = [&](int tt, int rem) {
    int z = (tt << zsh) + rem;
    if (z > 4 * KS * kT32TT - 1) z = 4 * KS * kT32TT - 1;
    const int slot = z / (KS * kT32TT), pos = z - slot * KS * kT32TT;
    const h8* base = slot == 0 ? &sH0[0][0][0] : slot == 1 ? &sH1[0][0][0] : slot == 2 ? &sH2[0][0][0] : &sH3[0][0][0];
    return base[pos * 64 + lane];
  };
  // output of the straight-line epilogue: Y, or for a split tile its partial
  // sums (every row of the tile, whole or not)
  const bool ybf = !split && a.y_bf16;
  const uint64_t es = ybf ? 2 : 4;
  const uint64_t ys = split ? kT32CB * 32 : (uint64_t)a.Y_stride;  // row stride
  const bool whole = 32 * (int64_t)(tt0 + kT32TT) <= a.N && 32 * ((int64_t)vt * kT32CB + kT32CB) <= a.V;
  const bool fast = zlds && (split || (ST ? whole : vec && whole && (uint64_t)a.N * (uint64_t)a.Y_stride * es < (1ull << 32)));
  if (fast) {
    __syncthreads();  // every wave's Z copies (complete after the wait above) are visible
    const __amdgpu_buffer_rsrc_t yrs =
        split ? buffer_rsrc(ypart, (uint32_t)(kT32TT * 32 * kT32CB * 32 * 4))
              : buffer_rsrc(a.Y, (uint32_t)((uint64_t)a.N * (uint64_t)a.Y_stride * es));
    const int ytt0 = split ? 0 : tt0;                        // first token tile of the output
    const uint64_t ycb0 = split ? 0 : (uint64_t)vt * kT32CB;  // first vocabulary block of the output
    // lane part of the output offset: token c32 of the tile, the lane's run of block cb
    uint32_t yoff[kT32WCB];
#pragma unroll
    for (int cb = 0; cb < kT32WCB; ++cb)
      yoff[cb] = (uint32_t)(((uint64_t)c32 * ys + 32 * (ycb0 + kT32WCB * wn + cb) + 4 * g) * es);
    // The wave's tiles (m, cb) one at a time, each its own scheduling region
    // (the two waves of a SIMD overlap one's scaling with the other's MFMAs).
    auto epilogue = [&](auto CS_) {
      constexpr int CS = decltype(CS_)::value;
      constexpr int kTiles = kT32MT * kT32WCB;
      auto low_rank = [&](auto J_, f16x& pc, f16x& pw) {
        constexpr int m = decltype(J_)::value / kT32WCB, cb = decltype(J_)::value % kT32WCB;
        const int tt = kT32MT * wm + m;
        pc = f16x{};
        pw = f16x{};
        static_for<0, kEpiLdsSteps>([&](auto S_) {
          constexpr int s = decltype(S_)::value;
          const h8 zh = zfrag(tt, 2 * s);  // past the tile's zper: its A codes are 0
          const h8 zl = zfrag(tt, 2 * s + 1);
          const h8 av = unpack_i8x8(ac[cb][s][0], ac[cb][s][1]);
          if constexpr (s < CS) {
            pc = mfma32(av, zh, pc);
            pc = mfma32(av, zl, pc);
          } else {
            pw = mfma32(av, zh, pw);
            pw = mfma32(av, zl, pw);
          }
        });
      };
      auto finish = [&](auto J_, const f16x& pc, const f16x& pw) {
        constexpr int m = decltype(J_)::value / kT32WCB, cb = decltype(J_)::value % kT32WCB;
        const int tt = kT32MT * wm + m;
        const float hs = sTok[32 * tt + c32][0], zs = sTok[32 * tt + c32][1];
        const uint32_t trow = (uint32_t)((uint64_t)(32 * (ytt0 + tt)) * ys * es);
        const f16x& am = acc[m][cb];
        float y16[ST ? 16 : 1];  // statistics: the tile's 16 logits of this lane
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int lr = 32 * (kT32WCB * wn + cb) + 8 * vg + 4 * g;
          // row scales of block cb, run vg (rows 8 vg + 4 g + e)
          const f4 vr = *reinterpret_cast<const f4*>(&sVR[lr]);
          const f4 vc = *reinterpret_cast<const f4*>(&sVC[lr]);
          const f4 vw = *reinterpret_cast<const f4*>(&sVW[lr]);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * vg + e;
            y[e] = fmaf(zs, fmaf(vw[e], pw[v], vc[e] * pc[v]), hs * (vr[e] * am[v]));
          }
          if (ST && !split) {
            if constexpr (ST) {
#pragma unroll
              for (int e = 0; e < 4; ++e) y16[4 * vg + e] = y[e];
            }
          } else if (ybf) {
            __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(y[0], y[1], y[2], y[3]), yrs, yoff[cb],
                                                  trow + (uint32_t)(16 * vg), 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, f4{y[0], y[1], y[2], y[3]}), yrs,
                                                   yoff[cb], trow + (uint32_t)(32 * vg), 0);
          }
        }
        if constexpr (ST) {
          if (!split) stat_add16(st[m], y16, 32 * (vt * kT32CB + kT32WCB * wn + cb) + 4 * g, sTgt[32 * tt + c32]);
        }
      };
      static_for<0, kTiles>([&](auto J_) {
        __builtin_amdgcn_sched_barrier(0);
        f16x pc, pw;
        low_rank(J_, pc, pw);
        finish(J_, pc, pw);
      });
    };
    switch (csteps) {
      case 0: epilogue(std::integral_constant<int, 0>{}); break;
      case 2: epilogue(std::integral_constant<int, 2>{}); break;
      case 4: epilogue(std::integral_constant<int, 4>{}); break;
      case 6: epilogue(std::integral_constant<int, 6>{}); break;
      default: epilogue(std::integral_constant<int, 8>{}); break;
    }
    finish_stats();
    return;
  }

  if (zlds) {
    __syncthreads();  // every wave's Z copies (complete after the wait above) are visible
    h8 aun[kT32WCB][kEpiLdsSteps];  // A codes unpacked once for all token tiles
#pragma unroll
    for (int cb = 0; cb < kT32WCB; ++cb)
#pragma unroll
      for (int s = 0; s < kEpiLdsSteps; ++s) aun[cb][s] = unpack_i8x8(ac[cb][s][0], ac[cb][s][1]);
    // kEpiBlocks vocabulary blocks at a time: with 8 waves per workgroup the
    // registers only hold one block's low-rank accumulators next to the tile's
    constexpr int kEpiBlocks = kT32WCB >= 4 ? 2 : 1;
    auto tile_pair = [&](auto M_, auto P_) {
      constexpr int m = decltype(M_)::value, cp = kEpiBlocks * decltype(P_)::value;
      const int tt = kT32MT * wm + m;
      if (tt0 + tt >= G.ntiles) return;

      f16x pc[kEpiBlocks], pw[kEpiBlocks];
#pragma unroll
      for (int j = 0; j < kEpiBlocks; ++j) {
        pc[j] = f16x{};
        pw[j] = f16x{};
      }
#pragma unroll
      for (int s = 0; s < kEpiLdsSteps; ++s) {
        if (s < esteps) {
          const h8 zh = zfrag(tt, 2 * s);
          const h8 zl = zfrag(tt, 2 * s + 1);
          h8 av[kEpiBlocks];
#pragma unroll
          for (int j = 0; j < kEpiBlocks; ++j) av[j] = aun[cp + j][s];
          if (s < csteps) {
#pragma unroll
            for (int j = 0; j < kEpiBlocks; ++j) pc[j] = mfma32(av[j], zh, pc[j]);
#pragma unroll
            for (int j = 0; j < kEpiBlocks; ++j) pc[j] = mfma32(av[j], zl, pc[j]);
          } else {
#pragma unroll
            for (int j = 0; j < kEpiBlocks; ++j) pw[j] = mfma32(av[j], zh, pw[j]);
#pragma unroll
            for (int j = 0; j < kEpiBlocks; ++j) pw[j] = mfma32(av[j], zl, pw[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kEpiBlocks; ++j) store(m, cp + j, acc[m][cp + j], pc[j], pw[j]);
    };
    static_for<0, kT32MT>([&](auto M_) {
      static_for<0, kT32WCB / kEpiBlocks>([&](auto P_) { tile_pair(M_, P_); });
    });
    finish_stats();
    return;
  }

  // more ranks: chunks of kEpiChunk rank steps, every load of a chunk issued
  // before its MFMAs
  const h8* zf = reinterpret_cast<const h8*>(a.zf) + lane;
  auto low_rank_part = [&](int T, int s_begin, int s_end) {
    Acc4 p;
#pragma unroll
    for (int cb = 0; cb < kT32WCB; ++cb) p.v[cb] = f16x{};
    for (int s0 = s_begin; s0 < s_end; s0 += kEpiChunk) {
      h8 zh[kEpiChunk], zl[kEpiChunk];
      u2 ac[kEpiChunk][4];
#pragma unroll
      for (int j = 0; j < kEpiChunk; ++j) {
        const int s = s0 + j;
        const bool live = s < s_end;
        const int64_t zi = ((int64_t)T * 2 * esteps + 2 * (live ? s : s_begin)) * 64;
        zh[j] = live ? zf[zi] : h8{0, 0, 0, 0, 0, 0, 0, 0};
        zl[j] = live ? zf[zi + 64] : h8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int cb = 0; cb < kT32WCB; ++cb) ac[j][cb] = live ? a_code(cb, s) : u2{0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < kEpiChunk; ++j)
#pragma unroll
        for (int cb = 0; cb < kT32WCB; ++cb) {
          const h8 av = unpack_i8x8(ac[j][cb][0], ac[j][cb][1]);
          p.v[cb] = mfma32(av, zh[j], p.v[cb]);
          p.v[cb] = mfma32(av, zl[j], p.v[cb]);
        }
    }
    return p;
  };
  auto tile = [&](auto M_) {
    constexpr int m = decltype(M_)::value;
    const int T = tt0 + kT32MT * wm + m;
    if (T >= G.ntiles) return;
    const Acc4 pc = low_rank_part(T, 0, csteps);
    const Acc4 pw = low_rank_part(T, csteps, esteps);
#pragma unroll
    for (int cb = 0; cb < kT32WCB; ++cb) store(m, cb, acc[m][cb], pc.v[cb], pw.v[cb]);
  };
  static_for<0, kT32MT>(tile);
  finish_stats();
}

#undef T32_SLOT

// Y of the split tiles: the sum of each tile's sp.s partial tiles in part
// order, in the output format.  Workgroup w takes token rows 4 (w % (8 TT))
// .. + 3 of split tile w / (8 TT); thread t takes 4 consecutive vocabulary
// rows of one of them, and issues the loads of up to 8 parts at once.
// ST: statistics pieces instead (each wave takes one token row, so its 64
// lanes hold the tile's 256 logits of that token).
template <int TT, bool ST>
__global__ __launch_bounds__(256) void t32_reduce_kernel(const FwdArgs a, const T32Split sp) {
  constexpr int kRows = kT32CB * 32;       // vocabulary rows per tile
  constexpr int kTileF = TT * 32 * kRows;  // floats per partial tile
  constexpr int kBatch = 8;                // parts loaded together
  const T32Grid G = t32_grid(a, TT);
  const int j = blockIdx.x / (8 * TT), t = 4 * (blockIdx.x % (8 * TT)) + (threadIdx.x >> 6);
  int vt, ttile;
  t32_tile(G, sp.full + j, vt, ttile);
  const int c = 4 * (threadIdx.x & 63);
  const int64_t voc = (int64_t)vt * kRows + c, tok = 32 * (int64_t)ttile * TT + t;
  if constexpr (!ST) {
    if (voc >= a.V || tok >= a.N) return;
  } else {
    if (tok >= a.N) return;  // a whole wave: the token is uniform
  }
  const float* src = a.part + (size_t)j * sp.s * kTileF + t * kRows + c;
  f4 y = f4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < sp.s; p0 += kBatch) {
    f4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = p0 + i < sp.s ? p0 + i : sp.s - 1;
      v[i] = *reinterpret_cast<const f4*>(src + (size_t)p * kTileF);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (p0 + i < sp.s) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] += v[i][e];
      }
  }
  if constexpr (ST) {
    RowStat r = stat_empty();
    const int tgt = a.targets ? a.targets[tok] : -1;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (voc + e < a.V) stat_add(r, y[e], (int)(voc + e), tgt);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) r = stat_merge(r, stat_shfl_xor(r, off));
    if ((threadIdx.x & 63) == 0) reinterpret_cast<f4*>(a.st_part)[tok * a.st_nparts + vt] = stat_pack(r);
    return;
  }
  const int64_t o = tok * a.Y_stride + voc;
  if (((uintptr_t)a.Y & 15) == 0 && (a.Y_stride & 3) == 0 && voc + 3 < a.V) {
    if (a.y_bf16)
      *reinterpret_cast<u2*>(reinterpret_cast<uint16_t*>(a.Y) + o) = pack_bf16x4(y[0], y[1], y[2], y[3]);
    else
      *reinterpret_cast<f4*>(reinterpret_cast<float*>(a.Y) + o) = y;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (voc + e < a.V) {
        if (a.y_bf16)
          reinterpret_cast<uint16_t*>(a.Y)[o + e] = f32_to_bf16(y[e]);
        else
          reinterpret_cast<float*>(a.Y)[o + e] = y[e];
      }
    }
  }
}

// Token tiles per workgroup: 64 tokens for N <= 64, 128 for N <= 128, else
// 256.  The two smaller sizes run 128-column stages, which need at least two
// k-tiles (D >= 256).
inline int t32_tt(const FwdArgs& a) { return a.D < 256 ? 8 : a.N <= 64 ? 2 : a.N <= 128 ? 4 : 8; }

// Workgroups of one kernel instance resident at once on the current device
// (0 if unknown).
static int t32_slots(const void* kernel, size_t lds) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kT32Threads, lds) != hipSuccess)
    return 0;
  return cus > 0 && per_cu > 0 ? cus * per_cu : 0;
}

// Whole tiles fill whole rounds of resident workgroups; the tiles of a last,
// partly filled round are split over the hidden dimension into as many parts
// as that round has room for (at most a quarter of the stages, so every part
// has at least four, and as many as the workspace holds).
template <int TT>
static T32Split t32_split(const FwdArgs& a, int tiles, int slots) {
  const int rem = slots > 0 ? tiles % slots : 0;
  if (rem == 0 || !a.part) return T32Split{tiles, 1};
  const uint64_t tile_bytes = (uint64_t)TT * 32 * kT32CB * 32 * 4;
  int64_t s = slots / rem;
  s = std::min<int64_t>(s, a.D / (16 * t32_ks(TT)) / 4);
  s = std::min<int64_t>(s, (int64_t)(a.part_bytes / tile_bytes / (uint64_t)rem));
  if (s < 2) return T32Split{tiles, 1};
  return T32Split{tiles - rem, (int)s};
}

template <int GC, int TT, bool ST>
static hipError_t launch_t32_g(const FwdArgs& a, hipStream_t s) {
  const T32Grid G = t32_grid(a, TT);
  const int tiles = G.ttiles * G.vtiles;
  const size_t codes = (size_t)kT32CB * 32 * t32_code_stride(a.ng);  // dynamic LDS: the group-code table
  const T32Split sp = t32_split<TT>(a, tiles, t32_slots((const void*)&tile32_kernel<GC, TT, ST>, codes));
  const int nsplit = tiles - sp.full;
  const dim3 grid((unsigned)(sp.full + nsplit * sp.s)), block(kT32Threads);
  const bool reduce = nsplit > 0 && sp.s > 1;
  const hipError_t e = launch_main(tile32_kernel<GC, TT, ST>, grid, block, (uint32_t)codes, s, !reduce, a, sp);
  if (e != hipSuccess || !reduce) return e;
  return launch_main(t32_reduce_kernel<TT, ST>, dim3(nsplit * 8 * TT), dim3(256), 0u, s, true, a, sp);
}

template <int TT, bool ST>
static hipError_t launch_t32(const FwdArgs& a, hipStream_t s) {
  if (a.g == 32) return launch_t32_g<2, TT, ST>(a, s);
  if (a.g == 64) return launch_t32_g<1, TT, ST>(a, s);
  return launch_t32_g<0, TT, ST>(a, s);
}

}  // namespace

}  // namespace archead
