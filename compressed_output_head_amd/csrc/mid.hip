// Batched-decode kernel (up to 64 tokens): one persistent workgroup per CU.
//
// Y = [H | Z] [R | A_c ; A_w]^T (Algorithm 1's inference step with the
// quantised core evaluated through the same (H B^T) A^T association), for
// token counts too large to keep H in LDS and too small to fill the large-N
// tiles.  The packed head is read from HBM exactly once.
//
// The vocabulary is cut into groups of four 32-row blocks; each workgroup walks
// its groups, one block per wave.  A group is a stream of stages: one stage per
// 256 columns (two k-tiles) of the residual, then one per 128 ranks of the
// low-rank term.  Every stage moves
//   - the operand fragments of all token tiles (H for a residual stage, Z hi/lo
//     for a low-rank stage; 32-row layout from the prep kernel) into an LDS
//     ring slot by buffer loads straight into LDS, shared by the four waves;
//   - this wave's packed codes (INT4 residual codes and their group codes, or
//     INT8 A codes and the row's A scales) plus the row scale into a register
//     ring slot.
// Both rings have four slots and run kMidDist = 3 stages ahead across group
// boundaries, so about 12 KB per wave are in flight from HBM.  The two streams
// share one prefetch distance because vector-memory loads complete in order:
// waiting for a near load would also wait for every older far one.
// Accumulation is v_mfma_f32_32x32x16_f16 on exact integer operands (q4 * c8,
// INT8 A codes) with fp32 accumulators, one set per part; the scales are
// applied when a group's last stage is done.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace archead {

namespace {

constexpr int kMidThreads = 256;
constexpr int kMidDist = 3;      // stages of prefetch; both rings have 4 slots
constexpr int kMidWOps = 7;      // code-side loads per wave and stage
constexpr int kMidMaxTiles = 2;  // token tiles of 32 (the LDS ring is sized for the most)

// s_waitcnt immediate: wait until at most n vector-memory operations of this
// wave are outstanding (expcnt and lgkmcnt not waited on)
__device__ constexpr int mid_waitcnt(int n) { return 0x0F70 | (n & 0xF) | (((n >> 4) & 3) << 14); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mid_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

struct MidGeom {
  int nb, ncb, ngroups, nkt, rst, esteps, csteps, lrst, glen;
};
__host__ __device__ inline MidGeom mid_geom(const FwdArgs& a) {
  MidGeom m;
  m.nb = (int)a.nb;
  m.ncb = (m.nb + 1) / 2;
  m.ngroups = (m.ncb + 3) / 4;
  m.nkt = a.nkt;
  m.rst = (m.nkt + 1) / 2;            // residual stages of two k-tiles
  m.esteps = (a.rc32 + a.rr32) / 16;  // 16-rank MFMA steps (even)
  m.csteps = a.rc32 / 16;
  m.lrst = (m.esteps + 7) / 8;        // low-rank stages of 8 steps
  m.glen = m.rst + m.lrst;            // stages per group
  return m;
}

// One slot of the code ring: four 16-byte quarters (residual: this lane's
// packed nibbles of both halves of two k-tiles; low rank: A codes of four step
// pairs), two words of group codes (one per k-tile) or of A scales (c, w), and
// the row scale.
struct WSlot {
  u4 w[4];
  uint32_t x0, x1;
  uint32_t sr;
  uint32_t mask;  // low rank: bit 2 h + e set when half e of quarter h holds real ranks
};

template <int NT, int GC>
__global__ __launch_bounds__(kMidThreads) void mid_kernel(const FwdArgs a) {
  // ring slots: token tile, 16 fragments of 1 KB (one per MFMA step, or per
  // step and hi/lo half)
  __shared__ h8 ring0[kMidMaxTiles][16][64], ring1[kMidMaxTiles][16][64];
  __shared__ h8 ring2[kMidMaxTiles][16][64], ring3[kMidMaxTiles][16][64];
  __shared__ float sTok[kMidMaxTiles * 32][2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const MidGeom M = mid_geom(a);
  const int niters = (M.ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int total = niters * M.glen;  // stages of this workgroup's stream
  const int r = a.r_c + a.r_r;

  // token scales, published by the first barrier (rows up to n32 exist)
  if (tid < NT * 32) {
    sTok[tid][0] = a.hscale[tid];
    sTok[tid][1] = a.zscale[tid];
  }

  // one buffer resource per allocation: the workspace (hf, then zf) and the
  // packed head (sections addressed from r_codes, which comes first)
  const uint32_t zoff = (uint32_t)((const char*)a.zf - (const char*)a.hf);
  const __amdgpu_buffer_rsrc_t wsr = mid_rsrc(a.hf, zoff + (uint32_t)(a.n32 * (a.rc32 + a.rr32) * 4));
  const char* pk = (const char*)a.r_codes;
  const uint32_t o_gc = (uint32_t)((const char*)a.r_gcodes - pk);
  const uint32_t o_rs = (uint32_t)((const char*)a.r_rowscale - pk);
  const uint32_t o_ac = (uint32_t)((const char*)a.a_codes - pk);
  const uint32_t o_as = (uint32_t)((const char*)a.a_scales - pk);
  const __amdgpu_buffer_rsrc_t pkr = mid_rsrc(pk, o_as + (uint32_t)(a.nb * 16 * (a.nA > 0 ? a.nA : 1) * 2));
  const uint32_t lane16 = (uint32_t)lane * 16u;
  const int lg = __builtin_ctz((unsigned)a.g);

  // the lane's 16-row block in the k-th group: block 2 cb + (lane / 16) % 2,
  // whose row lane % 16 is vocabulary row 32 cb + lane % 32 (clamped)
  auto lane_block = [&](int k) __attribute__((always_inline)) {
    int cb = 4 * ((int)blockIdx.x + k * (int)gridDim.x) + wave;
    if (cb >= M.ncb) cb = M.ncb - 1;
    int b = 2 * cb + ((lane >> 4) & 1);
    if (b >= M.nb) b = M.nb - 1;
    return b;
  };

  // ---- the loads of stage j of the k-th group
  auto issue_h = [&](int j, h8 (&dst)[kMidMaxTiles][16][64]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4 * NT; ++i) {
      const int f = wave + 4 * i;  // fragment: token tile f / 16, position f % 16
      const int T = f >> 4, t = f & 15;
      uint32_t off;
      if (j < M.rst) {
        int kt = 2 * j + (t >> 3);
        if (kt >= M.nkt) kt = M.nkt - 1;  // odd k-tile count: its codes are zero
        off = (uint32_t)((T * M.nkt + kt) * 8 + (t & 7)) * 1024u;
      } else {
        const int e = 16 * (j - M.rst) + t;  // step e / 2, hi/lo e % 2
        off = zoff + (uint32_t)(T * 2 * M.esteps + (e < 2 * M.esteps ? e : 2 * M.esteps - 1)) * 1024u;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wsr, &dst[T][t][0], 16, lane16, off, 0, 0);
    }
  };
  auto issue_w = [&](int k, int j, WSlot& ws) __attribute__((always_inline)) {
    const int b = lane_block(k);
    const uint32_t row = (uint32_t)b * 16u + (uint32_t)(lane & 15);
    if (j < M.rst) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kt = 2 * j + h < M.nkt ? 2 * j + h : M.nkt - 1;
        const uint32_t off = ((uint32_t)kt * (uint32_t)M.nb + (uint32_t)b) * 1024u + (uint32_t)(lane & 15) * 16u +
                             (uint32_t)g * 256u;
        // (a k-tile past an odd count is loaded again and skipped when used)
        ws.w[2 * h] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(pkr, off, 0, 0));
        ws.w[2 * h + 1] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(pkr, off + 512u, 0, 0));
        // group codes of k-tile kt: 4 bytes (g = 32), 2 (g = 64), 1 (g >= 128)
        const uint32_t cbase = o_gc + row * (uint32_t)a.ng;
        uint32_t x;
        if constexpr (GC == 2)
          x = __builtin_amdgcn_raw_buffer_load_b32(pkr, cbase + 4u * (uint32_t)kt, 0, 0);
        else if constexpr (GC == 1)
          x = __builtin_amdgcn_raw_buffer_load_b16(pkr, cbase + 2u * (uint32_t)kt, 0, 0);
        else
          x = __builtin_amdgcn_raw_buffer_load_b8(pkr, cbase + ((uint32_t)(kKTile * kt) >> lg), 0, 0);
        if (h == 0)
          ws.x0 = x;
        else
          ws.x1 = x;
      }
    } else {
      // A codes of step pairs 4 lb .. 4 lb + 3: 16 bytes at rank
      // 32 (pair within its part) + 16 (lane / 32) of the part.  Which 8-byte
      // halves hold real ranks goes to a mask applied when the codes are used,
      // so nothing here waits for a load.
      const int lb = j - M.rst;
      uint32_t mask = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int P = 4 * lb + h;
        const bool part_c = 2 * P < M.csteps;
        const int col = 32 * (part_c ? P : P - M.csteps / 2) + 16 * g;
        const int rank = part_c ? a.r_c : a.r_r;
        const int base = part_c ? 0 : a.r_c;
        const bool live = 2 * P < M.esteps && col < rank;
        if (live) mask |= (col + 8 < rank ? 3u : 1u) << (2 * h);
        const uint32_t off = o_ac + row * (uint32_t)r + (uint32_t)(live ? base + col : 0);
        ws.w[h] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(pkr, off, 0, 0));
      }
      ws.mask = mask;
      // the row's A scales: part c first, part w last (one scale when a part is empty)
      const uint32_t as = o_as + row * (uint32_t)a.nA * 2u;
      ws.x0 = __builtin_amdgcn_raw_buffer_load_b16(pkr, as, 0, 0);
      ws.x1 = __builtin_amdgcn_raw_buffer_load_b16(pkr, as + 2u * (uint32_t)(a.nA - 1), 0, 0);
    }
    ws.sr = __builtin_amdgcn_raw_buffer_load_b16(pkr, o_rs + row * 2u, 0, 0);
  };

  f16x acc[NT], pc[NT], pw[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    acc[m] = f16x{};
    pc[m] = f16x{};
    pw[m] = f16x{};
  }
  WSlot wr[4];
  uint32_t keep_sr = 0, keep_ac = 0, keep_aw = 0;

  // stream position of the next stage to issue; past the end the last stage is
  // issued again (nothing reads it) so every stage issues the same loads
  const int last_k = (total - 1) / M.glen, last_j = (total - 1) - last_k * M.glen;
  int pos = 0, pk_ = 0, pj = 0;
  auto issue_stage = [&](h8 (&dst)[kMidMaxTiles][16][64], WSlot& ws) __attribute__((always_inline)) {
    const int k = pos < total ? pk_ : last_k, j = pos < total ? pj : last_j;
    issue_h(j, dst);
    issue_w(k, j, ws);
    ++pos;
    if (++pj == M.glen) {
      pj = 0;
      ++pk_;
    }
  };

  // prologue: stages 0 .. kMidDist-1
  issue_stage(ring0, wr[0]);
  issue_stage(ring1, wr[1]);
  issue_stage(ring2, wr[2]);

  int ck = 0, cj = 0;  // stage being computed

  // Y through a buffer resource: per element a per-lane offset (this lane's
  // column and token half) plus a wave-uniform one (token row), so no 64-bit
  // address per element stays live across the stream
  const uint32_t es = a.y_bf16 ? 2u : 4u;
  const uint32_t ystride = (uint32_t)a.Y_stride * es;  // bytes per token row
  const __amdgpu_buffer_rsrc_t yrs = mid_rsrc(a.Y, (uint32_t)a.N * ystride);
  auto epilogue = [&]() __attribute__((always_inline)) {
    const int cb = 4 * ((int)blockIdx.x + ck * (int)gridDim.x) + wave;
    const int voc = 32 * cb + c32;
    const bool col_ok = cb < M.ncb && voc < a.V;
    const float sR = f16_to_f32((uint16_t)keep_sr);
    const float sAc = a.r_c > 0 ? f16_to_f32((uint16_t)keep_ac) : 0.0f;
    const float sAw = a.r_r > 0 ? f16_to_f32((uint16_t)keep_aw) : 0.0f;
    const uint32_t lane_off = (uint32_t)(4 * g) * ystride + (uint32_t)voc * es;
#pragma unroll
    for (int m = 0; m < NT; ++m) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t0 = 32 * m + 8 * (v >> 2) + (v & 3);  // token of lanes 0..31 (lanes 32..63: + 4)
        const int tok = t0 + 4 * g;
        if (col_ok && tok < a.N) {
          float y = sTok[tok][0] * (sR * acc[m][v]);
          if (r > 0) y = fmaf(sTok[tok][1], fmaf(sAw, pw[m][v], sAc * pc[m][v]), y);
          const uint32_t soff = (uint32_t)t0 * ystride;
          if (a.y_bf16)
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(y), yrs, lane_off, soff, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), yrs, lane_off, soff, 0);
        }
      }
      acc[m] = f16x{};
      pc[m] = f16x{};
      pw[m] = f16x{};
    }
  };

  // One stage; S = stream position mod 4 picks the ring slots at compile time.
  // On entry this wave has in flight the copies and loads of stages
  // s .. s + kMidDist - 1, oldest first; waiting down to the newest
  // kMidDist - 1 stages completes stage s.  The barrier publishes every wave's
  // copies of stage s and retires all reads of slot (s - 1) mod 4, which the
  // loads for stage s + kMidDist then refill (its registers were consumed by
  // stage s - 1 as well).
  auto stage = [&](auto S_) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value, Q = (S + kMidDist) & 3;
    h8(&cur)[kMidMaxTiles][16][64] = S == 0 ? ring0 : S == 1 ? ring1 : S == 2 ? ring2 : ring3;
    h8(&nxt)[kMidMaxTiles][16][64] = Q == 0 ? ring0 : Q == 1 ? ring1 : Q == 2 ? ring2 : ring3;
    __builtin_amdgcn_s_waitcnt(mid_waitcnt((kMidDist - 1) * (4 * NT + kMidWOps)));
    __syncthreads();
    issue_stage(nxt, wr[Q]);
    const WSlot& w = wr[S];
    keep_sr = w.sr;
    if (cj < M.rst) {
      // residual k-tiles 2 cj + h: step t covers runs R = 4 (t % 4) + 2 (t / 4) + lane / 32
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // a k-tile past an odd count gets group code 0, so it adds exact zeros
        // (branching around it would make the accumulators change registers)
        const uint32_t codes = 2 * cj + h < M.nkt ? (h == 0 ? w.x0 : w.x1) : 0u;
        h8 bv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t code = GC == 2 ? (codes >> (8 * (t & 3))) & 0xffu
                              : GC == 1 ? (codes >> (8 * ((t & 3) >> 1))) & 0xffu
                                        : codes & 0xffu;
          bv[t] = unpack_q4_scaled(w.w[2 * h + (t >> 2)][t & 3], (_Float16)(float)code);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int m = 0; m < NT; ++m) acc[m] = mfma32(cur[m][8 * h + t][lane], bv[t], acc[m]);
      }
    } else {
      // low rank: step 8 lb + i, Z hi at fragment 2 i, lo at 2 i + 1
      const int lb = cj - M.rst;
      keep_ac = w.x0;
      keep_aw = w.x1;
      // every step feeds both parts, with the other part's codes zeroed:
      // branching per step would make the accumulators change registers
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u4 pr = w.w[i >> 1];
        const bool on = (w.mask >> i) & 1u;  // bit 2 (i / 2) + i % 2
        const bool in_c = 8 * lb + i < M.csteps;
        const uint32_t lo = on ? pr[2 * (i & 1)] : 0u, hi = on ? pr[2 * (i & 1) + 1] : 0u;
        const h8 bc = unpack_i8x8(in_c ? lo : 0u, in_c ? hi : 0u);
        const h8 bw = unpack_i8x8(in_c ? 0u : lo, in_c ? 0u : hi);
#pragma unroll
        for (int m = 0; m < NT; ++m) {
          const h8 zh = cur[m][2 * i][lane], zl = cur[m][2 * i + 1][lane];
          pc[m] = mfma32(zh, bc, pc[m]);
          pw[m] = mfma32(zh, bw, pw[m]);
          pc[m] = mfma32(zl, bc, pc[m]);
          pw[m] = mfma32(zl, bw, pw[m]);
        }
      }
    }
    if (cj == M.glen - 1) epilogue();
    if (++cj == M.glen) {
      cj = 0;
      ++ck;
    }
  };

  for (int s0 = 0; s0 < total; s0 += 4) {
    stage(std::integral_constant<int, 0>{});
    if (s0 + 1 < total) stage(std::integral_constant<int, 1>{});
    if (s0 + 2 < total) stage(std::integral_constant<int, 2>{});
    if (s0 + 3 < total) stage(std::integral_constant<int, 3>{});
  }
  __builtin_amdgcn_s_waitcnt(0);  // the repeated prefetches past the end land before exit
}

template <int NT>
hipError_t launch_mid_nt(const FwdArgs& a, hipStream_t s, int grid) {
  if (a.g == 32)
    hipLaunchKernelGGL((mid_kernel<NT, 2>), dim3(grid), dim3(kMidThreads), 0, s, a);
  else if (a.g == 64)
    hipLaunchKernelGGL((mid_kernel<NT, 1>), dim3(grid), dim3(kMidThreads), 0, s, a);
  else
    hipLaunchKernelGGL((mid_kernel<NT, 0>), dim3(grid), dim3(kMidThreads), 0, s, a);
  return hipGetLastError();
}

// CUs of the current device (256 if the runtime cannot tell)
int mid_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

}  // namespace

// 1..64 tokens, with every section the kernel reads or writes within 32-bit
// offsets of the start of its allocation.
bool mid_eligible(const FwdArgs& a) {
  if (a.N < 1 || a.N > 32 * kMidMaxTiles) return false;
  if ((uint64_t)a.N * (uint64_t)a.Y_stride * (a.y_bf16 ? 2 : 4) >= (1ull << 31)) return false;
  const uint64_t pk_span = (uint64_t)((const char*)a.a_scales - (const char*)a.r_codes) +
                           (uint64_t)a.nb * 16 * (uint64_t)(a.nA > 0 ? a.nA : 1) * 2;
  const uint64_t ws_span = (uint64_t)((const char*)a.zf - (const char*)a.hf) +
                           (uint64_t)a.n32 * (uint64_t)(a.rc32 + a.rr32) * 4;
  return pk_span < (1ull << 32) && ws_span < (1ull << 32);
}

hipError_t launch_mid(const FwdArgs& a, hipStream_t s) {
  const MidGeom M = mid_geom(a);
  const int grid = M.ngroups < mid_cu_count() ? M.ngroups : mid_cu_count();
  if (grid <= 0) return hipSuccess;
  return a.N <= 32 ? launch_mid_nt<1>(a, s, grid) : launch_mid_nt<2>(a, s, grid);
}

}  // namespace archead
