// Batched decode path (17 to 64 tokens): the few-token pre-projection kernel
// (H rows as scaled fp16 in kernel k-order, Z in fp32), then one kernel that
// streams the packed head once for all the tokens.
//
// Y = H W_d^T + (H B_w^T) A_w^T (Algorithm 1, inference step) with
// W_d = Q(A_c)Q(B_c) + SC4(R) (Sec. 3, quantized-core equation); the core is
// evaluated through the same association, (H B_c^T) A_c^T.
//
// Main kernel: one workgroup of 8 waves per CU.  The 16-row vocabulary blocks
// are split into one contiguous range per workgroup and evenly over its waves
// (at most MM blocks a wave).  Every wave keeps the accumulators of all its
// blocks and all T = ceil(N/16) token tiles for the whole hidden dimension and
// walks the k-tiles in order, each workgroup from its own starting k-tile
// (wrapping around): tiles are stored k-tile major, so a workgroup reads one
// contiguous run of about 37 KB per k-tile.
//   W: each wave keeps K k-tiles of its own packed tiles in flight in a
//     register ring; a stage multiplies one k-tile and then refills its slot.
//   H: the workgroup's T x 4 KB of fp16 operand fragments per k-tile, copied
//     straight from the converted rows into two LDS halves of HK k-tiles by
//     buffer-to-LDS loads; all waves meet once every HK k-tiles, when the
//     half just finished is refilled.
//   Group codes: the workgroup's rows of codes are copied to LDS once; each
//     k-tile, a lane reads the dword with its row's codes of that k-tile.
// Per 32-column step and block: the INT4 codes unpacked once to the exact
// fp16 integers q4 * c8 (|q4 c8| <= 2040), then one v_mfma_f32_16x16x32_f16
// per token tile against H.
//
// Epilogue per block: Z hi/lo (fp16, 22 significant bits, one power-of-two
// scale per token) against the exact INT8 A codes, one accumulator per part,
// then the fp16 row scale s_R and the token scales.  No atomics on results:
// every run gives the same bits.
//
// The same kernel streams the two storage-matched comparison heads (ARCHead,
// results discussion of Tables 7 and 8), which have no low-rank term:
//   group INT4: the INT4 tiles as above; the exact codes go through the MFMAs
//     of one group into a fresh accumulator, which is then added to the
//     result times the group's fp16 scale (the scales of the workgroup's rows
//     sit in LDS where the group codes would);
//   row INT8: 2 KB tiles (two 16-byte loads per lane and tile), the exact
//     INT8 codes as fp16 operands, the fp16 row scale in the epilogue.
#pragma once

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace archead {

namespace {

constexpr int kBWaves = 8;
constexpr int kBThreads = 64 * kBWaves;
constexpr int kBMaxTiles = 4;    // 16-token tiles (N <= 64)
constexpr int kBMaxSteps = 4;    // 32-rank steps of the low-rank term: rc32 + rr32 <= 128
constexpr int kBMaxBlocks = 5;   // blocks per wave (the accumulators stay in registers)
constexpr int kBMaxBlocks2 = 3;  // ... with two workgroups per CU
constexpr int kBMaxGroups = 64;  // group codes per row (D/g)
constexpr int kNonTemporal = 2;  // cache policy of the packed tiles: streamed once

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// This wave's vector-memory operations up to the last n and all its LDS
// accesses are complete, then every wave meets.  Buffer-to-LDS copies land
// when their vmcnt retires, so after the barrier every wave's copies are
// visible.  No fence (it would wait for every load in flight).
template <int n>
__device__ __forceinline__ void ring_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt has six bits");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | (n & 0xF) | (((n >> 4) & 3) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// This wave's vector-memory operations up to the last n and all its LDS
// accesses are complete (no barrier).
template <int n>
__device__ __forceinline__ void vm_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt has six bits");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | (n & 0xF) | (((n >> 4) & 3) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One 16-byte buffer-to-LDS copy per lane (lane l writes dst + 16 l).  Not
// inlined into the kernel template by hand: called there directly, the
// builtin keeps the host pass from emitting the template's launch stub.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rs, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 0);
}

// Wait states after the last MFMA of a chain whose results are copied or
// read by VALU instructions in another basic block: the compiler does not
// always count the MFMA result latency across a branch (seen as a copy of the
// first two result registers right after the MFMA), so 24 are inserted by
// hand, more than the longest 16x16x32 MFMA needs.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}

// LDS row stride of the group codes: an odd number of dwords, so the 16 rows
// a wave reads at once fall in 16 different banks
__host__ __device__ constexpr uint32_t bcode_stride(int ng) { return 4u * (uint32_t)(((ng + 3) / 4) | 1); }

// Dynamic LDS: the workgroup's group codes [rows][stride], Z hi/lo fragments
// [steps][hi, lo][T][64 lanes], per token its H and Z scales.
struct BLds {
  uint32_t codes;  // group codes
  uint32_t zf;     // Z fragments
  uint32_t tok;    // float [64][2]: hscale, zscale
  uint32_t total;
};

__host__ __device__ inline BLds batch_lds(int T, int esteps, int rows, int ng) {
  BLds L;
  L.codes = 0;
  L.zf = ((uint32_t)rows * bcode_stride(ng) + 15u) & ~15u;
  L.tok = L.zf + (uint32_t)esteps * 2u * (uint32_t)T * 1024u;
  L.total = L.tok + 64u * 2u * 4u;
  return L;
}

#define B_HALF(X) (*((X) == 0 ? &sHa : &sHb))

// Bytes of one row's group codes (ARCHead) or group scales (group INT4) in
// LDS; the row-INT8 head keeps nothing there.
__host__ __device__ constexpr int bcode_row_bytes(int fmt, int ng) {
  return fmt == ARCHEAD_FMT_ARCHEAD ? ng : fmt == ARCHEAD_FMT_GROUP_INT4 ? 2 * ng : 0;
}

// FMT: storage format (archead_format); T: token tiles of 16; MM: blocks per
// wave; CPT: groups per k-tile (1: g >= 128, 2: g = 64, 4: g = 32); HK:
// k-tiles per half of the H ring; K: k-tiles of packed tiles in flight per
// wave; OCC: workgroups per CU.
template <int FMT, int T, int MM, int CPT, int HK, int K, int OCC>
__global__ __launch_bounds__(kBThreads, OCC) void batch_kernel(const FwdArgs a, const BLds L) {
  constexpr int NF = 4 * T;                               // 1 KB H fragments per k-tile: (token tile, step)
  constexpr int NHH = (HK * NF + kBWaves - 1) / kBWaves;  // H copies per wave and half
  constexpr int WV = FMT == ARCHEAD_FMT_ROW_INT8 ? 2 : 1;  // 16-byte loads per lane and packed tile
  constexpr uint32_t TB = 1024u * WV;                      // bytes per packed tile
  static_assert((2 * HK) % K == 0 && K <= HK, "the unrolled loop turns both rings a whole number of times");
  __shared__ __align__(16) h8 sHa[HK][NF][64], sHb[HK][NF][64];
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = (int)a.N, D = (int)a.D;
  const int r = a.r_c + a.r_r, G = a.g;
  const int nkt = a.nkt, ng = a.ng;
  const int i16 = lane & 15, q = lane >> 4;
  const int cbytes_row = bcode_row_bytes(FMT, ng);
  const uint32_t cstride = bcode_stride(cbytes_row);
  unsigned char* sCode = smem + L.codes;
  h8* sZf = reinterpret_cast<h8*>(smem + L.zf);
  float* sTok = reinterpret_cast<float*>(smem + L.tok);

  // this wave's blocks [bw0, bw0 + Mw): the workgroup's range, evenly split
  const int B0 = (int)((int64_t)blockIdx.x * a.nb / gridDim.x);
  const int cnt = (int)((int64_t)(blockIdx.x + 1) * a.nb / gridDim.x) - B0;
  const int bw0 = B0 + cnt * wave / kBWaves;
  const int Mw = B0 + cnt * (wave + 1) / kBWaves - bw0;

  // Workgroups start their walk at different k-tiles (rot) and wrap around:
  // all workgroups read the same converted rows of H, and in step they would
  // all hit the same few cache lines at once.
  const int rot = (int)((int64_t)blockIdx.x * nkt / gridDim.x);
  auto ktile = [&](int ks) {
    ks = ks < nkt ? ks : nkt - 1;  // stages past the end re-read the last k-tile (cache hits, never used)
    return ks + rot < nkt ? ks + rot : ks + rot - nkt;
  };

  // ---- H: two halves of HK k-tiles in LDS ------------------------------------------
  // H fragment f = 4 t + s of a k-tile ks: lane l reads token 16 t + l%16
  // (rows past N repeat row N - 1 and are never stored), columns 128 ks + 32 s +
  // 8 (l/16) .. +8 of the converted rows.  A half's HK NF fragments are dealt to
  // the waves, NHH each (clamped: extra copies rewrite the last fragment).
  // Offsets are fixed per lane and the k-tile goes into the uniform offset:
  // issuing takes no vector instruction (a vector temporary for an address
  // can land on a register of a load still in flight and make the issue wait
  // for every load).
  const uint32_t hbytes = (uint32_t)N * (uint32_t)D * 2u;
  const __amdgpu_buffer_rsrc_t hrs = buffer_rsrc(a.hc, hbytes);
  uint32_t hvo[NHH];
  int hslot[NHH], hfr[NHH];
#pragma unroll
  for (int i = 0; i < NHH; ++i) {
    const int f = min(wave * NHH + i, HK * NF - 1);
    const int j = f / NF, ff = f - j * NF;
    const int t = ff >> 2, s = ff & 3;
    const int row = min(16 * t + i16, N - 1);
    hslot[i] = j;
    hfr[i] = ff;
    hvo[i] = ((uint32_t)row * (uint32_t)D + 32u * (uint32_t)s + 8u * (uint32_t)q) * 2u;
  }
  // the k-tiles ks0 .. ks0 + HK - 1 into half X
  auto issue_h = [&](auto X_, int ks0) {
    constexpr int X = decltype(X_)::value;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NHH; ++i) {
      const uint32_t kc = (uint32_t)__builtin_amdgcn_readfirstlane(ktile(ks0 + hslot[i]));
      lds_copy16(hrs, &B_HALF(X)[hslot[i]][hfr[i]][0], hvo[i], kc * 256u);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- W: a ring of K k-tiles of this wave's packed tiles in registers -------------
  // tile (b, kt) at (kt*nb + b)*TB, lane l's bytes at TB/64 l; slots past a
  // wave's blocks re-read its first block (cache hits; their results are never
  // stored), so every stage issues the same loads and each wait counts exactly.
  const uint32_t tstride = (uint32_t)a.nb * TB;
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(a.r_codes, tstride * (uint32_t)nkt);
  const uint32_t wlane = (uint32_t)lane * 16u * WV;
  uint32_t wblk[MM];  // wave-uniform byte offset of each block's tile within a k-tile
#pragma unroll
  for (int m = 0; m < MM; ++m)
    wblk[m] = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bw0 + (m < Mw ? m : 0)) * TB);
  u4 wr[K][MM][WV];
  // Stages past the end of the walk (never used) all read the last k-tile of
  // the head's last block: the same lines for every wave, cache hits after the
  // first.  The wave's own last k-tile, streamed a stage earlier without
  // staying in the cache, would come from memory again.
  const uint32_t wpast = (uint32_t)(nkt - 1) * tstride + (uint32_t)(a.nb - 1) * TB;
  auto issue_w = [&](auto J_, int ks) {
    constexpr int J = decltype(J_)::value;
    const bool past = ks >= nkt;  // wave-uniform
    const uint32_t kc = (uint32_t)__builtin_amdgcn_readfirstlane(ktile(ks));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
      for (int v = 0; v < WV; ++v)
        wr[J][m][v] = __builtin_bit_cast(
            u4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wlane, (past ? wpast : kc * tstride + wblk[m]) + 16u * v,
                                                      kNonTemporal));
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: the workgroup's group codes (or group scales) into LDS -------------
  // rows [16 B0, 16 (B0 + cnt)), cbytes_row bytes each, contiguous in the
  // packed buffer: 16-byte loads, each byte to its row's padded place
  if constexpr (FMT != ARCHEAD_FMT_ROW_INT8) {
    const uint32_t rb = (uint32_t)cbytes_row;
    const uint32_t cbytes = (uint32_t)cnt * 16u * rb;
    const __amdgpu_buffer_rsrc_t crs = buffer_rsrc(a.r_gcodes, (uint32_t)a.nb * 16u * rb);
    const uint32_t cbase = (uint32_t)B0 * 16u * rb;
    for (uint32_t o = 16u * (uint32_t)tid; o < cbytes; o += 16u * kBThreads) {
      const u4 v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(crs, cbase + o, 0, 0));
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const uint32_t ob = o + (uint32_t)b;
        if (ob < cbytes) {
          const uint32_t row = ob / rb, col = ob - row * rb;
          sCode[row * cstride + col] = (unsigned char)((v[b >> 2] >> (8 * (b & 3))) & 0xffu);
        }
      }
    }
  }

  // ---- Z hi/lo fragments and the token scales ---------------------------------------
  // token n (wave w takes n = w, w + 8, ..): exponent of its largest |Z|;
  // fragment (step s, part hi/lo, tile t), lane 16 qq + n%16: ranks
  // 32 sl + 8 qq + k_order_z(jj) of the step's part (zero past the part's rank
  // and for rows past N)
  const int csteps = a.rc32 / 32;
  const int esteps = FMT == ARCHEAD_FMT_ARCHEAD ? (a.rc32 + a.rr32) / 32 : 0;
  for (int n = wave; n < 16 * T; n += kBWaves) {
    float m = 0.0f;
    if (n < N)
      for (int k = lane; k < r; k += 64) m = fmaxf(m, fabsf(a.z32[(int64_t)n * r + k]));
    m = wave_max(m);
    const int F = n < N ? row_exponent(m) : 0;
    if (lane == 0) {
      sTok[2 * n] = n < N ? a.hscale[n] : 0.0f;
      sTok[2 * n + 1] = ldexpf(1.0f, -F);
    }
    const int t = n >> 4, nn = n & 15;
    for (int e = lane; e < esteps * 4; e += 64) {
      const int s = e >> 2, qq = e & 3;
      const bool part_c = s < csteps;
      const int sl = part_c ? s : s - csteps;
      const int rank = part_c ? a.r_c : a.r_r, base = part_c ? 0 : a.r_c;
      h8 zh, zl;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int col = 32 * sl + 8 * qq + k_order_z(jj);
        const float z = (n < N && col < rank) ? ldexpf(a.z32[(int64_t)n * r + base + col], F) : 0.0f;
        zh[jj] = (_Float16)z;
        zl[jj] = (_Float16)(z - (float)zh[jj]);
      }
      sZf[((2 * s) * T + t) * 64 + 16 * qq + nn] = zh;
      sZf[((2 * s + 1) * T + t) * 64 + 16 * qq + nn] = zl;
    }
  }

  // the first half of H and K k-tiles of W go in flight (after the
  // prologue's own loads, which it waited for)
  issue_h(std::integral_constant<int, 0>{}, 0);
  static_for<0, K>([&](auto J_) { issue_w(J_, decltype(J_)::value); });
  // The barriers below wait until at most HK stages of W loads are in flight,
  // which are the loads issued after the half they publish.  Here only K
  // stages follow the first half: with K < HK, wait for it now.
  if constexpr (K < HK) vm_wait<K * MM * WV>();

  // ---- main loop: one k-tile per stage ---------------------------------------------
  // Stage s multiplies k-tile ktile(s) (H from half (s / HK) % 2, W from slot
  // s % K), then refills its W slot with stage s + K.  Every HK stages all
  // waves meet: each wave's copies into the half about to be read must have
  // landed (they were issued before the last HK stages of MM WV W loads each;
  // K <= HK), the code rows and Z fragments written above are visible, and
  // the other half (finished, or not yet filled at s = 0) is filled with the
  // stages HK ahead.  The host takes this kernel only when 2 HK divides the
  // k-tile count, so every stage of the unrolled loop runs: with no branch
  // around a stage, the compiler's waits for the packed tiles count exactly.
  f4 acc[MM][T];
  [[maybe_unused]] f4 part[MM][T];  // group INT4: one group's sum before its scale
#pragma unroll
  for (int m = 0; m < MM; ++m)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[m][t] = f4{0.f, 0.f, 0.f, 0.f};
  // this lane's row of each block in the workgroup's code rows (slots past
  // the wave's blocks read its first block, or the workgroup's last one)
  uint32_t crow[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m)
    crow[m] = (uint32_t)(16 * min(bw0 - B0 + (m < Mw ? m : 0), cnt - 1) + i16) * cstride;
  for (int s0 = 0; s0 < nkt; s0 += 2 * HK) {
    static_for<0, 2 * HK>([&](auto U_) {
      constexpr int U = decltype(U_)::value;
      constexpr int X = U / HK, J = U % K, SL = U % HK;
      const int s = s0 + U;
      {
        if constexpr (SL == 0) {
          ring_barrier<HK * MM * WV>();
          issue_h(std::integral_constant<int, 1 - X>{}, s + HK);
        }
        // this k-tile's first group: CPT kr (g = 256: kr / 2)
        const int kr = ktile(s);
        const uint32_t bb = (CPT > 1 || G <= kKTile) ? (uint32_t)(CPT * kr) : (uint32_t)(kr >> 1);
        constexpr int kStepsPerCode = 4 / CPT;
        [[maybe_unused]] _Float16 cf[MM][CPT];
        [[maybe_unused]] float sg[MM][CPT];
        if constexpr (FMT == ARCHEAD_FMT_ARCHEAD) {
          // the lane's row's CPT group codes (consecutive bytes within one
          // dword) as exact fp16 values
          const uint32_t bsh = 8u * (bb & 3u);
          static_for<0, MM>([&](auto M_) {
            constexpr int m = decltype(M_)::value;
            const uint32_t w = *reinterpret_cast<const uint32_t*>(sCode + crow[m] + (bb & ~3u)) >> bsh;
#pragma unroll
            for (int ci = 0; ci < CPT; ++ci) cf[m][ci] = (_Float16)(uint16_t)((w >> (8 * ci)) & 0xffu);
          });
        } else if constexpr (FMT == ARCHEAD_FMT_GROUP_INT4) {
          // the lane's row's CPT fp16 group scales: bytes 2 bb .. 2 bb + 2 CPT
          // (whole dwords for CPT > 1, a half of one for CPT = 1)
          static_for<0, MM>([&](auto M_) {
            constexpr int m = decltype(M_)::value;
            const uint32_t* p = reinterpret_cast<const uint32_t*>(sCode + crow[m] + ((2u * bb) & ~3u));
            if constexpr (CPT == 1) {
              sg[m][0] = f16_to_f32((uint16_t)(p[0] >> (16u * (bb & 1u))));
            } else {
#pragma unroll
              for (int ci = 0; ci < CPT; ci += 2) {
                const uint32_t w = p[ci / 2];
                sg[m][ci] = f16_to_f32((uint16_t)(w & 0xffffu));
                sg[m][ci + 1] = f16_to_f32((uint16_t)(w >> 16));
              }
            }
          });
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          h8 hf[T];
#pragma unroll
          for (int t = 0; t < T; ++t) hf[t] = B_HALF(X)[SL][4 * t + st][lane];
          static_for<0, MM>([&](auto M_) {
            constexpr int m = decltype(M_)::value;
            if constexpr (FMT == ARCHEAD_FMT_ARCHEAD) {
              const h8 w = unpack_q4_scaled(wr[J][m][0][st], cf[m][st / kStepsPerCode]);
#pragma unroll
              for (int t = 0; t < T; ++t) acc[m][t] = mfma16(hf[t], w, acc[m][t]);
            } else if constexpr (FMT == ARCHEAD_FMT_GROUP_INT4) {
              const h8 w = unpack_q4(wr[J][m][0][st]);
              const bool first = st % kStepsPerCode == 0, last = st % kStepsPerCode == kStepsPerCode - 1;
#pragma unroll
              for (int t = 0; t < T; ++t) {
                part[m][t] = mfma16(hf[t], w, first ? f4{0.f, 0.f, 0.f, 0.f} : part[m][t]);
                if (last) {
                  const float sc = sg[m][st / kStepsPerCode];
#pragma unroll
                  for (int e = 0; e < 4; ++e) acc[m][t][e] = fmaf(sc, part[m][t][e], acc[m][t][e]);
                }
              }
            } else {
              // step st: bytes 8 st .. 8 st + 7 of the lane's 32
              const u4& raw = wr[J][m][st >> 1];
              const h8 w = unpack_i8x8(raw[2 * (st & 1)], raw[2 * (st & 1) + 1]);
#pragma unroll
              for (int t = 0; t < T; ++t) acc[m][t] = mfma16(hf[t], w, acc[m][t]);
            }
          });
        }
        issue_w(std::integral_constant<int, J>{}, s + K);
        mfma_drain();
      }
    });
  }

  // ---- epilogue per block: low-rank term, scales, store ---------------------------
  const uint32_t v16 = (uint32_t)a.nb * 16u;
  const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(a.a_codes, v16 * (uint32_t)r);
  const __amdgpu_buffer_rsrc_t rrs = buffer_rsrc(a.r_rowscale, 2u * v16);
  const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(a.a_scales, 2u * v16 * (uint32_t)a.nA);
  const uint32_t ystride = (uint32_t)a.Y_stride;
  const __amdgpu_buffer_rsrc_t yrs =
      buffer_rsrc(a.Y, (uint32_t)((uint64_t)(N - 1) * (uint64_t)a.Y_stride + (uint64_t)a.V) * (a.y_bf16 ? 2u : 4u));
  // every block's operands at once: A codes of the lane's row (8 ranks per
  // step), s_R and the part scales; rows past the wave's blocks read zero
  u2 ac[MM][kBMaxSteps];
  uint32_t sR[MM], sAc[MM], sAw[MM];
  static_for<0, MM>([&](auto M_) {
    constexpr int m = decltype(M_)::value;
    const uint32_t row = (uint32_t)(bw0 + m) * 16u + (uint32_t)i16;
    const bool on = m < Mw;
    if constexpr (FMT != ARCHEAD_FMT_ARCHEAD) {
      // no low-rank term; the group INT4 head has no row scale (1.0)
      sR[m] = FMT == ARCHEAD_FMT_ROW_INT8
                  ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rrs, on ? 2u * row : 2u * v16, 0, 0)
                  : 0x3c00u;
      sAc[m] = sAw[m] = 0u;
    } else {
#pragma unroll
      for (int s = 0; s < kBMaxSteps; ++s) {
        const bool part_c = s < csteps;
        const int col = 32 * (part_c ? s : s - csteps) + 8 * q;
        const bool cv = on && s < esteps && col < (part_c ? a.r_c : a.r_r);
        const uint32_t off = row * (uint32_t)r + (uint32_t)((part_c ? 0 : a.r_c) + col);
        ac[m][s] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(ars, cv ? off : v16 * (uint32_t)r, 0, 0));
      }
      sR[m] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rrs, on ? 2u * row : 2u * v16, 0, 0);
      sAc[m] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(srs, 2u * row * (uint32_t)a.nA, 0, 0);
      sAw[m] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(srs, 2u * (row * (uint32_t)a.nA + (uint32_t)a.nA - 1u), 0, 0);
    }
  });
  static_for<0, MM>([&](auto M_) {
    constexpr int m = decltype(M_)::value;
    f4 pc[T], pw[T];
#pragma unroll
    for (int t = 0; t < T; ++t) pc[t] = pw[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kBMaxSteps; ++s) {
      if (s < esteps) {  // uniform
        const h8 av = unpack_i8x8(ac[m][s][0], ac[m][s][1]);
        if (s < csteps) {
#pragma unroll
          for (int t = 0; t < T; ++t) {
            pc[t] = mfma16(sZf[((2 * s) * T + t) * 64 + lane], av, pc[t]);
            pc[t] = mfma16(sZf[((2 * s + 1) * T + t) * 64 + lane], av, pc[t]);
          }
          mfma_drain();
        } else {
#pragma unroll
          for (int t = 0; t < T; ++t) {
            pw[t] = mfma16(sZf[((2 * s) * T + t) * 64 + lane], av, pw[t]);
            pw[t] = mfma16(sZf[((2 * s + 1) * T + t) * 64 + lane], av, pw[t]);
          }
          mfma_drain();
        }
      }
    }
    mfma_drain();
    const uint32_t v = (uint32_t)(bw0 + m) * 16u + (uint32_t)i16;
    if (m < Mw && (int64_t)v < a.V) {
      const float fR = f16_to_f32((uint16_t)sR[m]);
      const float fAc = a.r_c > 0 ? f16_to_f32((uint16_t)sAc[m]) : 0.0f;
      const float fAw = a.r_r > 0 ? f16_to_f32((uint16_t)sAw[m]) : 0.0f;
#pragma unroll
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = 16 * t + 4 * q + e;
          if (n >= N) continue;
          float y = sTok[2 * n] * (fR * acc[m][t][e]);
          if (r > 0) y = fmaf(sTok[2 * n + 1], fmaf(fAw, pw[t][e], fAc * pc[t][e]), y);
          const uint32_t off = (uint32_t)n * ystride + v;  // the host keeps N rows of Y below 4 GiB
          if (a.y_bf16)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16(y), yrs, 2u * off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), yrs, 4u * off, 0, 0);
        }
      }
    }
  });
}

inline int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || n <= 0)
    return 256;
  return n;
}

// most blocks a workgroup gets when the blocks are split over `grid` workgroups
inline int64_t batch_wg_blocks(int64_t nb, int64_t grid) { return (nb + grid - 1) / grid; }
// most blocks a wave gets
inline int batch_blocks_per_wave(int64_t nb, int64_t grid) {
  return (int)((batch_wg_blocks(nb, grid) + kBWaves - 1) / kBWaves);
}

// Workgroups per CU.  One: two workgroups of two token tiles (sixteen waves
// a CU, two k-tiles in flight per wave) measured slower than one with four
// k-tiles in flight per wave.
inline int batch_occupancy(int) { return 1; }

inline int64_t batch_grid(int64_t nb, int occ) {
  int64_t grid = std::min<int64_t>((int64_t)occ * device_cus(), (nb + kBWaves - 1) / kBWaves);
  while (batch_blocks_per_wave(nb, grid) > (occ > 1 ? kBMaxBlocks2 : kBMaxBlocks)) ++grid;
  return grid;
}

// k-tiles per half of the H ring, which is also the number of packed tiles a
// wave keeps in flight: four for up to three token tiles when 8 divides the
// k-tile count, else two (the accumulators of four token tiles leave room
// for no more registers of packed tiles)
inline int batch_hk(int T, int nkt) { return T <= 3 && nkt % 8 == 0 ? 4 : 2; }
// static LDS of the H ring
inline uint32_t batch_ring_lds(int T, int hk) { return 2u * (uint32_t)hk * 4u * (uint32_t)T * 1024u; }

inline BLds batch_layout(const archead_dims* d, int64_t n_tokens, int64_t nb, int64_t grid) {
  const int T = (int)((n_tokens + 15) / 16);
  const int esteps = d->format == ARCHEAD_FMT_ARCHEAD
                         ? (int)((round_up((uint64_t)d->r_c, 32) + round_up((uint64_t)d->r_r, 32)) / 32)
                         : 0;
  return batch_lds(T, esteps, (int)(16 * batch_wg_blocks(nb, grid)),
                   bcode_row_bytes(d->format, (int)(d->D / d->g)));
}

// k-tiles of packed tiles in flight per wave: a row-INT8 tile is twice the
// bytes, so half as many keep the same bytes in flight
constexpr int batch_k(int fmt, int hk) { return fmt == ARCHEAD_FMT_ROW_INT8 ? hk / 2 : hk; }

template <int FMT, int T, int MM, int CPT>
hipError_t launch_tmc(const FwdArgs& a, const BLds& L, unsigned grid, hipStream_t s) {
  // the batched kernel ends every launch of a forward that gives it events
  constexpr bool last = true;
  if constexpr (T <= 3) {
    if (batch_hk(T, a.nkt) == 4)
      return launch_main(batch_kernel<FMT, T, MM, CPT, 4, batch_k(FMT, 4), 1>, dim3(grid), dim3(kBThreads), L.total,
                         s, last, a, L);
  }
  return launch_main(batch_kernel<FMT, T, MM, CPT, 2, batch_k(FMT, 2), 1>, dim3(grid), dim3(kBThreads), L.total, s,
                     last, a, L);
}

template <int FMT, int T, int CPT>
hipError_t launch_tc(const FwdArgs& a, hipStream_t s) {
  const int64_t grid = batch_grid(a.nb, batch_occupancy(T));
  const archead_dims d{a.V, a.D, a.r_c, a.r_r, a.g, FMT};
  const BLds L = batch_layout(&d, a.N, a.nb, grid);
  const unsigned gu = (unsigned)grid;
  switch (batch_blocks_per_wave(a.nb, grid)) {
    case 1: return launch_tmc<FMT, T, 1, CPT>(a, L, gu, s);
    case 2: return launch_tmc<FMT, T, 2, CPT>(a, L, gu, s);
    case 3: return launch_tmc<FMT, T, 3, CPT>(a, L, gu, s);
    case 4: return launch_tmc<FMT, T, 4, CPT>(a, L, gu, s);
    case 5: return launch_tmc<FMT, T, 5, CPT>(a, L, gu, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, int T>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  if constexpr (FMT == ARCHEAD_FMT_ROW_INT8) {
    return launch_tc<FMT, T, 1>(a, s);  // no groups
  } else {
    switch (a.g) {
      case 32: return launch_tc<FMT, T, 4>(a, s);
      case 64: return launch_tc<FMT, T, 2>(a, s);
      default: return launch_tc<FMT, T, 1>(a, s);
    }
  }
}

}  // namespace

// launchers of the comparison heads' instances (batch_g4.hip, batch_r8.hip)
hipError_t launch_batch_group_int4(const FwdArgs& a, hipStream_t s);
hipError_t launch_batch_row_int8(const FwdArgs& a, hipStream_t s);

}  // namespace archead
