// Decode path (N <= 64 tokens): stream the packed head once.
//
// Y = H W_d^T + (H B_w^T) A_w^T (Algorithm 1, inference step) with
// W_d = Q(A_c)Q(B_c) + SC4(R) (Sec. 3, quantized-core equation).
//
// Work split: one wave owns RB consecutive 16-row vocabulary blocks and all
// N (<= 16*NT) tokens, and walks the whole hidden dimension, so every packed
// byte is read from HBM exactly once and no cross-wave reduction is needed.
// Per 32-column step the wave issues one v_mfma_f32_16x16x32_f16 per
// (block, token tile): operand A = 16 tokens of the converted H (hf, fp16),
// operand B = 16 vocabulary rows of INT4 codes turned into exact fp16 integers
// in registers.  Products are exact and accumulate in fp32; each group's
// partial sum is multiplied by its uint8 group code once per group (g >= 32),
// and the fp16 row scale s_R, the token scale and the low-rank term are
// applied in the epilogue.  The low-rank term is (Z * A^T) with Z split into
// fp16 hi/lo and the INT8 A codes as exact fp16 integers, one accumulator per
// part (c, w) so each part gets its own row scale.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace archead {

namespace {

constexpr int kDecodeThreads = 256;  // 4 waves, each independent

template <int NT, int RB>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t blk0 = ((int64_t)blockIdx.x * (kDecodeThreads / 64) + wave) * RB;
  if (blk0 >= a.nb) return;
  const int nblk = (int)((a.nb - blk0) < RB ? (a.nb - blk0) : RB);
  const int i16 = lane & 15;
  const int q = lane >> 4;

  f4 acc[RB][NT], part[RB][NT];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[b][t] = f4{0.f, 0.f, 0.f, 0.f};
      part[b][t] = f4{0.f, 0.f, 0.f, 0.f};
    }

  const int ntiles = (int)(a.n16 >> 4);
  const int steps_per_group = a.g / 32;
  const u4* wbase = reinterpret_cast<const u4*>(a.r_codes) + blk0 * 64 + lane;
  const h8* hbase = reinterpret_cast<const h8*>(a.hf) + lane;

  for (int kt = 0; kt < a.nkt; ++kt) {
    u4 w[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b)
      w[b] = (b < nblk) ? __builtin_nontemporal_load(wbase + ((int64_t)kt * a.nb + b) * 64)
                        : u4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ks = 4 * kt + s;
      h8 hv[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < ntiles) {
          hv[t] = hbase[((int64_t)t * a.nks + ks) * 64];
        } else {
          hv[t] = h8{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const h8 wv = unpack_q4(w[b][s]);
#pragma unroll
        for (int t = 0; t < NT; ++t) part[b][t] = mfma16(hv[t], wv, part[b][t]);
      }
      if ((ks + 1) % steps_per_group == 0) {
        const int grp = ks / steps_per_group;
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const float c = (b < nblk)
              ? (float)a.r_gcodes[((blk0 + b) * 16 + i16) * a.ng + grp] : 0.0f;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc[b][t] += c * part[b][t];
            part[b][t] = f4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
  }

  const int r = a.r_c + a.r_r;
  const int csteps = a.rc32 / 32, wsteps = a.rr32 / 32;
  const h8* zbase = reinterpret_cast<const h8*>(a.zf) + lane;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (b >= nblk) break;
    const int64_t v = 16 * (blk0 + b) + i16;
    const float sR = f16_to_f32(a.r_rowscale[v]);
    const float sAc = a.r_c > 0 ? f16_to_f32(a.a_scales[v * a.nA]) : 0.0f;
    const float sAw = a.r_r > 0 ? f16_to_f32(a.a_scales[v * a.nA + a.nA - 1]) : 0.0f;
    f4 pc[NT], pw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      pc[t] = f4{0.f, 0.f, 0.f, 0.f};
      pw[t] = f4{0.f, 0.f, 0.f, 0.f};
    }
    const int8_t* arow = a.a_codes + v * r;
    for (int s = 0; s < csteps + wsteps; ++s) {
      const bool part_c = s < csteps;
      const int col = 32 * (part_c ? s : s - csteps) + 8 * q;
      const int rank = part_c ? a.r_c : a.r_r;
      u2 raw = {0u, 0u};
      if (col < rank) raw = *reinterpret_cast<const u2*>(arow + (part_c ? 0 : a.r_c) + col);
      const h8 av = unpack_i8x8(raw[0], raw[1]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < ntiles) {
          const h8 zh = zbase[((int64_t)t * 2 * a.zsteps + 2 * s) * 64];
          const h8 zl = zbase[((int64_t)t * 2 * a.zsteps + 2 * s + 1) * 64];
          if (part_c) {
            pc[t] = mfma16(zh, av, pc[t]);
            pc[t] = mfma16(zl, av, pc[t]);
          } else {
            pw[t] = mfma16(zh, av, pw[t]);
            pw[t] = mfma16(zl, av, pw[t]);
          }
        }
      }
    }
    if (v >= a.V) continue;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t n = 16 * t + 4 * q + e;
        if (n >= a.N) continue;
        float y = a.hscale[n] * (sR * acc[b][t][e]);
        if (r > 0) y = fmaf(a.zscale[n], fmaf(sAw, pw[t][e], sAc * pc[t][e]), y);
        if (a.y_bf16)
          reinterpret_cast<uint16_t*>(a.Y)[n * a.Y_stride + v] = f32_to_bf16(y);
        else
          reinterpret_cast<float*>(a.Y)[n * a.Y_stride + v] = y;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-N decode (N <= 16 and all of H plus Z fit in LDS), persistent.
//
// The grid holds only co-resident workgroups (at most kLdsWgPerCu per CU).
// Every wave walks a grid-strided list of 16-row blocks (b, b + W, b + 2W, ...
// with W the number of waves), so at any moment neighbouring waves read
// neighbouring 1 KB tiles of the same k-tile plane.  Each wave keeps a ring of
// P packed tiles in flight in registers, plus one vector of group codes per
// chunk of 4 tiles (the lane's row codes for 512 columns, one small load).  The
// ring runs across block boundaries, so a wave never drains its pipeline.  H
// (already scaled fp16 from the pre-projection kernel) and Z (fp32) sit in
// LDS; LDS reads use the separate lgkm counter and never wait behind the ring.
// MFMA rows past the tokens read a zero row of H in LDS.
constexpr int kLdsWaves = 4;
constexpr int kLdsThreads = 64 * kLdsWaves;
#ifndef ARCHEAD_DECODE_WG_PER_CU
#define ARCHEAD_DECODE_WG_PER_CU 4
#endif
constexpr int kLdsWgPerCu = ARCHEAD_DECODE_WG_PER_CU;
constexpr int kEpiSteps = 2;  // low-rank 32-column steps whose A codes are prefetched

// The lane's group codes for one chunk of 4 tiles (512 columns): 512/g bytes.
template <int G> struct CodeVec;
template <> struct CodeVec<256> { typedef uint16_t T; };
template <> struct CodeVec<128> { typedef uint32_t T; };
template <> struct CodeVec<64> { typedef u2 T; };
template <> struct CodeVec<32> { typedef u4 T; };

template <int G>
__device__ __forceinline__ float code_at(const typename CodeVec<G>::T& v, int idx) {
  if constexpr (G == 256 || G == 128) {
    return (float)((((uint32_t)v) >> (8 * idx)) & 0xffu);
  } else {
    return (float)((v[idx >> 2] >> (8 * (idx & 3))) & 0xffu);
  }
}

// LDS carve-up of the small-N kernel: H as fp16 [N + 1][D + 8] (8 halves of
// padding per row spread the rows over the banks; row N is zero, read by the
// MFMA lanes that carry no token), then Z as fp32 [N][r].
__host__ __device__ inline size_t lds_h_bytes(int64_t N, int64_t D) { return (size_t)(N + 1) * (D + 8) * 2; }
__host__ __device__ inline size_t lds_bytes(int64_t N, int64_t D, int r) {
  return lds_h_bytes(N, D) + (size_t)N * r * 4;
}

template <int P, int G>
__global__ __launch_bounds__(kLdsThreads) void decode_lds_kernel(const FwdArgs a) {
  static_assert(P % 4 == 0, "the ring holds whole 4-tile code chunks");
  using CV = typename CodeVec<G>::T;
  constexpr int NC = P / 4;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float s_hs[kDecodeLdsTokens];
  __shared__ int s_F[kDecodeLdsTokens];
  _Float16* sH = reinterpret_cast<_Float16*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = (int)a.N;
  const int D = (int)a.D;
  const int ldh = D + 8;
  const int r = a.r_c + a.r_r;
  float* sZ = reinterpret_cast<float*>(smem + lds_h_bytes(N, D));
  const int i16 = lane & 15, q = lane >> 4;
  const int nkt = a.nkt;
  const int ng = a.ng;
  const int64_t nb = a.nb;
  const int64_t nwaves = (int64_t)gridDim.x * kLdsWaves;
  const int csteps = a.rc32 / 32, wsteps = a.rr32 / 32;
  const int esteps = csteps + wsteps;

  // residual tiles are k-tile major: tile kt of block b at (kt*nb + b)*1024
  // bytes; group codes are row-major [V16][ng].  32-bit byte offsets from the
  // section bases (the host checks both sections are below 4 GiB).
  const uint32_t tstride = (uint32_t)nb * 1024u;
  const unsigned char* wbase = a.r_codes;
  const unsigned char* cbase = a.r_gcodes;
  auto tile_at = [&](int64_t blk, int kt) {
    return __builtin_nontemporal_load(reinterpret_cast<const u4*>(
        wbase + ((uint32_t)blk * 1024u + (uint32_t)kt * tstride + (uint32_t)lane * 16u)));
  };
  auto codes_at = [&](int64_t blk, int kt4) {  // codes of tiles kt4..kt4+3 for this lane's row
    return *reinterpret_cast<const CV*>(
        cbase + ((uint32_t)(blk * 16 + i16) * (uint32_t)ng + (uint32_t)(kt4 * 128 / G)));
  };
  // epilogue sections: s_R [V16], A scales [V16][nA], A codes [V16][r]
  const uint32_t v16 = (uint32_t)nb * 16u;
  const __amdgpu_buffer_rsrc_t rrs = buffer_rsrc(a.r_rowscale, 2u * v16);
  const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(a.a_scales, 2u * v16 * (uint32_t)a.nA);
  const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(a.a_codes, v16 * (uint32_t)r);

  int64_t b = (int64_t)blockIdx.x * kLdsWaves + wave;
  const int64_t b0 = b < nb ? b : nb - 1;  // waves without work load a valid block, store nothing
  const int per_row = D / 8;

  // prologue, one round trip: this thread's first pieces of H, Z and the
  // token scales, then the weight ring, then those pieces into LDS
  constexpr int kPre = 2;
  u4 hpre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int c = tid + i * kLdsThreads;
    hpre[i] = c < N * per_row ? *reinterpret_cast<const u4*>(a.hc + (int64_t)(c / per_row) * D + 8 * (c % per_row))
                              : u4{0u, 0u, 0u, 0u};
  }
  const float zpre = tid < N * r ? a.z32[tid] : 0.0f;
  const float hspre = tid < N ? a.hscale[tid] : 0.0f;
  u4 wr[P];
  CV cv[NC];
#pragma unroll
  for (int j = 0; j < P; ++j) wr[j] = tile_at(b0, j);
#pragma unroll
  for (int c = 0; c < NC; ++c) cv[c] = codes_at(b0, 4 * c);
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int c = tid + i * kLdsThreads;
    if (c < N * per_row) *reinterpret_cast<u4*>(sH + (c / per_row) * ldh + 8 * (c % per_row)) = hpre[i];
  }
  if (tid < N * r) sZ[tid] = zpre;
  if (tid < N) s_hs[tid] = hspre;
  for (int c = tid; c < (D + 8) / 8; c += kLdsThreads)
    *reinterpret_cast<u4*>(sH + N * ldh + 8 * c) = u4{0u, 0u, 0u, 0u};
  for (int c = tid + kPre * kLdsThreads; c < N * per_row; c += kLdsThreads) {
    const int n = c / per_row, k8 = c - n * per_row;
    *reinterpret_cast<u4*>(sH + n * ldh + 8 * k8) =
        *reinterpret_cast<const u4*>(a.hc + (int64_t)n * D + 8 * k8);
  }
  for (int c = tid + kLdsThreads; c < N * r; c += kLdsThreads) sZ[c] = a.z32[c];
  __syncthreads();
  if (b >= nb) return;

  const bool real = i16 < N;
  const _Float16* hrow = sH + (real ? i16 : N) * ldh + 8 * q;
  // per-token Z exponent from LDS: lanes i16 + 16 q split the ranks of token
  // i16; every wave writes the same values to s_F
  int F = 0;
  {
    float m = 0.0f;
    if (real)
      for (int j = q; j < r; j += 4) m = fmaxf(m, fabsf(sZ[i16 * r + j]));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    F = real ? row_exponent(m) : 0;
    if (q == 0 && real) s_F[i16] = F;
  }

  int64_t bn = b + nwaves;
  while (b < nb) {
    const int64_t bnx = bn < nb ? bn : b;  // the ring's next block (or a harmless re-read)
    const int64_t v = 16 * b + i16;
    // epilogue operands of this block, loaded now so they arrive long before
    // use: buffer loads with no branches (past a section's end they read zero),
    // every choice made where the values are used, so nothing here waits
    const uint32_t vv = (uint32_t)v;
    const uint16_t sRb = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rrs, 2u * vv, 0, 0);
    const uint16_t sAcb = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(srs, 2u * vv * (uint32_t)a.nA, 0, 0);
    const uint16_t sAwb =
        (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(srs, 2u * (vv * (uint32_t)a.nA + (uint32_t)a.nA - 1u), 0, 0);
    u2 araw[kEpiSteps];
#pragma unroll
    for (int s = 0; s < kEpiSteps; ++s) {
      const bool part_c = s < csteps;
      const int col = 32 * (part_c ? s : s - csteps) + 8 * q;
      araw[s] = __builtin_bit_cast(
          u2, __builtin_amdgcn_raw_buffer_load_b64(ars, vv * (uint32_t)r + (uint32_t)((part_c ? 0 : a.r_c) + col), 0, 0));
    }

    f4 acc = {0.f, 0.f, 0.f, 0.f}, part = {0.f, 0.f, 0.f, 0.f};
    // nkt >= 4: the loop body runs at least once, which lets the compiler
    // count the loads between the prefetches above and their use
    int kt0 = 0;
    do {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        // keep the scheduler from hoisting work of later ring slots
        __builtin_amdgcn_sched_barrier(0);
        const int kt = kt0 + j;
        float c[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) c[s] = code_at<G>(cv[j / 4], (128 * (j & 3) + 32 * s) / G);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const h8 hv = *reinterpret_cast<const h8*>(hrow + 32 * (4 * kt + s));
          part = mfma16(hv, unpack_q4(wr[j][s]), part);
          // a group of g columns ends after this 32-column step
          const bool flush = ((128 * (j & 3) + 32 * (s + 1)) % G) == 0;
          if (flush) {
            acc += c[s] * part;
            part = f4{0.f, 0.f, 0.f, 0.f};
          }
        }
        {
          // refill the slot with the tile P positions ahead in this wave's sequence
          const bool same = kt + P < nkt;
          wr[j] = tile_at(same ? b : bnx, same ? kt + P : kt + P - nkt);
          if ((j & 3) == 3) {
            const int k4 = kt - 3 + P;  // first tile of the chunk this code slot serves next
            cv[j / 4] = codes_at(k4 < nkt ? b : bnx, k4 < nkt ? k4 : k4 - nkt);
          }
        }
      }
      kt0 += P;
    } while (kt0 < nkt);

    // epilogue: row scale, low-rank term (Z hi/lo from LDS against exact INT8
    // A codes, one accumulator per part), store
    f4 pc = {0.f, 0.f, 0.f, 0.f}, pw = {0.f, 0.f, 0.f, 0.f};
    auto low_rank_step = [&](int s, u2 raw) {
      const bool part_c = s < csteps;
      const int col = 32 * (part_c ? s : s - csteps) + 8 * q;
      const int rank = part_c ? a.r_c : a.r_r;
      const int base = part_c ? 0 : a.r_c;
      if (col >= rank) raw = u2{0u, 0u};
      const h8 av = unpack_i8x8(raw[0], raw[1]);
      h8 zh, zl;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int cc = col + k_order_z(jj);
        const float z = (real && cc < rank) ? ldexpf(sZ[i16 * r + base + cc], F) : 0.0f;
        zh[jj] = (_Float16)z;
        zl[jj] = (_Float16)(z - (float)zh[jj]);
      }
      if (part_c) {
        pc = mfma16(zh, av, pc);
        pc = mfma16(zl, av, pc);
      } else {
        pw = mfma16(zh, av, pw);
        pw = mfma16(zl, av, pw);
      }
    };
    if (esteps <= kEpiSteps) {  // every A code was prefetched
#pragma unroll
      for (int s = 0; s < kEpiSteps; ++s)
        if (s < esteps) low_rank_step(s, araw[s]);
    } else {
      const int8_t* arow = a.a_codes + v * r;
#pragma unroll
      for (int s = 0; s < kEpiSteps; ++s) low_rank_step(s, araw[s]);
      for (int s = kEpiSteps; s < esteps; ++s) {
        const bool part_c = s < csteps;
        const int col = 32 * (part_c ? s : s - csteps) + 8 * q;
        const int rank = part_c ? a.r_c : a.r_r;
        u2 raw = {0u, 0u};
        if (col < rank) raw = *reinterpret_cast<const u2*>(arow + (part_c ? 0 : a.r_c) + col);
        low_rank_step(s, raw);
      }
    }
    if (v < a.V) {
      const float sR = f16_to_f32(sRb);
      const float sAc = a.r_c > 0 ? f16_to_f32(sAcb) : 0.0f, sAw = a.r_r > 0 ? f16_to_f32(sAwb) : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 4 * q + e;
        if (n >= N) continue;
        float y = s_hs[n] * (sR * acc[e]);
        if (r > 0) y = fmaf(ldexpf(1.0f, -s_F[n]), fmaf(sAw, pw[e], sAc * pc[e]), y);
        if (a.y_bf16)
          reinterpret_cast<uint16_t*>(a.Y)[n * a.Y_stride + v] = f32_to_bf16(y);
        else
          reinterpret_cast<float*>(a.Y)[n * a.Y_stride + v] = y;
      }
    }
    b = bn;
    bn = b + nwaves;
  }
}

#ifndef ARCHEAD_RING_DEPTH
#define ARCHEAD_RING_DEPTH 4
#endif
constexpr int kRingDepth = ARCHEAD_RING_DEPTH;  // largest packed-tile ring per wave

// CUs of the current device (256 if the runtime cannot tell)
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <int P, int G>
hipError_t launch_lds_p(const FwdArgs& a, hipStream_t s) {
  const size_t lds = lds_bytes(a.N, a.D, a.r_c + a.r_r);
  // persistent grid: never more workgroups than can be resident at once
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_lds_kernel<P, G>, kLdsThreads, lds) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  per_cu = std::min(per_cu, kLdsWgPerCu);
  const int64_t need = (a.nb + kLdsWaves - 1) / kLdsWaves;
  const int64_t grid = std::min<int64_t>(need, (int64_t)device_cu_count() * per_cu);
  hipLaunchKernelGGL((decode_lds_kernel<P, G>), dim3((unsigned)grid), dim3(kLdsThreads), lds, s, a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_lds(const FwdArgs& a, hipStream_t s) {
  if (kRingDepth >= 8 && a.nkt % 8 == 0) return launch_lds_p<(kRingDepth >= 8 ? 8 : 4), G>(a, s);
  return launch_lds_p<4, G>(a, s);
}

}  // namespace

bool decode_lds_eligible(const FwdArgs& a) {
  const uint64_t rbytes = (uint64_t)a.nb * 16 * (uint64_t)a.D / 2;  // 32-bit section offsets
  return a.N >= 1 && a.N <= kDecodeLdsTokens && a.nkt % 4 == 0 &&
         lds_bytes(a.N, a.D, a.r_c + a.r_r) <= kDecodeLdsBytes && rbytes < (1ull << 32);
}

hipError_t launch_decode_lds(const FwdArgs& a, hipStream_t s) {
  switch (a.g) {
    case 32: return launch_lds<32>(a, s);
    case 64: return launch_lds<64>(a, s);
    case 128: return launch_lds<128>(a, s);
    default: return launch_lds<256>(a, s);
  }
}

namespace {

template <int NT, int RB>
hipError_t launch_nt(const FwdArgs& a, hipStream_t s) {
  const int64_t tasks = (a.nb + RB - 1) / RB;
  const int64_t blocks = (tasks + 3) / 4;
  hipLaunchKernelGGL((decode_kernel<NT, RB>), dim3((unsigned)blocks), dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const FwdArgs& a, hipStream_t s) {
  const int nt = (int)(a.n16 >> 4);
  switch (nt) {
    case 1: return launch_nt<1, 1>(a, s);
    case 2: return launch_nt<2, 2>(a, s);
    case 3: return launch_nt<3, 2>(a, s);
    default: return launch_nt<4, 2>(a, s);
  }
}

}  // namespace archead
