// Pre-projection kernels.
//
// Algorithm 1 (inference step) evaluates the correction as (H B_w^T) A_w^T;
// the quantised core A_c B_c is evaluated the same way.  These kernels form
// Z = H [B_c_hat ; B_w_hat]^T once per call (r dot products of length D per
// token, fp32), and convert H into the fp16 MFMA operand the forward kernels
// stream:
//   hf  : H * 2^S_n in fp16, S_n chosen per token so the row maximum lands in
//         [2^14, 2^15); every bf16 value at most 2^31 below the row maximum is
//         then exact in fp16.  hscale[n] = 2^-S_n undoes it in the epilogue.
//   zf  : Z * 2^F_n split into fp16 hi + lo (22 significant bits), per-token
//         exponent F_n chosen the same way; zscale[n] = 2^-F_n.
// Both are stored in MFMA operand order (see device_common.h) so the forward
// kernels read each operand fragment as one contiguous 1 KB block: 16 rows x
// 32 columns for the 16 x 16 x 32 MFMA kernels, 32 rows x 16 columns for the
// 32 x 32 x 16 MFMA kernels (layouts in internal.h).
//
// The 32-row layouts are produced in three passes: prep_h32_kernel converts
// H; zmm_kernel forms Z on the 32 x 32 x 16 MFMA from that fp16 H and the
// exact INT8 B codes (so B is read once per 32-token tile, not once per
// token); zsplit_kernel picks F_n and writes the hi/lo fragments.
#include "device_common.h"
#include "internal.h"

namespace archead {

namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / 64;

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = 0.0f;
#pragma unroll
  for (int w = 0; w < kPrepWaves; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

// 16-row layouts, one workgroup per token row n (rows N..n16-1 are zero padding):
//   1. S_n from max|H[n,:]|; hf = fp16(H[n,:] * 2^S_n)
//   2. z[j] = sum_k H[n,k] B_hat[j,k] for all j < r (fp32, one wave per j, kept in LDS)
//   3. F_n from max_j |z[j]|; zf = fp16 hi/lo split of z * 2^F_n
constexpr bool ROWS32 = false;
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const FwdArgs a) {
  __shared__ float red[kPrepWaves];
  __shared__ float zrow[2 * kMaxRank];
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool real = n < a.N;
  const uint16_t* hrow = a.H + (real ? n : 0) * a.H_stride;
  const int nchunk = (int)(a.D / 8);
  const int64_t tile = ROWS32 ? n >> 5 : n >> 4;
  const int i = ROWS32 ? (int)(n & 31) : (int)(n & 15);

  // 1. hidden-state row -> scaled fp16 operand fragments
  float m = 0.0f;
  if (real) {
    for (int c = tid; c < nchunk; c += kPrepThreads) {
      const u4 raw = *reinterpret_cast<const u4*>(hrow + 8 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(raw[w] & 0xffffu))));
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(raw[w] >> 16))));
      }
    }
  }
  m = block_max(m, red);
  const int S = row_exponent(m);
  if (tid == 0) a.hscale[n] = real ? ldexpf(1.0f, -S) : 0.0f;
  for (int c = tid; c < nchunk; c += kPrepThreads) {
    const int64_t k0 = 8 * (int64_t)c;
    const int64_t ks = k0 >> 5;
    const int q = (int)((k0 >> 3) & 3);
    float v[8];
    if (real) {
      const u4 raw = *reinterpret_cast<const u4*>(hrow + k0);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = bf16_to_f32((uint16_t)(raw[w] & 0xffffu));
        v[2 * w + 1] = bf16_to_f32((uint16_t)(raw[w] >> 16));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
    h8 out;
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = (_Float16)ldexpf(v[k_order_h(j)], S);
    int64_t frag;
    if (ROWS32) {
      const int64_t kt = k0 >> 7;
      const int R = (int)((k0 >> 3) & 15);
      const int t = (R >> 2) + 4 * ((R >> 1) & 1);
      frag = ((tile * a.nkt + kt) * 8 + t) * 64 + 32 * (R & 1) + i;
    } else {
      frag = (tile * a.nks + ks) * 64 + 16 * q + i;
    }
    *reinterpret_cast<h8*>(a.hf + frag * 8) = out;
  }

  const int r = a.r_c + a.r_r;
  if (r == 0) return;
  // 2. pre-projection z[j] for this token
  for (int j = wave; j < r; j += kPrepWaves) {
    float acc = 0.0f;
    if (real) {
      const int8_t* brow = a.b_codes + (int64_t)j * a.D;
      const uint16_t* srow = a.b_scales + (int64_t)j * a.ng;
      for (int c = lane; c < nchunk; c += 64) {
        const int64_t k0 = 8 * (int64_t)c;
        const u4 hraw = *reinterpret_cast<const u4*>(hrow + k0);
        const u2 braw = *reinterpret_cast<const u2*>(brow + k0);
        float part = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t bw = braw[w >> 1] >> (16 * (w & 1));
          part = fmaf(bf16_to_f32((uint16_t)(hraw[w] & 0xffffu)), (float)(int8_t)(bw & 0xff), part);
          part = fmaf(bf16_to_f32((uint16_t)(hraw[w] >> 16)), (float)(int8_t)((bw >> 8) & 0xff), part);
        }
        acc = fmaf(f16_to_f32(srow[k0 / a.g]), part, acc);
      }
      acc = wave_sum(acc);
    }
    if (lane == 0) zrow[j] = acc;
  }
  __syncthreads();

  // 3. token exponent of z and its fp16 hi/lo operand fragments
  float mz = 0.0f;
  if (real)
    for (int j = tid; j < r; j += kPrepThreads) mz = fmaxf(mz, fabsf(zrow[j]));
  mz = block_max(mz, red);
  const int F = row_exponent(mz);
  if (tid == 0) a.zscale[n] = real ? ldexpf(1.0f, -F) : 0.0f;
  // 16-row layout: fragments of 32 ranks, lane 16 q + i holds ranks 8 q ..;
  // 32-row layout: fragments of 16 ranks, lane 32 q + i (order below)
  constexpr int kRanks = ROWS32 ? 16 : 32, kQ = ROWS32 ? 2 : 4, kRows = ROWS32 ? 32 : 16;
  const int csteps = a.rc32 / kRanks, nsteps = (a.rc32 + a.rr32) / kRanks;
  for (int e = tid; e < nsteps * kQ; e += kPrepThreads) {
    const int s = e / kQ, q = e % kQ;
    const bool part_c = s < csteps;
    const int sl = part_c ? s : s - csteps;
    const int rank = part_c ? a.r_c : a.r_r;
    const int base = part_c ? 0 : a.r_c;
    h8 hi, lo;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      // 32-row layout: steps come in pairs; lane half q of the pair (2j, 2j+1)
      // holds ranks 32 j + 16 q + 8 (s & 1) .., so one 16-byte load of A codes
      // feeds both steps of a pair
      const int col = ROWS32 ? 32 * (sl >> 1) + 16 * q + 8 * (sl & 1) + k_order_z(jj)
                             : kRanks * sl + 8 * q + k_order_z(jj);
      float z = 0.0f;
      if (real && col < rank) z = ldexpf(zrow[base + col], F);
      const _Float16 zh = (_Float16)z;
      hi[jj] = zh;
      lo[jj] = (_Float16)(z - (float)zh);
    }
    _Float16* dst = a.zf + ((tile * (2 * nsteps) + 2 * s) * 64 + kRows * q + i) * 8;
    *reinterpret_cast<h8*>(dst) = hi;
    *reinterpret_cast<h8*>(dst + 64 * 8) = lo;
  }
}

// ---------------------------------------------------------------------------
// 32-row layouts.
//
// hf: within a 128-column k-tile, 8-column run R (0..15) of token n goes to
// MFMA step t = (R >> 2) + 4 * ((R >> 1) & 1), lane (n & 31) + 32 * (R & 1);
// the forward kernels read the residual codes in the same run order.
__host__ __device__ inline int64_t h32_frag(int64_t n, int64_t nkt, int64_t k0) {
  const int64_t kt = k0 >> 7;
  const int R = (int)((k0 >> 3) & 15);
  const int t = (R >> 2) + 4 * ((R >> 1) & 1);
  return (((n >> 5) * nkt + kt) * 8 + t) * 64 + 32 * (R & 1) + (n & 31);
}

// One wave per token row n < n32 (rows from N on are zero), four per
// workgroup: S_n from max|H[n,:]|, hscale[n] = 2^-S_n, hf = fp16(H[n,:] 2^S_n).
// Rows of up to 64 * 8 * kPrepHChunks columns stay in registers between the
// two passes; longer rows are read twice.
constexpr int kPrepHThreads = 256;
constexpr int kPrepHChunks = 16;
__global__ __launch_bounds__(kPrepHThreads) void prep_h32_kernel(const FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t n = 4 * (int64_t)blockIdx.x + (threadIdx.x >> 6);
  if (n >= a.n32) return;
  const bool real = n < a.N;
  const uint16_t* hrow = a.H + (real ? n : 0) * a.H_stride;
  const int nchunk = (int)(a.D / 8);
  const bool cached = nchunk <= 64 * kPrepHChunks;
  u4 raw[kPrepHChunks];
  float m = 0.0f;
  if (real) {
    for (int c0 = 0; c0 < nchunk; c0 += 64 * kPrepHChunks) {
#pragma unroll
      for (int u = 0; u < kPrepHChunks; ++u) {
        const int c = c0 + lane + 64 * u;
        raw[u] = c < nchunk ? *reinterpret_cast<const u4*>(hrow + 8 * c) : u4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kPrepHChunks; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(raw[u][w] & 0xffffu))));
          m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(raw[u][w] >> 16))));
        }
    }
  }
  m = wave_max(m);
  const int S = row_exponent(m);
  if (lane == 0) a.hscale[n] = real ? ldexpf(1.0f, -S) : 0.0f;
  for (int c0 = 0; c0 < nchunk; c0 += 64 * kPrepHChunks) {
#pragma unroll
    for (int u = 0; u < kPrepHChunks; ++u) {
      const int c = c0 + lane + 64 * u;
      if (c < nchunk) {
        const u4 x = !real ? u4{0u, 0u, 0u, 0u} : cached ? raw[u] : *reinterpret_cast<const u4*>(hrow + 8 * c);
        float v[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          v[2 * w] = bf16_to_f32((uint16_t)(x[w] & 0xffffu));
          v[2 * w + 1] = bf16_to_f32((uint16_t)(x[w] >> 16));
        }
        h8 out;
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = (_Float16)ldexpf(v[k_order_h(j)], S);
        *reinterpret_cast<h8*>(a.hf + h32_frag(n, a.nkt, 8 * (int64_t)c) * 8) = out;
      }
    }
  }
}

// Eight INT8 codes (two dwords, column order) -> fp16 in k_order_h, the slot
// order of the hf runs: bytes (k0 k1 k4 k5) and (k2 k3 k6 k7) through the
// k_order_z unpacking give k0 k4 k1 k5 k2 k6 k3 k7.
__device__ __forceinline__ h8 unpack_i8x8_h(uint32_t lo, uint32_t hi) {
  return unpack_i8x8(__builtin_amdgcn_perm(hi, lo, 0x05040100u), __builtin_amdgcn_perm(hi, lo, 0x07060302u));
}

// Z on the MFMA, grid (n32/32 token tiles, ceil(r/32) rank blocks), 16
// waves: wave w takes slice w of the k range (whole groups) for the
// workgroup's 32 tokens and 32 ranks.  MFMA A operand = hf fragments
// (tokens), B operand = the exact INT8 codes of the same 16 columns (ranks);
// each group of g columns is accumulated on its own and added times its fp16
// scale.  The slices are summed through LDS and z32[n][j] = hscale[n] * sum
// is written.
// GC: group size 0 -> g >= 128, 1 -> 64, 2 -> 32 (steps of a k-tile per group).
constexpr int kZmmWaves = 16;
template <int GC>
__global__ __launch_bounds__(64 * kZmmWaves) void zmm_kernel(const FwdArgs a) {
  __shared__ float red[kZmmWaves][32][33];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = a.r_c + a.r_r;
  const int64_t tile = blockIdx.x;
  const int j = 32 * (int)blockIdx.y + (lane & 31);
  const bool jv = j < r;
  const int8_t* brow = a.b_codes + (int64_t)(jv ? j : 0) * a.D;
  const uint16_t* srow = a.b_scales + (int64_t)(jv ? j : 0) * a.ng;
  const h8* hf = reinterpret_cast<const h8*>(a.hf) + tile * a.nkt * 8 * 64 + lane;
  const int kpu = a.g > kKTile ? a.g / kKTile : 1;  // k-tiles per unit (a unit holds whole groups)
  const int units = (int)(a.nkt / kpu);
  const int u0 = wave * units / kZmmWaves, u1 = (wave + 1) * units / kZmmWaves;
  const int half = lane >> 5;
  f16x tot = {}, part = {};
  for (int kt = u0 * kpu; kt < u1 * kpu; ++kt) {
    h8 hv[8];
    u2 bc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int R = 4 * (t & 3) + 2 * (t >> 2) + half;
      hv[t] = hf[(kt * 8 + t) * 64];
      bc[t] = *reinterpret_cast<const u2*>(brow + kKTile * (int64_t)kt + 8 * R);
    }
    // lanes past the last rank read row 0 and are zeroed by their scale
    auto codes = [&](int t) { return unpack_i8x8_h(bc[t][0], bc[t][1]); };
    if constexpr (GC == 0) {
      // g = 128 ends a group with every k-tile, g = 256 with every second
#pragma unroll
      for (int t = 0; t < 8; ++t) part = mfma32(hv[t], codes(t), part);
      if (((kt + 1) * kKTile) % a.g == 0) {
        const float sc = jv ? f16_to_f32(srow[(kt * kKTile) / a.g]) : 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) tot[v] = fmaf(sc, part[v], tot[v]);
        part = f16x{};
      }
    } else {
      // group q of the k-tile: the 16-column block of step t is 2 (t % 4) + t / 4,
      // so g = 64 takes t % 4 in {0, 1} / {2, 3} and g = 32 takes t % 4 == q
      constexpr int kGroups = GC == 2 ? 4 : 2;
#pragma unroll
      for (int q = 0; q < kGroups; ++q) {
        f16x p = {};
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (GC == 2 ? (t & 3) == q : ((t & 3) >> 1) == q) p = mfma32(hv[t], codes(t), p);
        const float sc = jv ? f16_to_f32(srow[(kt * kKTile) / a.g + q]) : 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) tot[v] = fmaf(sc, p[v], tot[v]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) red[wave][8 * (v >> 2) + 4 * half + (v & 3)][lane & 31] = tot[v];
  __syncthreads();
  if (tid < 32 * 32) {
    const int tok = tid >> 5, jr = tid & 31;
    const int jj = 32 * (int)blockIdx.y + jr;
    float z = 0.0f;
#pragma unroll
    for (int w = 0; w < kZmmWaves; ++w) z += red[w][tok][jr];
    const int64_t n = 32 * tile + tok;
    if (jj < r) a.z32[n * r + jj] = z * a.hscale[n];
  }
}

// One wave per token row n < n32: F_n from max_j |z32[n][j]|, zscale[n] =
// 2^-F_n (0 for padding rows), zf = fp16 hi/lo split of z * 2^F_n in the
// 32-row layout: fragments of 16 ranks, steps in pairs (2i, 2i+1) whose lane
// half q holds ranks 32 i + 16 q + 8 (s & 1) .. (one 16-byte load of A codes
// feeds both steps of a pair), slot order k_order_z.
constexpr int kZsplitThreads = 256;
__global__ __launch_bounds__(kZsplitThreads) void zsplit_kernel(const FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t n = 4 * (int64_t)blockIdx.x + (threadIdx.x >> 6);
  if (n >= a.n32) return;
  const bool real = n < a.N;
  const int r = a.r_c + a.r_r;
  const float* zrow = a.z32 + n * r;
  float m = 0.0f;
  if (real)
    for (int j = lane; j < r; j += 64) m = fmaxf(m, fabsf(zrow[j]));
  m = wave_max(m);
  const int F = row_exponent(m);
  if (lane == 0) a.zscale[n] = real ? ldexpf(1.0f, -F) : 0.0f;
  const int csteps = a.rc32 / 16, nsteps = (a.rc32 + a.rr32) / 16;
  const int64_t tile = n >> 5;
  const int i = (int)(n & 31);
  for (int e = lane; e < nsteps * 2; e += 64) {
    const int s = e >> 1, q = e & 1;
    const bool part_c = s < csteps;
    const int sl = part_c ? s : s - csteps;
    const int rank = part_c ? a.r_c : a.r_r;
    const int base = part_c ? 0 : a.r_c;
    h8 hi, lo;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int col = 32 * (sl >> 1) + 16 * q + 8 * (sl & 1) + k_order_z(jj);
      float z = 0.0f;
      if (real && col < rank) z = ldexpf(zrow[base + col], F);
      const _Float16 zh = (_Float16)z;
      hi[jj] = zh;
      lo[jj] = (_Float16)(z - (float)zh);
    }
    _Float16* dst = a.zf + ((tile * (2 * nsteps) + 2 * s) * 64 + 32 * q + i) * 8;
    *reinterpret_cast<h8*>(dst) = hi;
    *reinterpret_cast<h8*>(dst + 64 * 8) = lo;
  }
}

// Small-N pre-projection, grid (N, ceil(r/4) + 1):
//   blockIdx.y < ceil(r/4): z32[n][j] = sum_k H[n,k] B_hat[j,k] in fp32, one
//     wave per (token, j); every lane issues all its loads before the arithmetic.
//   blockIdx.y == ceil(r/4): hscale[n] = 2^-S_n and hc[n][:] = fp16(H[n,:] 2^S_n)
//     in kernel k-order (S_n as in prep_kernel).
constexpr int kPrepZThreads = 256;
constexpr int kPrepZMaxChunks = 16;  // D <= 64*8*16 = 8192 columns per lane loop

__global__ __launch_bounds__(kPrepZThreads) void prep_z_kernel(const FwdArgs a) {
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r_c + a.r_r;
  const int nJ = (r + 3) / 4;
  const uint16_t* hrow = a.H + n * a.H_stride;
  const int nchunk = (int)(a.D / 8);
  if ((int)blockIdx.y == nJ) {
    // the row's first kPrepZKeep * 256 chunks stay in registers between the
    // maximum and the conversion (one read of H for D <= 8192)
    constexpr int kPrepZKeep = 4;
    __shared__ float red[kPrepZThreads / 64];
    u4 keep[kPrepZKeep];
#pragma unroll
    for (int i = 0; i < kPrepZKeep; ++i) {
      const int c = tid + i * kPrepZThreads;
      keep[i] = c < nchunk ? *reinterpret_cast<const u4*>(hrow + 8 * c) : u4{0u, 0u, 0u, 0u};
    }
    // f(chunk index, its 8 bf16 values) for every chunk of this thread
    auto each_chunk = [&](auto f) {
#pragma unroll
      for (int i = 0; i < kPrepZKeep; ++i)
        if (tid + i * kPrepZThreads < nchunk) f(tid + i * kPrepZThreads, keep[i]);
      for (int c = tid + kPrepZKeep * kPrepZThreads; c < nchunk; c += kPrepZThreads)
        f(c, *reinterpret_cast<const u4*>(hrow + 8 * c));
    };
    float m = 0.0f;
    each_chunk([&](int, const u4& raw) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(raw[w] & 0xffffu))));
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(raw[w] >> 16))));
      }
    });
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int S = row_exponent(m);
    if (tid == 0) a.hscale[n] = ldexpf(1.0f, -S);
    each_chunk([&](int c, const u4& raw) {
      float v[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = bf16_to_f32((uint16_t)(raw[w] & 0xffffu));
        v[2 * w + 1] = bf16_to_f32((uint16_t)(raw[w] >> 16));
      }
      h8 out;
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] = (_Float16)ldexpf(v[k_order_h(j)], S);
      *reinterpret_cast<h8*>(a.hc + n * a.D + 8 * c) = out;
    });
    return;
  }
  const int j = blockIdx.y * (kPrepZThreads / 64) + wave;
  if (j >= r) return;
  const int8_t* brow = a.b_codes + (int64_t)j * a.D;
  const uint16_t* srow = a.b_scales + (int64_t)j * a.ng;
  float acc = 0.0f;
  for (int c0 = 0; c0 < nchunk; c0 += 64 * kPrepZMaxChunks) {
    u4 hr[kPrepZMaxChunks];
    u2 br[kPrepZMaxChunks];
    uint16_t sr[kPrepZMaxChunks];
#pragma unroll
    for (int u = 0; u < kPrepZMaxChunks; ++u) {
      const int c = c0 + lane + 64 * u;
      if (c < nchunk) {
        hr[u] = *reinterpret_cast<const u4*>(hrow + 8 * (int64_t)c);
        br[u] = *reinterpret_cast<const u2*>(brow + 8 * (int64_t)c);
        sr[u] = srow[(8 * c) / a.g];
      }
    }
#pragma unroll
    for (int u = 0; u < kPrepZMaxChunks; ++u) {
      const int c = c0 + lane + 64 * u;
      if (c < nchunk) {
        float part = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t bw = br[u][w >> 1] >> (16 * (w & 1));
          part = fmaf(bf16_to_f32((uint16_t)(hr[u][w] & 0xffffu)), (float)(int8_t)(bw & 0xff), part);
          part = fmaf(bf16_to_f32((uint16_t)(hr[u][w] >> 16)), (float)(int8_t)((bw >> 8) & 0xff), part);
        }
        acc = fmaf(f16_to_f32(sr[u]), part, acc);
      }
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) a.z32[n * r + j] = acc;
}

}  // namespace

hipError_t launch_prep_z(const FwdArgs& a, hipStream_t s) {
  const int r = a.r_c + a.r_r;
  hipLaunchKernelGGL(prep_z_kernel, dim3((unsigned)a.N, (unsigned)((r + 3) / 4 + 1)), dim3(kPrepZThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prep(const FwdArgs& a, bool rows32, hipStream_t s) {
  if (!rows32) {
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)a.n16), dim3(kPrepThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(prep_h32_kernel, dim3((unsigned)((a.n32 + 3) / 4)), dim3(kPrepHThreads), 0, s, a);
  const int r = a.r_c + a.r_r;
  if (r > 0) {
    const dim3 grid((unsigned)(a.n32 / 32), (unsigned)((r + 31) / 32));
    if (a.g == 32)
      hipLaunchKernelGGL(zmm_kernel<2>, grid, dim3(64 * kZmmWaves), 0, s, a);
    else if (a.g == 64)
      hipLaunchKernelGGL(zmm_kernel<1>, grid, dim3(64 * kZmmWaves), 0, s, a);
    else
      hipLaunchKernelGGL(zmm_kernel<0>, grid, dim3(64 * kZmmWaves), 0, s, a);
  }
  hipLaunchKernelGGL(zsplit_kernel, dim3((unsigned)((a.n32 + 3) / 4)), dim3(kZsplitThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace archead
