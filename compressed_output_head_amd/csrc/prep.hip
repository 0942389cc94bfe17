// Pre-projection kernels of the tile path.
//
// Algorithm 1 (inference step) evaluates the correction as (H B_w^T) A_w^T;
// the quantised core A_c B_c is evaluated the same way.  These kernels form
// Z = H [B_c_hat ; B_w_hat]^T once per call (r dot products of length D per
// token, fp32), and convert H into the fp16 MFMA operand the tile kernel
// streams:
//   hf  : H * 2^S_n in fp16, S_n chosen per token so the row maximum lands in
//         [2^14, 2^15); every bf16 value at most 2^31 below the row maximum is
//         then exact in fp16.  hscale[n] = 2^-S_n undoes it in the epilogue.
//   zf  : Z * 2^F_n split into fp16 hi + lo (22 significant bits), per-token
//         exponent F_n chosen the same way; zscale[n] = 2^-F_n.
// Both are stored in the operand order of the 32 x 32 x 16 MFMA (see
// device_common.h) so the tile kernel reads each operand fragment (32 rows x
// 16 columns) as one contiguous 1 KB block (layouts in internal.h).
//
// They are produced in three passes: prep_h32_kernel converts
// H; zmm_kernel forms Z on the 32 x 32 x 16 MFMA from that fp16 H and the
// exact INT8 B codes (so B is read once per 32-token tile, not once per
// token); zsplit_kernel picks F_n and writes the hi/lo fragments.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace archead {

namespace {

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
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

// Z on the MFMA, grid (n32/32 token tiles, ceil(r/32) rank blocks, S parts of
// the k range), 16 waves: wave w takes slice w of its part's k range (whole
// groups) for the workgroup's 32 tokens and 32 ranks.  MFMA A operand = hf
// fragments (tokens), B operand = the exact INT8 codes of the same 16 columns
// (ranks); each group of g columns is accumulated on its own and added times
// its fp16 scale.  The slices are summed through LDS and
// z32[part][n][j] = hscale[n] * sum is written; zsplit_kernel adds the parts
// in order (S > 1 only when the token and rank tiles alone would leave most
// CUs idle).
// GC: group size 0 -> g >= 128, 1 -> 64, 2 -> 32 (steps of a k-tile per group).
constexpr int kZmmWaves = 16;
template <int GC>
__global__ __launch_bounds__(64 * kZmmWaves) void zmm_kernel(const FwdArgs a, int parts) {
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
  const int p0 = (int)blockIdx.z * units / parts, pn = ((int)blockIdx.z + 1) * units / parts - p0;
  const int u0 = p0 + wave * pn / kZmmWaves, u1 = p0 + (wave + 1) * pn / kZmmWaves;
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
    if (jj < r) a.z32[((int64_t)blockIdx.z * a.n32 + n) * r + jj] = z * a.hscale[n];
  }
}

// One wave per token row n < n32: F_n from max_j |z32[n][j]|, zscale[n] =
// 2^-F_n (0 for padding rows), zf = fp16 hi/lo split of z * 2^F_n in the
// 32-row layout: fragments of 16 ranks, steps in pairs (2i, 2i+1) whose lane
// half q holds ranks 32 i + 16 q + 8 (s & 1) .. (one 16-byte load of A codes
// feeds both steps of a pair), slot order k_order_z.
constexpr int kZsplitThreads = 256;
__global__ __launch_bounds__(kZsplitThreads) void zsplit_kernel(const FwdArgs a, int parts) {
  const int lane = threadIdx.x & 63;
  const int64_t n = 4 * (int64_t)blockIdx.x + (threadIdx.x >> 6);
  if (n >= a.n32) return;
  const bool real = n < a.N;
  const int r = a.r_c + a.r_r;
  // z[j]: the parts of the k range added in order
  auto zrow = [&](int j) {
    float z = 0.0f;
    for (int p = 0; p < parts; ++p) z += a.z32[((int64_t)p * a.n32 + n) * r + j];
    return z;
  };
  float m = 0.0f;
  if (real)
    for (int j = lane; j < r; j += 64) m = fmaxf(m, fabsf(zrow(j)));
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
      if (real && col < rank) z = ldexpf(zrow(base + col), F);
      const _Float16 zh = (_Float16)z;
      hi[jj] = zh;
      lo[jj] = (_Float16)(z - (float)zh);
    }
    _Float16* dst = a.zf + ((tile * (2 * nsteps) + 2 * s) * 64 + 32 * q + i) * 8;
    *reinterpret_cast<h8*>(dst) = hi;
    *reinterpret_cast<h8*>(dst + 64 * 8) = lo;
  }
}

}  // namespace

// Parts of the k range zmm_kernel splits Z into: at least about 128
// workgroups (half the CUs), at least one unit of whole groups per wave of a
// part; one part once the token and rank tiles alone reach that.
int zmm_parts(int64_t n32, int r, int64_t D, int g) {
  const int64_t base = (n32 / 32) * ((r + 31) / 32);
  const int64_t kpu = g > kKTile ? g / kKTile : 1;
  const int64_t units = D / kKTile / kpu;
  int64_t p = base > 0 ? (128 + base - 1) / base : 1;
  p = std::min<int64_t>(p, units / kZmmWaves);
  return p < 1 ? 1 : (int)p;
}

hipError_t launch_prep(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prep_h32_kernel, dim3((unsigned)((a.n32 + 3) / 4)), dim3(kPrepHThreads), 0, s, a);
  const int r = a.r_c + a.r_r;
  const int parts = r > 0 ? zmm_parts(a.n32, r, a.D, a.g) : 1;
  if (r > 0) {
    const dim3 grid((unsigned)(a.n32 / 32), (unsigned)((r + 31) / 32), (unsigned)parts);
    if (a.g == 32)
      hipLaunchKernelGGL(zmm_kernel<2>, grid, dim3(64 * kZmmWaves), 0, s, a, parts);
    else if (a.g == 64)
      hipLaunchKernelGGL(zmm_kernel<1>, grid, dim3(64 * kZmmWaves), 0, s, a, parts);
    else
      hipLaunchKernelGGL(zmm_kernel<0>, grid, dim3(64 * kZmmWaves), 0, s, a, parts);
  }
  hipLaunchKernelGGL(zsplit_kernel, dim3((unsigned)((a.n32 + 3) / 4)), dim3(kZsplitThreads), 0, s, a, parts);
  return hipGetLastError();
}

}  // namespace archead
