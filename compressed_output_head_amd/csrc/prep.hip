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
// 32 x 32 x 16 MFMA kernel (layouts in internal.h).
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

// One workgroup per token row n (rows N..n16-1, or N..n32-1 for the 32-row
// layout, are zero padding):
//   1. S_n from max|H[n,:]|; hf = fp16(H[n,:] * 2^S_n)
//   2. z[j] = sum_k H[n,k] B_hat[j,k] for all j < r (fp32, one wave per j, kept in LDS)
//   3. F_n from max_j |z[j]|; zf = fp16 hi/lo split of z * 2^F_n
//
// 32-row layout: within a 128-column k-tile, 8-column run R (0..15) of token
// n goes to MFMA step t = (R >> 2) + 4 * ((R >> 1) & 1), lane (n & 31) + 32 * (R & 1);
// the residual codes are read in the same run order (tile32_kernel).
template <bool ROWS32>
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
    __shared__ float red[kPrepZThreads / 64];
    float m = 0.0f;
    for (int c = tid; c < nchunk; c += kPrepZThreads) {
      const u4 raw = *reinterpret_cast<const u4*>(hrow + 8 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(raw[w] & 0xffffu))));
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(raw[w] >> 16))));
      }
    }
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int S = row_exponent(m);
    if (tid == 0) a.hscale[n] = ldexpf(1.0f, -S);
    for (int c = tid; c < nchunk; c += kPrepZThreads) {
      const u4 raw = *reinterpret_cast<const u4*>(hrow + 8 * c);
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
    }
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
  if (rows32)
    hipLaunchKernelGGL(prep_kernel<true>, dim3((unsigned)a.n32), dim3(kPrepThreads), 0, s, a);
  else
    hipLaunchKernelGGL(prep_kernel<false>, dim3((unsigned)a.n16), dim3(kPrepThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace archead
