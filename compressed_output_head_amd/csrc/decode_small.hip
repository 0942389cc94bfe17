// Decode path for a few tokens (N <= 16 at D = 4096): a per-token
// pre-projection kernel, then a streaming kernel whose workgroups each hold a
// copy of H and Z in LDS: two workgroups of 8 waves per CU when a copy fits
// 76 KiB (N <= 8 at D = 4096), else one workgroup of 16 waves per CU with one
// copy of up to 152 KiB.
//
// Y = H W_d^T + (H B_w^T) A_w^T (Algorithm 1, inference step) with
// W_d = Q(A_c)Q(B_c) + SC4(R) (Sec. 3, quantized-core equation); the core is
// evaluated through the same association, (H B_c^T) A_c^T.
//
// Pre-projection, grid (N, S ceil(r/4) + 1): z32[s][n][j] = sum over the
// columns k of slice s of H[n,k] B_hat[j,k] in fp32, one wave per (slice,
// token, rank) (S = 1 for the batched kernel; the few-token kernel adds the S
// slices in order), and for each token hscale[n] = 2^-S_n
// and hc[n][:] = fp16(H[n,:] 2^S_n) in kernel k-order, S_n putting the row
// maximum in [2^14, 2^15) (exact for every bf16 value within 2^31 of it).
//
// Streaming kernel: every wave walks a grid-strided list of 16-row vocabulary
// blocks and keeps a ring of packed tiles in flight; per 32-column step one
// v_mfma_f32_16x16x32_f16 (H fp16 from LDS against the INT4 codes as exact
// fp16 integers), each g-column group's sum times its uint8 code once; a
// block's epilogue adds the low-rank term (Z hi/lo against the exact INT8 A
// codes, one accumulator per part) and the fp16 row scale s_R.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace archead {

namespace {

constexpr int kSmallMaxTokens = 16;       // token rows of the per-WG arrays
constexpr uint64_t kSmallLdsBytes = 76 * 1024;  // H and Z per workgroup: two fit a CU
constexpr uint64_t kWideLdsBytes = 152 * 1024;  // one 16-wave workgroup per CU (160 KiB of LDS)

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Small-N pre-projection, grid (N, S ceil(r/4) + 1) with S = a.zsl slices of D:
//   blockIdx.y < S ceil(r/4): z32[s][n][j] = sum over slice s of H[n,k] B_hat[j,k]
//     in fp32, one wave per (slice, token, j); every lane issues all its loads
//     before the arithmetic.
//   blockIdx.y == S ceil(r/4): hscale[n] = 2^-S_n and hc[n][:] = fp16(H[n,:] 2^S_n)
//     in kernel k-order (S_n as in prep_kernel).
constexpr int kSmallPrepThreads = 256;
constexpr int kSmallPrepChunks = 16;  // D <= 64*8*16 = 8192 columns per lane loop

__global__ __launch_bounds__(kSmallPrepThreads) void small_prep_kernel(const FwdArgs a) {
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r_c + a.r_r;
  const int nJ = (r + 3) / 4;
  const uint16_t* hrow = a.H + n * a.H_stride;
  const int nchunk = (int)(a.D / 8);
  const int nsl = a.zsl;
  if ((int)blockIdx.y == nJ * nsl) {
    // the row's first kSmallPrepKeep * 256 chunks stay in registers between the
    // maximum and the conversion (one read of H for D <= 8192)
    constexpr int kSmallPrepKeep = 4;
    __shared__ float red[kSmallPrepThreads / 64];
    u4 keep[kSmallPrepKeep];
#pragma unroll
    for (int i = 0; i < kSmallPrepKeep; ++i) {
      const int c = tid + i * kSmallPrepThreads;
      keep[i] = c < nchunk ? *reinterpret_cast<const u4*>(hrow + 8 * c) : u4{0u, 0u, 0u, 0u};
    }
    // f(chunk index, its 8 bf16 values) for every chunk of this thread
    auto each_chunk = [&](auto f) {
#pragma unroll
      for (int i = 0; i < kSmallPrepKeep; ++i)
        if (tid + i * kSmallPrepThreads < nchunk) f(tid + i * kSmallPrepThreads, keep[i]);
      for (int c = tid + kSmallPrepKeep * kSmallPrepThreads; c < nchunk; c += kSmallPrepThreads)
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
  const int sl = (int)blockIdx.y / nJ;
  const int j = ((int)blockIdx.y - sl * nJ) * (kSmallPrepThreads / 64) + wave;
  if (j >= r) return;
  const int8_t* brow = a.b_codes + (int64_t)j * a.D;
  const uint16_t* srow = a.b_scales + (int64_t)j * a.ng;
  // this wave's 8-column chunks: [c_lo, c_hi) of the row
  const int c_lo = (int)((int64_t)sl * nchunk / nsl), c_hi = (int)((int64_t)(sl + 1) * nchunk / nsl);
  float acc = 0.0f;
  for (int c0 = c_lo; c0 < c_hi; c0 += 64 * kSmallPrepChunks) {
    u4 hr[kSmallPrepChunks];
    u2 br[kSmallPrepChunks];
    uint16_t sr[kSmallPrepChunks];
#pragma unroll
    for (int u = 0; u < kSmallPrepChunks; ++u) {
      const int c = c0 + lane + 64 * u;
      if (c < c_hi) {
        hr[u] = *reinterpret_cast<const u4*>(hrow + 8 * (int64_t)c);
        br[u] = *reinterpret_cast<const u2*>(brow + 8 * (int64_t)c);
        sr[u] = srow[(8 * c) / a.g];
      }
    }
#pragma unroll
    for (int u = 0; u < kSmallPrepChunks; ++u) {
      const int c = c0 + lane + 64 * u;
      if (c < c_hi) {
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
  if (lane == 0) a.z32[((int64_t)sl * a.N + n) * r + j] = acc;
}


// ---------------------------------------------------------------------------
// Streaming kernel, persistent.
//
// The grid holds only co-resident workgroups: 16 waves per CU, two workgroups
// of NW = 8 waves or one of NW = 16 (launch bounds of four waves per SIMD, so
// at most 128 VGPRs a wave).  Measured on the decode workload, two 8-wave
// workgroups per CU are as fast as four of 4 waves for one token and faster
// for 4 to 8; three per CU (six waves per SIMD, 80 VGPRs and spills) are
// about 15% slower; one of 16 waves serves the copies of H that two would not
// fit, its waves a grid apart (with neighbouring blocks it was about 15%
// slower).
// Every wave walks a grid-strided list of 16-row blocks (b, b + W, b + 2W, ...
// with W the number of waves), so at any moment the waves read neighbouring
// 1 KB tiles of the same k-tile plane.  Each wave keeps a ring of
// P packed tiles in flight in registers, plus one vector of group codes per
// chunk of 4 tiles (the lane's row codes for 512 columns, one small load).  The
// ring runs across block boundaries, so a wave never drains its pipeline.  H
// (already scaled fp16 from the pre-projection kernel) and Z (fp32) sit in
// LDS; LDS reads use the separate lgkm counter and never wait behind the ring.
// MFMA rows past the tokens read a zero row of H in LDS.
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

template <int P, int G, int NW>
__global__ __launch_bounds__(64 * NW, 4) void small_decode_kernel(const FwdArgs a) {
  constexpr int kLdsWaves = NW;
  constexpr int kLdsThreads = 64 * NW;
  static_assert(P % 4 == 0, "the ring holds whole 4-tile code chunks");
  using CV = typename CodeVec<G>::T;
  constexpr int NC = P / 4;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float s_hs[kSmallMaxTokens];
  __shared__ int s_F[kSmallMaxTokens];
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

  // first block of this wave: the 16-wave workgroup spreads its waves a grid
  // apart (measured about 10% faster than 16 neighbouring blocks per CU for
  // 9 to 16 tokens); the 8-wave workgroups keep neighbouring blocks (the
  // spread measured no faster there)
  int64_t b = NW == 16 ? (int64_t)blockIdx.x + (int64_t)gridDim.x * wave : (int64_t)blockIdx.x * kLdsWaves + wave;
  const int64_t b0 = b < nb ? b : nb - 1;  // waves without work load a valid block, store nothing
  const int per_row = D / 8;

  // prologue, one round trip: this thread's first pieces of H, Z and the
  // token scales, then the weight ring, then those pieces into LDS.  Eight
  // 16-byte pieces a thread hold all of H at D = 4096 (up to 8 tokens in an
  // 8-wave workgroup, 16 in a 16-wave one); the loop after them serves
  // larger D, one round trip per pass.
  constexpr int kPre = 8;
  u4 hpre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int c = tid + i * kLdsThreads;
    hpre[i] = c < N * per_row ? *reinterpret_cast<const u4*>(a.hc + (int64_t)(c / per_row) * D + 8 * (c % per_row))
                              : u4{0u, 0u, 0u, 0u};
  }
  // Z = the sum of its slices' partial sums, added in slice order
  const int zs = a.zsl;
  auto zsum = [&](int c) {
    float z = 0.0f;
    for (int sl = 0; sl < zs; ++sl) z += a.z32[(int64_t)sl * N * r + c];
    return z;
  };
  const float zpre = tid < N * r ? zsum(tid) : 0.0f;
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
  for (int c = tid + kLdsThreads; c < N * r; c += kLdsThreads) sZ[c] = zsum(c);
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
    // the ring's next block; after the wave's last block the ring's loads go to
    // the head's last block, the same few lines for every wave (cache hits after
    // the first, never used; re-reading this block's first tiles, streamed long
    // before, would fetch them from memory again)
    const int64_t bnx = bn < nb ? bn : nb - 1;
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

constexpr int kRingDepth = 4;  // packed tiles in flight per wave

// CUs of the current device (256 if the runtime cannot tell)
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <int P, int G, int NW>
hipError_t launch_lds_p(const FwdArgs& a, hipStream_t s) {
  const size_t lds = lds_bytes(a.N, a.D, a.r_c + a.r_r);
  constexpr int kThreads = 64 * NW;
  if (lds > 64 * 1024) {  // dynamic LDS beyond 64 KiB is opted into per kernel
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&small_decode_kernel<P, G, NW>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  // persistent grid: never more workgroups than can be resident at once
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, small_decode_kernel<P, G, NW>, kThreads, lds) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  per_cu = std::min(per_cu, 16 / NW);
  const int64_t need = (a.nb + NW - 1) / NW;
  const int64_t grid = std::min<int64_t>(need, (int64_t)device_cu_count() * per_cu);
  return launch_main(small_decode_kernel<P, G, NW>, dim3((unsigned)grid), dim3(kThreads), (uint32_t)lds, s, true, a);
}

template <int G>
hipError_t launch_lds(const FwdArgs& a, hipStream_t s) {
  // two workgroups of 8 waves per CU when their copies of H and Z fit, else one of 16
  if (lds_bytes(a.N, a.D, a.r_c + a.r_r) <= kSmallLdsBytes) return launch_lds_p<kRingDepth, G, 8>(a, s);
  return launch_lds_p<kRingDepth, G, 16>(a, s);
}

}  // namespace

bool small_decode_fits(const archead_dims* d, int64_t n_tokens) {
  if (n_tokens < 1 || n_tokens > kSmallMaxTokens || (d->D / kKTile) % 4 != 0) return false;
  if (d->g != 32 && d->g != 64 && d->g != 128 && d->g != 256) return false;
  if (lds_bytes(n_tokens, d->D, d->r_c + d->r_r) > kWideLdsBytes) return false;
  // 32-bit offsets into the residual tiles, the group codes and the A codes
  const uint64_t V16 = round_up((uint64_t)d->V, 16);
  return V16 * (uint64_t)d->D / 2 < (1ull << 32) && V16 * (uint64_t)(d->D / d->g) < (1ull << 32) &&
         V16 * (uint64_t)(d->r_c + d->r_r) < (1ull << 32);
}

hipError_t launch_small_decode(const FwdArgs& a, hipStream_t s) {
  switch (a.g) {
    case 32: return launch_lds<32>(a, s);
    case 64: return launch_lds<64>(a, s);
    case 128: return launch_lds<128>(a, s);
    default: return launch_lds<256>(a, s);
  }
}


// One to four 8-column chunks of a row per lane of a Z wave (more tokens,
// fewer slices: the few-token kernel reads S N r partial sums per workgroup).
int small_z_slices(int64_t D, int64_t n_tokens) {
  const int64_t cpl = n_tokens <= 2 ? 1 : n_tokens <= 8 ? 2 : 4;
  const int64_t sl = D / (512 * cpl);
  return sl < 1 ? 1 : (int)sl;
}

hipError_t launch_small_prep(const FwdArgs& a, hipStream_t s) {
  const int r = a.r_c + a.r_r;
  hipLaunchKernelGGL(small_prep_kernel, dim3((unsigned)a.N, (unsigned)(a.zsl * ((r + 3) / 4) + 1)),
                     dim3(kSmallPrepThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace archead
