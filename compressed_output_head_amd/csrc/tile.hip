// Tile path (any N the few-token decode kernel does not take): the 32-row
// tile kernel (tile32.h) when every section fits 32-bit buffer offsets, else
// the 16-row LDS-tiled kernel below.
//
// Y = [H | Z] [R | A_c ; A_w]^T, i.e. Algorithm 1's inference step with the
// quantised core evaluated through the same (H B^T) A^T association.
//
// 16-row kernel: a workgroup owns a TM x TN (tokens x vocabulary) output tile and walks the
// hidden dimension in 128-column steps.  Per step it copies the TM token rows
// of hf (already fp16 operand fragments) into LDS, and unpacks the TN/16
// residual tiles from their packed INT4 form into LDS as exact fp16 integers
// q4 * c8 (|q4 * c8| <= 2040, so the group code folds in with no rounding).
// Waves then run v_mfma_f32_16x16x32_f16 on LDS fragments.  The fp16 row scale
// s_R, the per-token exponent and the low-rank term (fp16 hi/lo Z against
// exact INT8 A codes, one accumulator per part) are applied in the epilogue.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "rowstat.h"

namespace archead {

namespace {

template <int TM, int TN, int WM, int WN>
struct TileCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kMT = TM / WM / 16;  // token tiles per wave
  static constexpr int kNB = TN / WN / 16;  // vocabulary blocks per wave
  static constexpr int kHT = TM / 16;       // token tiles per workgroup
  static constexpr int kWB = TN / 16;       // vocabulary blocks per workgroup
};

template <int TM, int TN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void tile_kernel(const FwdArgs a) {
  using C = TileCfg<TM, TN, WM, WN>;
  __shared__ h8 sH[C::kHT][4][64];
  __shared__ h8 sW[C::kWB][4][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t blk0 = (int64_t)blockIdx.x * C::kWB;
  const int64_t tt0 = (int64_t)blockIdx.y * C::kHT;  // first token tile
  const int64_t ntiles = a.n16 >> 4;

  f4 acc[C::kMT][C::kNB];
#pragma unroll
  for (int m = 0; m < C::kMT; ++m)
#pragma unroll
    for (int n = 0; n < C::kNB; ++n) acc[m][n] = f4{0.f, 0.f, 0.f, 0.f};

  const h8* hf = reinterpret_cast<const h8*>(a.hf);
  const u4* rc = reinterpret_cast<const u4*>(a.r_codes);

  for (int kt = 0; kt < a.nkt; ++kt) {
    for (int p = tid; p < C::kHT * 256; p += C::kThreads) {
      const int ht = p >> 8, s = (p >> 6) & 3, l = p & 63;
      const int64_t T = tt0 + ht;
      sH[ht][s][l] = (T < ntiles) ? hf[((T * a.nks) + 4 * kt + s) * 64 + l]
                                  : h8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    for (int p = tid; p < C::kWB * 64; p += C::kThreads) {
      const int wb = p >> 6, l = p & 63;
      const int64_t B = blk0 + wb;
      if (B < a.nb) {
        const u4 w = rc[((int64_t)kt * a.nb + B) * 64 + l];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int grp = (kKTile * kt + 32 * s + 8 * (l >> 4)) / a.g;
          const _Float16 c = (_Float16)(float)a.r_gcodes[(B * 16 + (l & 15)) * a.ng + grp];
          sW[wb][s][l] = unpack_q4_scaled(w[s], c);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) sW[wb][s][l] = h8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h8 av[C::kMT];
#pragma unroll
      for (int m = 0; m < C::kMT; ++m) av[m] = sH[wm * C::kMT + m][s][lane];
#pragma unroll
      for (int n = 0; n < C::kNB; ++n) {
        const h8 bv = sW[wn * C::kNB + n][s][lane];
#pragma unroll
        for (int m = 0; m < C::kMT; ++m) acc[m][n] = mfma16(av[m], bv, acc[m][n]);
      }
    }
    __syncthreads();
  }

  // epilogue: row scales, low-rank term, store
  const int r = a.r_c + a.r_r;
  const int csteps = a.rc32 / 32, wsteps = a.rr32 / 32;
  const h8* zf = reinterpret_cast<const h8*>(a.zf);
#pragma unroll
  for (int n = 0; n < C::kNB; ++n) {
    const int64_t B = blk0 + wn * C::kNB + n;
    if (B >= a.nb) continue;
    const int64_t v = 16 * B + i16;
    const float sR = f16_to_f32(a.r_rowscale[v]);
    const float sAc = a.r_c > 0 ? f16_to_f32(a.a_scales[v * a.nA]) : 0.0f;
    const float sAw = a.r_r > 0 ? f16_to_f32(a.a_scales[v * a.nA + a.nA - 1]) : 0.0f;
    f4 pc[C::kMT], pw[C::kMT];
#pragma unroll
    for (int m = 0; m < C::kMT; ++m) {
      pc[m] = f4{0.f, 0.f, 0.f, 0.f};
      pw[m] = f4{0.f, 0.f, 0.f, 0.f};
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
      for (int m = 0; m < C::kMT; ++m) {
        const int64_t T = tt0 + wm * C::kMT + m;
        if (T >= ntiles) continue;
        const h8 zh = zf[((T * 2 * a.zsteps) + 2 * s) * 64 + lane];
        const h8 zl = zf[((T * 2 * a.zsteps) + 2 * s + 1) * 64 + lane];
        if (part_c) {
          pc[m] = mfma16(zh, av, pc[m]);
          pc[m] = mfma16(zl, av, pc[m]);
        } else {
          pw[m] = mfma16(zh, av, pw[m]);
          pw[m] = mfma16(zl, av, pw[m]);
        }
      }
    }
    if (v >= a.V) continue;
#pragma unroll
    for (int m = 0; m < C::kMT; ++m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t tok = 16 * (tt0 + wm * C::kMT + m) + 4 * q + e;
        if (tok >= a.N) continue;
        float y = a.hscale[tok] * (sR * acc[m][n][e]);
        if (r > 0) y = fmaf(a.zscale[tok], fmaf(sAw, pw[m][e], sAc * pc[m][e]), y);
        if (a.y_bf16)
          reinterpret_cast<uint16_t*>(a.Y)[tok * a.Y_stride + v] = f32_to_bf16(y);
        else
          reinterpret_cast<float*>(a.Y)[tok * a.Y_stride + v] = y;
      }
    }
  }
}

}  // namespace

}  // namespace archead

#include "tile32.h"

namespace archead {

// The 32 x 32 x 16 kernel serves any N whose sections fit 32-bit buffer
// offsets and whose group codes fit the workgroup's LDS table.
bool tile32_eligible(const FwdArgs& a) {
  if ((uint64_t)a.nb * 16 * (uint64_t)a.D / 2 >= (1ull << 32)) return false;
  if (a.ng > kT32MaxCodes) return false;
  if (((uint64_t)a.nb * 16 + kT32CB * 32) * (uint64_t)a.ng >= (1ull << 32)) return false;
  if ((uint64_t)a.n32 * (uint64_t)a.D * 2 >= (1ull << 32)) return false;
  const T32Grid G = t32_grid(a, t32_tt(a));
  return (int64_t)G.ttiles * G.vtiles < (1ll << 31);
}

hipError_t launch_tile(const FwdArgs& a, hipStream_t s) {
  if (tile32_eligible(a)) {
    switch (t32_tt(a)) {
      case 2: return launch_t32<2, false>(a, s);
      case 4: return launch_t32<4, false>(a, s);
      default: return launch_t32<8, false>(a, s);
    }
  }
  constexpr int TM = 64, TN = 64, WM = 2, WN = 2;
  using C = TileCfg<TM, TN, WM, WN>;
  const int64_t gx = (a.nb + C::kWB - 1) / C::kWB;
  const int64_t gy = ((a.n16 >> 4) + C::kHT - 1) / C::kHT;
  if (gy > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((tile_kernel<TM, TN, WM, WN>), dim3((unsigned)gx, (unsigned)gy),
                     dim3(C::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace archead
