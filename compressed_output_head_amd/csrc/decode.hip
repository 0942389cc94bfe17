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
  const u4* wbase = reinterpret_cast<const u4*>(a.r_codes) + (blk0 * a.nkt) * 64 + lane;
  const h8* hbase = reinterpret_cast<const h8*>(a.hf) + lane;

  for (int kt = 0; kt < a.nkt; ++kt) {
    u4 w[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b)
      w[b] = (b < nblk) ? __builtin_nontemporal_load(wbase + ((int64_t)b * a.nkt + kt) * 64)
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
              ? (float)a.r_gcodes[((blk0 + b) * a.ng + grp) * 16 + i16] : 0.0f;
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
