// Packing step of the construction (ARCHead, Algorithm 1 and the Sec. 3
// quantized-core sentence) on the GPU: quantise the core factors to INT8,
// compute the residual the quantised core leaves, R = W - Q(A_c) Q(B_c), and
// store it as SC4; quantise the correction factors to INT8; write everything
// in the packed format (archead_pack_layout).
//
// The page fixes no rounding rule, scale formula or range.  Readings (the
// same as the CPU reference): symmetric absmax scaling, round half to even;
//   INT8 (rows of A, g-column groups of rows of B): s = fp16(amax / 127),
//     code = clamp(rint(x / s), -127, 127), 0 where s = 0;
//   SC4 (rows of R in g-column groups, m_t = the group's amax):
//     s_R = fp16(max_t m_t / (7 * 255)), c8_t = clamp(ceil(m_t / (7 s_R)), 1, 255),
//     q4 = clamp(rint(r / (c8_t s_R)), -8, 7); s_R = 0 gives c8 = 0, q4 = 0.
// Every decision is taken in fp32 (IEEE division, rint, round to fp16); the
// residual is accumulated in fp64 over the core rank in index order, each
// product being exact, and rounded once to fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "archead.h"
#include "device_common.h"
#include "quantize.h"

namespace archead {

namespace {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / 64;
constexpr int kQMaxRunsPerThread = kQuantMaxD / (8 * kQThreads);  // 8-column runs per thread
constexpr int kQTermBatch = 4;                                     // core terms loaded together

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// INT8 of nseg segments of len values, one wave per segment.  Segment p is
// part t = p % spr of row i = p / spr: values M[i * m_ld + t * len + k],
// codes[i * c_ld + t * len + k], scale scales[i * s_ld + t].
__global__ __launch_bounds__(kQThreads) void quant_i8_kernel(const float* M, int64_t m_ld, int spr, int len,
                                                             int64_t nseg, int8_t* codes, int64_t c_ld,
                                                             uint16_t* scales, int64_t s_ld) {
  const int lane = threadIdx.x & 63;
  const int64_t p = (int64_t)blockIdx.x * kQWaves + (threadIdx.x >> 6);
  if (p >= nseg) return;
  const int64_t i = p / spr;
  const int t = (int)(p - i * spr);
  const float* x = M + i * m_ld + (int64_t)t * len;
  float amax = 0.0f;
  for (int k = lane; k < len; k += 64) amax = fmaxf(amax, fabsf(x[k]));
  amax = wave_max_f(amax);
  const _Float16 s = (_Float16)(amax / 127.0f);
  const float s32 = (float)s;
  int8_t* q = codes + i * c_ld + (int64_t)t * len;
  for (int k = lane; k < len; k += 64)
    q[k] = s32 > 0.0f ? (int8_t)fminf(fmaxf(rintf(x[k] / s32), -127.0f), 127.0f) : (int8_t)0;
  if (lane == 0) scales[i * s_ld + t] = __builtin_bit_cast(uint16_t, s);
}

// RB vocabulary rows per workgroup: R = W - Q(A_c) Q(B_c), then SC4 and the
// packed residual tile bytes (4 bytes = one 8-column run), the group codes,
// the row scale and E = fp32(R) - SC4(R).  Thread t takes the 8-column runs
// t, t + 256, ... of all RB rows, so each dequantised B_c value (converted
// once) feeds RB fp64 multiply-adds; the dequantised A_c values of the RB rows
// sit in LDS as [j][RB].  Per element the core rank is accumulated in index
// order with one fma per term (each product is exact, so the fma rounds as
// the sum acc + a b does).
template <int RB, int NR>
__global__ __launch_bounds__(kQThreads) void core_sc4_kernel(const QuantArgs q) {
  extern __shared__ double sA[];  // [r_c][RB]
  __shared__ float sMax[kQWaves][RB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t v0 = (int64_t)blockIdx.x * RB;
  const int D = (int)q.D, g = q.g, ng = D / g, nruns = D / 8, gr = g / 8;  // runs per group: 4 .. 32
  for (int idx = tid; idx < q.r_c * RB; idx += kQThreads) {
    const int j = idx / RB, rr = idx % RB;
    const int64_t v = v0 + rr;
    sA[idx] = v < q.V ? (double)q.a_codes[v * q.r + j] * (double)half_bits_to_f32(q.a_scales[v * q.nA]) : 0.0;
  }
  __syncthreads();
  float R[RB][NR][8];
  float rmax[RB];
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) rmax[rr] = 0.0f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int run = tid + kQThreads * i;
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int e = 0; e < 8; ++e) R[rr][i][e] = 0.0f;  // runs past D and rows past V stay zero
    if (run < nruns) {
      const int k0 = 8 * run, t = k0 / g;
      double acc[RB][8];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[rr][e] = 0.0;
      // one term j of the core: codes c as unsigned bytes u = c + 128, and
      // u sb - 128 sb = c sb is exact in fp32 (an 8-bit code times an 11-bit
      // significand), so the fma returns it
      auto term = [&](const u2 braw, const uint16_t sbits, const int j) {
        const float sb = half_bits_to_f32(sbits);
        const float nsb = -128.0f * sb;
        const uint32_t x[2] = {braw[0] ^ 0x80808080u, braw[1] ^ 0x80808080u};
        double b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = (double)fmaf((float)((x[e >> 2] >> (8 * (e & 3))) & 0xffu), sb, nsb);
        double a[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) a[rr] = sA[j * RB + rr];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[rr][e] = fma(a[rr], b[e], acc[rr][e]);
      };
      const int8_t* bp = q.b_codes + k0;
      const uint16_t* sp = q.b_scales + t;
      int j = 0;
      for (; j + kQTermBatch <= q.r_c; j += kQTermBatch) {  // the batch's loads are in flight together
        u2 br[kQTermBatch];
        uint16_t sh[kQTermBatch];
#pragma unroll
        for (int u = 0; u < kQTermBatch; ++u) {
          br[u] = *reinterpret_cast<const u2*>(bp + (int64_t)(j + u) * D);
          sh[u] = sp[(int64_t)(j + u) * ng];
        }
#pragma unroll
        for (int u = 0; u < kQTermBatch; ++u) term(br[u], sh[u], j + u);
      }
      for (; j < q.r_c; ++j) term(*reinterpret_cast<const u2*>(bp + (int64_t)j * D), sp[(int64_t)j * ng], j);
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int64_t v = v0 + rr;
        if (v < q.V) {
          double w[8];
          if (q.w_bf16) {
            const u4 raw =
                *reinterpret_cast<const u4*>(reinterpret_cast<const uint16_t*>(q.W) + v * q.W_stride + k0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[2 * e] = (double)bf16_to_f32((uint16_t)(raw[e] & 0xffffu));
              w[2 * e + 1] = (double)bf16_to_f32((uint16_t)(raw[e] >> 16));
            }
          } else {
            const float* wf = reinterpret_cast<const float*>(q.W) + v * q.W_stride + k0;
            const f4 lo = *reinterpret_cast<const f4*>(wf), hi = *reinterpret_cast<const f4*>(wf + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] = (double)lo[e];
              w[4 + e] = (double)hi[e];
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            R[rr][i][e] = (float)(w[e] - acc[rr][e]);
            rmax[rr] = fmaxf(rmax[rr], fabsf(R[rr][i][e]));
          }
        }
      }
    }
  }
  // row maxima over the workgroup
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    const float m = wave_max_f(rmax[rr]);
    if (lane == 0) sMax[wave][rr] = m;
  }
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    float m = sMax[0][rr];
#pragma unroll
    for (int w = 1; w < kQWaves; ++w) m = fmaxf(m, sMax[w][rr]);
    rmax[rr] = m;
  }
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    const int64_t v = v0 + rr;
    const _Float16 sR = (_Float16)(rmax[rr] / (7.0f * 255.0f));
    const float sR32 = (float)sR;
    const float den = 7.0f * sR32;  // exact
    if (tid == 0 && v < q.V) q.r_rowscale[v] = __builtin_bit_cast(uint16_t, sR);
    const int64_t b = v / 16;
    const int i16 = (int)(v % 16);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int run = tid + kQThreads * i;
      // group maximum: a group is gr consecutive runs, held by gr consecutive lanes
      float gm = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) gm = fmaxf(gm, fabsf(R[rr][i][e]));
      for (int off = 1; off < gr; off <<= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
      if (run < nruns && v < q.V) {
        const int k0 = 8 * run;
        const float c8 = sR32 > 0.0f ? fminf(fmaxf(ceilf(gm / den), 1.0f), 255.0f) : 0.0f;
        if (run % gr == 0) q.r_gcodes[v * ng + k0 / g] = (uint8_t)c8;
        const float scale = c8 * sR32;  // exact
        uint32_t word = 0u;
        float deq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = scale > 0.0f ? fminf(fmaxf(rintf(R[rr][i][e] / scale), -8.0f), 7.0f) : 0.0f;
          deq[e] = c * scale;  // exact
          word |= ((uint32_t)(int)c & 0xFu) << (4 * e);
        }
        // tile (b, kt) of the packed residual; lane row i16 + 16 (k mod 32) / 8,
        // dword (k mod 128) / 32 holds these 8 codes, low nibble first
        const int kt = k0 / 128, kk = k0 % 128;
        const int64_t off = ((int64_t)kt * q.nb + b) * 1024 + 16 * (i16 + 16 * ((kk % 32) / 8)) + 4 * (kk / 32);
        *reinterpret_cast<uint32_t*>(q.r_codes + off) = word;
        if (q.E) {
          float* er = q.E + v * q.E_stride + k0;
          const float(&x)[8] = R[rr][i];
          *reinterpret_cast<f4*>(er) = f4{x[0] - deq[0], x[1] - deq[1], x[2] - deq[2], x[3] - deq[3]};
          *reinterpret_cast<f4*>(er + 4) = f4{x[4] - deq[4], x[5] - deq[5], x[6] - deq[6], x[7] - deq[7]};
        }
      }
    }
  }
}

// Zero n16 16-byte words (padding rows and the gaps between sections stay 0).
__global__ __launch_bounds__(kQThreads) void zero_kernel(u4* p, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * kQThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kQThreads + threadIdx.x; i < n16; i += stride) p[i] = u4{0u, 0u, 0u, 0u};
}

// The 64-byte header: magic, version, V, D, r_c, r_r, g, flags 0, zeros.
__global__ void header_kernel(uint8_t* buf, uint64_t V, uint64_t D, uint32_t r_c, uint32_t r_r, uint32_t g) {
  if (threadIdx.x != 0) return;
  uint32_t* w = reinterpret_cast<uint32_t*>(buf);
  w[0] = ARCHEAD_MAGIC;
  w[1] = ARCHEAD_FORMAT_VERSION;
  w[2] = (uint32_t)V;
  w[3] = (uint32_t)(V >> 32);
  w[4] = (uint32_t)D;
  w[5] = (uint32_t)(D >> 32);
  w[6] = r_c;
  w[7] = r_r;
  w[8] = g;
}

hipError_t quant_i8(const float* M, int64_t m_ld, int spr, int len, int64_t nseg, int8_t* codes, int64_t c_ld,
                    uint16_t* scales, int64_t s_ld, hipStream_t s) {
  if (nseg <= 0 || len <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_i8_kernel, dim3((unsigned)((nseg + kQWaves - 1) / kQWaves)), dim3(kQThreads), 0, s, M,
                     m_ld, spr, len, nseg, codes, c_ld, scales, s_ld);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_core(const QuantArgs& q, const float* A_c, const float* B_c, uint64_t total_bytes,
                                hipStream_t s) {
  const uint64_t n16 = total_bytes / 16;
  const unsigned zb = (unsigned)std::min<uint64_t>((n16 + kQThreads - 1) / kQThreads, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(zb), dim3(kQThreads), 0, s, reinterpret_cast<u4*>(q.buf), n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(header_kernel, dim3(1), dim3(64), 0, s, q.buf, (uint64_t)q.V, (uint64_t)q.D, (uint32_t)q.r_c,
                     (uint32_t)(q.r - q.r_c), (uint32_t)q.g);
  const int ng = (int)(q.D / q.g);
  if (q.r_c > 0) {
    // A_c: rows into a_codes columns [0, r_c), scales column 0; B_c: groups into rows [0, r_c)
    if ((e = quant_i8(A_c, q.r_c, 1, q.r_c, q.V, q.a_codes, q.r, q.a_scales, q.nA, s)) != hipSuccess) return e;
    if ((e = quant_i8(B_c, q.D, ng, q.g, (int64_t)q.r_c * ng, q.b_codes, q.D, q.b_scales, ng, s)) != hipSuccess)
      return e;
  }
  {
    // rows per workgroup x runs per thread: at most 16 register runs of 8 fp32
    const int nr = (int)((q.D / 8 + kQThreads - 1) / kQThreads);  // runs per thread
    const int rb = nr <= 2 ? 8 : 4;
    const dim3 grid((unsigned)((q.V + rb - 1) / rb));
    const size_t lds = (size_t)q.r_c * rb * sizeof(double);
    if (nr <= 1)
      hipLaunchKernelGGL((core_sc4_kernel<8, 1>), grid, dim3(kQThreads), lds, s, q);
    else if (nr <= 2)
      hipLaunchKernelGGL((core_sc4_kernel<8, 2>), grid, dim3(kQThreads), lds, s, q);
    else
      hipLaunchKernelGGL((core_sc4_kernel<4, kQMaxRunsPerThread>), grid, dim3(kQThreads), lds, s, q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize_corr(const QuantArgs& q, const float* A_w, const float* B_w, hipStream_t s) {
  const int ng = (int)(q.D / q.g);
  const int r_r = q.r - q.r_c;
  if (r_r <= 0) return hipSuccess;
  hipError_t e = quant_i8(A_w, r_r, 1, r_r, q.V, q.a_codes + q.r_c, q.r, q.a_scales + (q.nA - 1), q.nA, s);
  if (e != hipSuccess) return e;
  return quant_i8(B_w, q.D, ng, q.g, (int64_t)r_r * ng, q.b_codes + (int64_t)q.r_c * q.D, q.D,
                  q.b_scales + (int64_t)q.r_c * ng, ng, s);
}

hipError_t launch_quantize(const QuantArgs& q, const float* A_c, const float* B_c, const float* A_w,
                           const float* B_w, uint64_t total_bytes, hipStream_t s) {
  hipError_t e = launch_quantize_core(q, A_c, B_c, total_bytes, s);
  return e != hipSuccess ? e : launch_quantize_corr(q, A_w, B_w, s);
}

QuantArgs quant_args(const archead_dims* d, const archead_layout& L, void* packed, const void* W, int64_t W_stride,
                     bool w_bf16, float* E, int64_t E_stride) {
  uint8_t* buf = static_cast<uint8_t*>(packed);
  QuantArgs q{};
  q.W = W;
  q.W_stride = W_stride;
  q.w_bf16 = w_bf16;
  q.V = d->V;
  q.D = d->D;
  q.r_c = d->r_c;
  q.r = d->r_c + d->r_r;
  q.g = d->g;
  q.nA = (d->r_c > 0) + (d->r_r > 0);
  q.nb = L.padded_rows / 16;
  q.buf = buf;
  q.r_codes = buf + L.r_codes.offset;
  q.r_gcodes = buf + L.r_gcodes.offset;
  q.r_rowscale = reinterpret_cast<uint16_t*>(buf + L.r_rowscale.offset);
  q.a_codes = reinterpret_cast<int8_t*>(buf + L.a_codes.offset);
  q.a_scales = reinterpret_cast<uint16_t*>(buf + L.a_scales.offset);
  q.b_codes = reinterpret_cast<int8_t*>(buf + L.b_codes.offset);
  q.b_scales = reinterpret_cast<uint16_t*>(buf + L.b_scales.offset);
  q.E = E;
  q.E_stride = E_stride;
  return q;
}

}  // namespace archead

using namespace archead;

extern "C" {

int archead_quantize(const archead_dims* d, const archead_dense_head* src, void* packed, uint64_t packed_bytes,
                     archead_tensor* E, void* stream) {
  if (!d || !src || !packed || !src->W) return ARCHEAD_E_NULL;
  archead_layout L;
  int rc = archead_pack_layout(d, &L);
  if (rc) return rc;
  if (d->format != ARCHEAD_FMT_ARCHEAD) return ARCHEAD_E_UNSUPPORTED;  // writes an ARCHead-format head
  if (d->g != 32 && d->g != 64 && d->g != 128 && d->g != 256) return ARCHEAD_E_UNSUPPORTED;
  if (d->D > kQuantMaxD || d->r_c > kQuantMaxCoreRank || d->r_r > (1 << 16)) return ARCHEAD_E_UNSUPPORTED;
  if ((d->r_c > 0 && (!src->A_c || !src->B_c)) || (d->r_r > 0 && (!src->A_w || !src->B_w))) return ARCHEAD_E_NULL;
  if (src->W_dtype != ARCHEAD_BF16 && src->W_dtype != ARCHEAD_F32) return ARCHEAD_E_DTYPE;
  if (src->W_stride < d->D) return ARCHEAD_E_SHAPE;
  const int64_t welem = src->W_dtype == ARCHEAD_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(src->W) | (uintptr_t)(src->W_stride * welem)) % 16) return ARCHEAD_E_ALIGN;
  for (const float* f : {src->A_c, src->B_c, src->A_w, src->B_w})
    if (reinterpret_cast<uintptr_t>(f) % 4) return ARCHEAD_E_ALIGN;
  if (reinterpret_cast<uintptr_t>(packed) % ARCHEAD_ALIGNMENT) return ARCHEAD_E_ALIGN;
  if (packed_bytes < L.total_bytes) return ARCHEAD_E_SIZE;
  if (E) {
    if (!E->data) return ARCHEAD_E_NULL;
    if (E->dtype != ARCHEAD_F32) return ARCHEAD_E_DTYPE;
    if (E->rows != d->V || E->cols != d->D || E->row_stride < d->D) return ARCHEAD_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(E->data) | (uintptr_t)(E->row_stride * 4)) % 16) return ARCHEAD_E_ALIGN;
  }
  const QuantArgs q = quant_args(d, L, packed, src->W, src->W_stride, src->W_dtype == ARCHEAD_BF16,
                                 E ? static_cast<float*>(E->data) : nullptr, E ? E->row_stride : 0);
  const hipError_t e =
      launch_quantize(q, src->A_c, src->B_c, src->A_w, src->B_w, L.total_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ARCHEAD_OK : ARCHEAD_E_HIP;
}

}  // extern "C"
