// Decode path (up to 16 tokens): a small, wide kernel forms partial sums of
// Z = H [B_c; B_w]^T, then one kernel streams the packed head once and
// writes Y.
//
// Y = H W_d^T + (H B_w^T) A_w^T (Algorithm 1, inference step) with
// W_d = Q(A_c)Q(B_c) + SC4(R) (Sec. 3, quantized-core equation); the core is
// evaluated through the same association, (H B_c^T) A_c^T.
//
// Z kernel: workgroup (slice sl, rank block j) of 4 waves; wave w takes two
// k-tiles (8 steps of 32 columns) of slice sl for the 16 ranks of block j on
// the 16 x 16 x 32 bf16 MFMA.  H is bf16 as given and every INT8 B code is
// an exact bf16, so each product is exact; each g-column group is summed on
// its own and added times its fp16 scale.  The waves' sums are added in LDS
// in wave order and written as zpart[(n r + k) zst + sl].
//
// Main kernel: one workgroup of 8 waves per CU.  The 16-row vocabulary
// blocks are dealt to all waves of the grid in contiguous ranges of at most
// MM blocks (ranges differ by at most one block).  Every wave walks the
// k-tiles in order and at k-tile kt reads tile (b, kt) of each of its blocks:
// tiles are stored k-tile major, so a workgroup reads one contiguous run of
// about 8 MM KB per step, and each wave keeps K k-tiles of loads in flight.
// Per 32-column step, per block: one v_mfma_f32_16x16x32_f16 with operand A =
// 16 token rows of H from LDS (fp16 times a per-token power of two: exact for
// every bf16 value within 2^31 of the row maximum) and operand B = 16
// vocabulary rows of INT4 codes as exact fp16 integers; one H fragment serves
// every block of the wave.  Each g-column group's sum is multiplied by its
// uint8 group code once.  The group codes of a block's rows are loaded once:
// the four lanes of a row hold a quarter of its codes each, and each step
// takes the dword it needs from the right lane (ds_bpermute), so the loop
// issues nothing but the 1 KB tile loads.
//
// Prologue: H into LDS (converted, zero row N for MFMA lanes with no token);
// Z = the sum of the slices' partial sums in slice order, split per token
// into fp16 hi + lo (22 significant bits) times a power of two.  Epilogue per
// block: Z hi/lo against the exact INT8 A codes (one accumulator per part, so
// each part gets its own row scale) and the fp16 row scale s_R.  No atomics
// on results: every run gives the same bits.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace archead {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecMaxRank32 = 256;   // rc32 + rr32: 32-rank steps of the epilogue
constexpr int kHChunks = 16;         // 16-byte pieces of H per thread in the prologue
constexpr int kEpiLoads = 8;         // 1 KB loads of A codes a wave holds: 16 MM r <= 8 KB
constexpr int kZWaves = 4;           // Z kernel: waves per workgroup
constexpr int kZKts = 2;             // Z kernel: k-tiles per wave
constexpr int kZSliceKts = kZWaves * kZKts;
constexpr int kZMaxSlices = 8;       // k-tiles <= 64 (D <= 8192)

// Cache policy of a buffer access: non-temporal (the nt bit of gfx950).
constexpr int kNonTemporal = 2;

// LDS carve-up (byte offsets), shared by the kernel and its launcher.  Two
// staging areas overlap the others: each wave's group codes (prologue, read
// back before H is written) and each wave's epilogue operands (after the
// main loop, over H and Z fp32).
struct DecLds {
  uint32_t z0;   // a zero row of H (MFMA lanes with no token read it)
  uint32_t h;    // H fp16 [N][D + 8]
  uint32_t zt;   // Z fp32 [N][r]
  uint32_t zf;   // Z hi/lo fragments [rank steps][2][64 lanes] h8
  uint32_t tok;  // per token: hscale, zscale, max |H| (float [16][4])
  uint32_t stp;  // prologue: wave w's group codes at h + w stp
  uint32_t ste;  // epilogue: wave w's A codes at w ste, its s_R at + esc, A scales at
  uint32_t esc;  //   + esc + 1024
  uint32_t total;
};

__host__ __device__ inline uint32_t dec_up(uint32_t x) { return (x + 15u) & ~15u; }

// KB-sized b128 loads (64 lanes x 16 bytes) a wave stages: its MM blocks'
// group codes (at most 16 WD bytes per row) and A codes (r bytes per row)
__host__ __device__ constexpr int code_loads(int MM, int WD) { return (MM * WD + 3) / 4; }
__host__ __device__ inline int acode_loads(int MM, int r) { return (MM * 16 * r + 1023) / 1024; }

__host__ __device__ inline DecLds dec_lds(int N, int D, int r, int rb32, int MM, int WD) {
  DecLds L;
  L.z0 = 0;
  L.h = dec_up((uint32_t)(D + 8) * 2u);
  L.zt = L.h + dec_up((uint32_t)N * (uint32_t)(D + 8) * 2u);
  L.stp = (uint32_t)code_loads(MM, WD) * 1024u + 16u;
  L.esc = (uint32_t)acode_loads(MM, r) * 1024u;
  L.ste = L.esc + 2048u;
  const uint32_t zfb = (uint32_t)(rb32 / 32) * 2u * 1024u;
  uint32_t zf = L.zt + dec_up((uint32_t)N * (uint32_t)r * 4u);
  if (zf < kDecWaves * L.ste) zf = kDecWaves * L.ste;
  L.zf = zf;
  uint32_t tok = L.zf + zfb;
  if (tok < L.h + kDecWaves * L.stp) tok = dec_up(L.h + kDecWaves * L.stp);
  L.tok = tok;
  L.total = L.tok + 16u * 4u * 4u;
  return L;
}

// Blocks of a workgroup's range [B0, B0 + cnt) dealt to its waves.  The
// four oldest waves of a workgroup (one per SIMD) win the issue arbitration
// and stream about an eighth faster than the four younger ones, so they take
// 9 parts against 8: wave w's blocks are [B0 + f(w), B0 + f(w + 1)) with
// f(w) = round(cnt * c(w) / 68), c(w) = 9 min(w, 4) + 8 max(w - 4, 0).
__host__ __device__ inline int wave_part(int w) { return 9 * (w < 4 ? w : 4) + 8 * (w > 4 ? w - 4 : 0); }
__host__ __device__ inline int wave_first(int cnt, int w) { return (int)(((int64_t)cnt * wave_part(w) + 34) / 68); }
// most blocks a wave gets when workgroups hold cnt or cnt - 1 blocks
__host__ inline int wave_blocks_max(int cnt) {
  int m = 0;
  for (int c = std::max(cnt - 1, 0); c <= cnt; ++c)
    for (int w = 0; w < 8; ++w) m = std::max(m, wave_first(c, w + 1) - wave_first(c, w));
  return m;
}

// slices of the Z kernel and the padded stride of its partial sums
__host__ __device__ inline int z_slices(int nkt) { return (nkt + kZSliceKts - 1) / kZSliceKts; }
__host__ __device__ inline int z_stride(int nkt) { return (z_slices(nkt) + 3) & ~3; }

// f(integral_constant<I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Workgroup barrier for LDS only: this wave's LDS accesses are complete, then
// every wave meets.  No memory fence: __syncthreads() would also wait for
// every global load in flight (the packed tiles).  The empty asm statements
// keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// ---------------------------------------------------------------------------
// Z kernel
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

// Eight INT8 codes (two dwords, column order) -> eight exact bf16 values, in order.
__device__ __forceinline__ bf8 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = i < 4 ? lo : hi;
    const float f = (float)(int8_t)((w >> (8 * (i & 3))) & 0xffu);
    b[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(f) >> 16));  // exact: 8 significant bits
  }
  return b;
}

__global__ __launch_bounds__(64 * kZWaves) void dec_zpart_kernel(const FwdArgs a, int zst) {
  __shared__ f4 red[kZWaves][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, q = lane >> 4;
  const int r = a.r_c + a.r_r, N = (int)a.N, D = (int)a.D, G = a.g;
  const int nsteps = 4 * a.nkt;
  const int k = 16 * (int)blockIdx.y + i16;  // rank of the B operand column
  const bool tv = i16 < N;                    // token row of the A operand
  const int st0 = 4 * ((int)blockIdx.x * kZSliceKts + wave * kZKts);
  constexpr int kSteps = 4 * kZKts;
  const uint32_t bbytes = (uint32_t)r * (uint32_t)D, sbytes = (uint32_t)r * (uint32_t)a.ng * 2u;
  const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(a.b_codes, bbytes);
  const __amdgpu_buffer_rsrc_t bss = buffer_rsrc(a.b_scales, sbytes);
  const uint16_t* hrow = a.H + (int64_t)(tv ? i16 : 0) * a.H_stride + 8 * q;
  // every load in flight at once; ranks past r and steps past the end read zero
  u2 bc[kSteps];
  u4 hb[kSteps];
  uint32_t sc[kSteps];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const int st = st0 + u;
    const bool live = st < nsteps;
    bc[u] = __builtin_bit_cast(
        u2, __builtin_amdgcn_raw_buffer_load_b64(
                brs, live ? (uint32_t)k * (uint32_t)D + 32u * (uint32_t)st + 8u * (uint32_t)q : bbytes, 0, 0));
    hb[u] = (tv && live) ? *reinterpret_cast<const u4*>(hrow + 32 * st) : u4{0u, 0u, 0u, 0u};
    sc[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
        bss, live ? 2u * ((uint32_t)k * (uint32_t)a.ng + (uint32_t)(32 * st / G)) : sbytes, 0, 0);
  }
  f4 acc = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const int st = st0 + u;
    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, hb[u]), i8x8_to_bf16(bc[u][0], bc[u][1]), p,
                                                 0, 0, 0);
    if ((32 * (st + 1)) % G == 0) {  // a group ends (every group ends in the range: 256 | 32 kSteps)
      acc += f16_to_f32((uint16_t)sc[u]) * p;
      p = f4{0.f, 0.f, 0.f, 0.f};
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f4 z = red[0][lane];
#pragma unroll
    for (int w = 1; w < kZWaves; ++w) z += red[w][lane];
    // lane: rank k, tokens 4 q + e
    if (k < r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 4 * q + e;
        if (n < N) a.z32[((int64_t)n * r + k) * zst + blockIdx.x] = z[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Main kernel.  MM: blocks per wave; WD: dwords of group codes a lane holds
// per block (its quarter of a row's D/g bytes).  K: k-tiles in flight.
template <int MM, int WD>
__global__ __launch_bounds__(kDecThreads, 1) void decode_kernel(const FwdArgs a, const DecLds L, int zst) {
  constexpr int K = MM >= 4 ? 2 : MM >= 2 ? 4 : 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = (int)a.N, D = (int)a.D, ldh = D + 8;
  const int r = a.r_c + a.r_r, G = a.g;
  const int nkt = a.nkt, ng = a.ng;
  const int i16 = lane & 15, q = lane >> 4;
  _Float16* sH = reinterpret_cast<_Float16*>(smem + L.h);
  _Float16* sH0 = reinterpret_cast<_Float16*>(smem + L.z0);
  float* sZt = reinterpret_cast<float*>(smem + L.zt);
  h8* sZf = reinterpret_cast<h8*>(smem + L.zf);
  float* sTok = reinterpret_cast<float*>(smem + L.tok);  // [16][4]: hscale, zscale, max |H| (bits)
  uint32_t* sTokU = reinterpret_cast<uint32_t*>(smem + L.tok);

  // this wave's blocks [bw0, bw0 + Mw), Mw <= MM: the workgroup's even share
  // of the blocks, dealt to its waves by wave_first
  static_assert(kDecWaves == 8, "wave_part assumes eight waves");
  const int B0 = (int)((int64_t)blockIdx.x * a.nb / gridDim.x);
  const int cnt = (int)((int64_t)(blockIdx.x + 1) * a.nb / gridDim.x) - B0;
  const int bw0 = B0 + wave_first(cnt, wave);
  const int Mw = B0 + wave_first(cnt, wave + 1) - bw0;

  // ---- prologue: loads of H, the group codes and the epilogue operands ---------
  // H chunk e of the N*D/8 (token e / nch, columns 8 (e % nch) ..) is thread
  // e % kDecThreads's number e / kDecThreads (the host keeps N*D/8 <= kHChunks * kDecThreads)
  const int nch = D / 8, hch = N * nch;
  u4 hv[kHChunks];
#pragma unroll
  for (int i = 0; i < kHChunks; ++i) {
    if (i * kDecThreads < hch) {  // uniform
      const int e = min(tid + i * kDecThreads, hch - 1), n = e / nch;
      hv[i] = *reinterpret_cast<const u4*>(a.H + (int64_t)n * a.H_stride + 8 * (e - n * nch));
    }
  }
  // group codes of the wave's blocks: rows [16 bw0, 16 (bw0 + Mw)), D/g bytes
  // each, contiguous and 16-byte aligned: a few 1 KB loads, staged in LDS below
  constexpr int CL = code_loads(MM, WD);
  const __amdgpu_buffer_rsrc_t crs = buffer_rsrc(a.r_gcodes, (uint32_t)a.nb * 16u * (uint32_t)ng);
  u4 cst[CL];
#pragma unroll
  for (int c = 0; c < CL; ++c)
    cst[c] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                        crs, (uint32_t)lane * 16u, (uint32_t)bw0 * 16u * (uint32_t)ng + 1024u * c, 0));

  // epilogue operands of the wave's rows, held in registers through the loop:
  // A codes [V16][r], s_R [V16] and A scales [V16][nA], each a contiguous,
  // 16-byte aligned run (1 KB per load; past a section's end: zero)
  const uint32_t v16 = (uint32_t)a.nb * 16u, r0 = (uint32_t)bw0 * 16u;
  const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(a.a_codes, v16 * (uint32_t)r);
  const __amdgpu_buffer_rsrc_t rrs = buffer_rsrc(a.r_rowscale, 2u * v16);
  const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(a.a_scales, 2u * v16 * (uint32_t)a.nA);
  const int nal = acode_loads(Mw, r);
  u4 eac[kEpiLoads];
#pragma unroll
  for (int c = 0; c < kEpiLoads; ++c)
    if (c < nal)
      eac[c] = __builtin_bit_cast(
          u4, __builtin_amdgcn_raw_buffer_load_b128(ars, 16u * lane, r0 * (uint32_t)r + 1024u * (uint32_t)c, 0));
  const u4 esR = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rrs, 16u * lane, 2u * r0, 0));
  const u4 esA =
      __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(srs, 16u * lane, 2u * r0 * (uint32_t)a.nA, 0));

  if (tid < kDecodeMaxTokens) sTokU[4 * tid + 2] = 0u;
  for (int c = tid; c < (D + 8) / 8; c += kDecThreads)
    *reinterpret_cast<u4*>(sH0 + 8 * c) = u4{0u, 0u, 0u, 0u};
  lds_barrier();  // the maxima start at zero

  // per-token maximum |H|
#pragma unroll
  for (int i = 0; i < kHChunks; ++i) {
    if (i * kDecThreads < hch) {
      float m = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(hv[i][w] & 0xffffu))));
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(hv[i][w] >> 16))));
      }
      const int e = tid + i * kDecThreads;
      if (nch % 64 == 0) {  // the wave's 64 chunks belong to one token
        const float mw = wave_max(m);
        if (lane == 0 && e < hch) atomicMax(&sTokU[4 * (e / nch) + 2], __float_as_uint(mw));
      } else if (e < hch) {
        atomicMax(&sTokU[4 * (e / nch) + 2], __float_as_uint(m));  // order-free: exact
      }
    }
  }

  // ---- the tile stream: tile (b, kt) at (kt*nb + b)*1024 --------------------------
  // A slot with no block, or a k-tile past the end, loads at a lane offset past
  // the section's end: zero, no traffic.  Every step issues the same loads, so
  // each wait counts exactly.
  const uint32_t tbytes = (uint32_t)a.nb * 16u * (uint32_t)(D / 2);
  const uint32_t tstride = (uint32_t)a.nb * 1024u;
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(a.r_codes, tbytes);
  const uint32_t wvoff = (uint32_t)lane * 16u;
  u4 wr[K][MM];
  auto issue = [&](auto J_, int ks) {
    constexpr int J = decltype(J_)::value;
    const bool live = ks < nkt;
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, MM>([&](auto M_) {
      constexpr int m = decltype(M_)::value;
      // 1: a real tile, 0: a dummy.  Hidden from the optimiser so the choice stays
      // arithmetic: a select of the address would become a branch around each
      // load, and the waits after a branch count conservatively.
      uint32_t on = (uint32_t)(live && m < Mw);
      asm volatile("" : "+v"(on));
      const uint32_t off = on * ((uint32_t)ks * tstride + (uint32_t)(bw0 + m) * 1024u + wvoff) + (1u - on) * tbytes;
      wr[J][m] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, kNonTemporal));
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  // the first K k-tiles go in flight now: the waits for H above are older
  static_for<0, K>([&](auto J_) { issue(J_, decltype(J_)::value); });

  // group codes through this wave's staging area: lane (i16, q) of block m
  // keeps bytes [4 WD q, 4 WD (q + 1)) of row 16 m + i16 (WD + 1 aligned
  // dwords, realigned).  One wave's LDS accesses complete in order.
  uint32_t cw[MM][WD];
  {
    unsigned char* stg = smem + L.h + (uint32_t)wave * L.stp;
#pragma unroll
    for (int c = 0; c < CL; ++c) *reinterpret_cast<u4*>(stg + 1024 * c + 16 * lane) = cst[c];
    asm volatile("" ::: "memory");
    static_for<0, MM>([&](auto M_) {
      constexpr int m = decltype(M_)::value;
      const uint32_t start = (uint32_t)(16 * m + i16) * (uint32_t)ng + 4u * WD * (uint32_t)q;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(stg + (start & ~3u));
      uint32_t w[WD + 1];
#pragma unroll
      for (int d = 0; d <= WD; ++d) w[d] = src[d];
#pragma unroll
      for (int d = 0; d < WD; ++d) cw[m][d] = __builtin_amdgcn_alignbyte(w[d + 1], w[d], start & 3u);
    });
  }

  lds_barrier();  // every maximum is in; every wave has read its group codes
  if (tid < N) sTok[4 * tid] = ldexpf(1.0f, -row_exponent(__uint_as_float(sTokU[4 * tid + 2])));
#pragma unroll
  for (int i = 0; i < kHChunks; ++i) {
    const int e = tid + i * kDecThreads;
    if (i * kDecThreads < hch && e < hch) {
      const int n = e / nch, c = e - n * nch;
      const int Sx = row_exponent(__uint_as_float(sTokU[4 * n + 2]));
      float v[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = bf16_to_f32((uint16_t)(hv[i][w] & 0xffffu));
        v[2 * w + 1] = bf16_to_f32((uint16_t)(hv[i][w] >> 16));
      }
      h8 out;
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] = (_Float16)ldexpf(v[k_order_h(j)], Sx);
      *reinterpret_cast<h8*>(sH + n * ldh + 8 * c) = out;
    }
  }
  lds_barrier();

  const _Float16* hrow = (i16 < N ? sH + i16 * ldh : sH0) + 8 * q;  // this lane's H operand row

  // ---- main loop: one k-tile per step, K steps per turn of the ring -------------
  f4 acc[MM], part[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) acc[m] = part[m] = f4{0.f, 0.f, 0.f, 0.f};
  const int cpt = G <= kKTile ? kKTile / G : 1;  // code bytes per k-tile (G = 256: one per two)
  for (int kt0 = 0; kt0 < nkt; kt0 += K) {
    static_for<0, K>([&](auto J_) {
      constexpr int J = decltype(J_)::value;
      const int kt = kt0 + J;
      __builtin_amdgcn_sched_barrier(0);
      if (kt < nkt) {  // uniform
        h8 hf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) hf[s] = *reinterpret_cast<const h8*>(hrow + 32 * (4 * kt + s));
        // the dword holding tile kt's codes: byte bb of the row, held by lane
        // 16 (dw / WD) + i16 as its dword dw % WD
        const int bb = G <= kKTile ? kt * cpt : kt >> 1;
        const int dw = bb >> 2, ld = dw % WD;
        const int src = 4 * (i16 + 16 * (dw / WD));
        const uint32_t bsh = 8u * (uint32_t)(bb & 3);
        uint32_t tc[MM];
        static_for<0, MM>([&](auto M_) {
          constexpr int m = decltype(M_)::value;
          uint32_t c = cw[m][0];
#pragma unroll
          for (int d = 1; d < WD; ++d) c = ld == d ? cw[m][d] : c;
          tc[m] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)c) >> bsh;
        });
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          static_for<0, MM>([&](auto M_) {
            constexpr int m = decltype(M_)::value;
            if (m < Mw) part[m] = mfma16(hf[s], unpack_q4(wr[J][m][s]), part[m]);
          });
          // a group of g columns ends after this step (G = 256: on odd k-tiles)
          const bool gend = G > kKTile ? (s == 3 && (kt & 1)) : ((32 * (s + 1)) % G) == 0;
          if (gend) {
            const uint32_t ci = G <= 32 ? (uint32_t)s : G == 64 ? (uint32_t)(s >> 1) : 0u;
            static_for<0, MM>([&](auto M_) {
              constexpr int m = decltype(M_)::value;
              if (m < Mw) {
                acc[m] += (float)((tc[m] >> (8u * ci)) & 0xffu) * part[m];
                part[m] = f4{0.f, 0.f, 0.f, 0.f};
              }
            });
          }
        }
      }
      // refill the slot with k-tile kt + K (past the end: dummies)
      issue(J_, kt + K);
      // The oldest wave of a SIMD wins its arbitration; left alone, the four
      // older waves of the workgroup finish long before the four younger ones
      // and the tail streams at half rate.  Alternate the halves' priority.
      if ((kt ^ (wave >> 2)) & 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    });
  }

  // ---- Z: the slices' partial sums, per-token exponent, hi/lo fragments ---------
  // by the four oldest waves, which win the arbitration and leave the loop
  // first: wave w takes tokens w, w + 4, ... (rows past N: zero fragments)
  const int csteps = a.rc32 / 32, esteps = (a.rc32 + a.rr32) / 32;
  if (wave < 4) {
    const int zs = z_slices(nkt);
    for (int n = wave; n < kDecodeMaxTokens; n += 4) {
      float m = 0.0f;
      if (n < N) {
        for (int k = lane; k < r; k += 64) {
          const float* zp = a.z32 + ((int64_t)n * r + k) * zst;
          float z = 0.0f;
          for (int c = 0; c < zs; ++c) z += zp[c];  // slice order
          sZt[n * r + k] = z;
          m = fmaxf(m, fabsf(z));
        }
      }
      m = wave_max(m);
      const int F = n < N ? row_exponent(m) : 0;
      if (lane == 0 && n < N) sTok[4 * n + 1] = ldexpf(1.0f, -F);
      // fragment of step s, lane 16 qq + n: ranks 32 sl + 8 qq + k_order_z(jj) of the step's part
      for (int e = lane; e < esteps * 4; e += 64) {
        const int s = e >> 2, qq = e & 3;
        const bool part_c = s < csteps;
        const int sl = part_c ? s : s - csteps;
        const int rank = part_c ? a.r_c : a.r_r, base = part_c ? 0 : a.r_c;
        h8 zh, zl;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int col = 32 * sl + 8 * qq + k_order_z(jj);
          const float z = (n < N && col < rank) ? ldexpf(sZt[n * r + base + col], F) : 0.0f;
          zh[jj] = (_Float16)z;
          zl[jj] = (_Float16)(z - (float)zh[jj]);
        }
        sZf[(2 * s) * 64 + 16 * qq + n] = zh;
        sZf[(2 * s + 1) * 64 + 16 * qq + n] = zl;
      }
    }
  }

  // ---- epilogue operands into the wave's area of LDS --------------------------------
  lds_barrier();  // every wave is done with H; Z's fragments are in
  unsigned char* est = smem + (uint32_t)wave * L.ste;
#pragma unroll
  for (int c = 0; c < kEpiLoads; ++c)
    if (c < nal) *reinterpret_cast<u4*>(est + 1024 * c + 16 * lane) = eac[c];
  *reinterpret_cast<u4*>(est + L.esc + 16 * lane) = esR;
  *reinterpret_cast<u4*>(est + L.esc + 1024 + 16 * lane) = esA;
  asm volatile("" ::: "memory");
  // eight A codes at byte offset o of the staged run (any alignment)
  auto a_codes = [&](uint32_t o) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(est + (o & ~3u));
    const uint32_t w0 = src[0], w1 = src[1], w2 = src[2];
    return u2{__builtin_amdgcn_alignbyte(w1, w0, o & 3u), __builtin_amdgcn_alignbyte(w2, w1, o & 3u)};
  };
  const uint16_t* eS = reinterpret_cast<const uint16_t*>(est + L.esc);

  // ---- epilogue per block: low-rank term, scales, store -------------------------
  // Y through a buffer resource with 32-bit offsets (row stride in elements)
  const uint32_t ystride = (uint32_t)a.Y_stride;
  const __amdgpu_buffer_rsrc_t yrs =
      buffer_rsrc(a.Y, (uint32_t)((uint64_t)(N - 1) * (uint64_t)a.Y_stride + (uint64_t)a.V) * (a.y_bf16 ? 2u : 4u));
  // Low-rank term of all the wave's blocks at once: no branch around a block,
  // so the LDS reads and MFMA chains of the blocks interleave (a slot with no
  // block reads staged bytes past the wave's rows and is never stored).
  f4 pcs[MM], pws[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) pcs[m] = pws[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int s = 0; s < esteps; ++s) {
    const bool part_c = s < csteps;  // uniform
    const int col = 32 * (part_c ? s : s - csteps) + 8 * q;
    const bool cv = col < (part_c ? a.r_c : a.r_r);
    const uint32_t cb = (uint32_t)((part_c ? 0 : a.r_c) + col);
    const h8 zh = sZf[(2 * s) * 64 + lane], zl = sZf[(2 * s + 1) * 64 + lane];
    h8 av[MM];
    static_for<0, MM>([&](auto M_) {
      constexpr int m = decltype(M_)::value;
      u2 raw = a_codes((uint32_t)(16 * m + i16) * (uint32_t)r + cb);
      if (!cv) raw = u2{0u, 0u};
      av[m] = unpack_i8x8(raw[0], raw[1]);
    });
    if (part_c) {
      static_for<0, MM>([&](auto M_) { constexpr int m = decltype(M_)::value; pcs[m] = mfma16(zh, av[m], pcs[m]); });
      static_for<0, MM>([&](auto M_) { constexpr int m = decltype(M_)::value; pcs[m] = mfma16(zl, av[m], pcs[m]); });
    } else {
      static_for<0, MM>([&](auto M_) { constexpr int m = decltype(M_)::value; pws[m] = mfma16(zh, av[m], pws[m]); });
      static_for<0, MM>([&](auto M_) { constexpr int m = decltype(M_)::value; pws[m] = mfma16(zl, av[m], pws[m]); });
    }
  }
  static_for<0, MM>([&](auto M_) {
    constexpr int m = decltype(M_)::value;
    const int row = 16 * m + i16;  // in the wave's staged runs
    const uint32_t v = (uint32_t)(bw0 + m) * 16u + (uint32_t)i16;
    if (m < Mw && (int64_t)v < a.V) {
      const float sR = f16_to_f32(eS[row]);
      const float sAc = a.r_c > 0 ? f16_to_f32(eS[512 + row * a.nA]) : 0.0f;
      const float sAw = a.r_r > 0 ? f16_to_f32(eS[512 + row * a.nA + a.nA - 1]) : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 4 * q + e;
        if (n >= N) continue;
        float y = sTok[4 * n] * (sR * acc[m][e]);
        if (r > 0) y = fmaf(sTok[4 * n + 1], fmaf(sAw, pws[m][e], sAc * pcs[m][e]), y);
        const uint32_t off = (uint32_t)n * ystride + v;  // the host keeps N rows of Y below 4 GiB
        if (a.y_bf16)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16(y), yrs, 2u * off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), yrs, 4u * off, 0, 0);
      }
    }
  });
}

int device_attr(hipDeviceAttribute_t at, int fallback) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, at, dev) != hipSuccess || n <= 0)
    return fallback;
  return n;
}

// dwords of group codes per lane and block: a quarter of D/g bytes, rounded up
int code_dwords(int ng) { return ng <= 16 ? 1 : ng <= 32 ? 2 : ng <= 64 ? 4 : 8; }
// most blocks per wave the registers hold, by WD (group codes) and r (the A
// codes held for the epilogue: 16 MM r <= kEpiLoads KB)
constexpr int max_blocks(int WD) { return WD >= 8 ? 4 : WD >= 2 ? 6 : 7; }
inline int max_blocks(int WD, int r) {
  const int cap = r > 0 ? kEpiLoads * 1024 / (16 * r) : max_blocks(WD);
  return std::max(1, std::min(max_blocks(WD), cap));
}

// LDS layout for N tokens of a head with MM blocks per wave (pure host arithmetic).
DecLds dec_layout(int64_t N, int64_t D, int r_c, int r_r, int MM, int WD, bool& ok) {
  const int rb32 = (int)(round_up((uint64_t)r_c, 32) + round_up((uint64_t)r_r, 32));
  const DecLds L = dec_lds((int)N, (int)D, r_c + r_r, rb32, MM, WD);
  ok = L.total <= kMaxLdsBytes;
  return L;
}

template <int MM, int WD>
hipError_t launch_mw(const FwdArgs& a, unsigned grid, int zst, hipStream_t s) {
  bool ok = false;
  const DecLds L = dec_layout(a.N, a.D, a.r_c, a.r_r, MM, WD, ok);
  if (!ok) return hipErrorInvalidValue;
  return launch_main(decode_kernel<MM, WD>, dim3(grid), dim3(kDecThreads), L.total, s, true, a, L, zst);
}

template <int WD>
hipError_t launch_w(const FwdArgs& a, int zst, hipStream_t s) {
  // one workgroup per CU (its registers allow no more), never more waves than
  // blocks; more workgroups only where a wave would get more blocks than its
  // registers hold
  constexpr int kMaxBlocks = max_blocks(WD);
  const int mmax = max_blocks(WD, a.r_c + a.r_r);
  const int64_t cus = device_attr(hipDeviceAttributeMultiprocessorCount, 256);
  int64_t grid = std::min<int64_t>(cus, (a.nb + kDecWaves - 1) / kDecWaves);
  while (wave_blocks_max((int)((a.nb + grid - 1) / grid)) > mmax) ++grid;
  const int mm = wave_blocks_max((int)((a.nb + grid - 1) / grid));
  const unsigned gu = (unsigned)grid;
  switch (mm) {  // blocks per wave, at most
    case 1: return launch_mw<1, WD>(a, gu, zst, s);
    case 2: return launch_mw<2, WD>(a, gu, zst, s);
    case 3: return launch_mw<3, WD>(a, gu, zst, s);
    case 4: return launch_mw<4, WD>(a, gu, zst, s);
    default: break;
  }
  if constexpr (kMaxBlocks >= 6) {
    switch (mm) {
      case 5: return launch_mw<5, WD>(a, gu, zst, s);
      case 6: return launch_mw<6, WD>(a, gu, zst, s);
      default: break;
    }
  }
  if constexpr (kMaxBlocks >= 7)
    if (mm == 7) return launch_mw<7, WD>(a, gu, zst, s);
  if constexpr (kMaxBlocks >= 8)
    if (mm == 8) return launch_mw<8, WD>(a, gu, zst, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_fits(const archead_dims* d, int64_t n_tokens) {
  if (n_tokens < 1 || n_tokens > kDecodeMaxTokens) return false;
  if (n_tokens * d->D / 8 > kHChunks * kDecThreads) return false;           // H chunks per thread
  if (d->g != 32 && d->g != 64 && d->g != 128 && d->g != 256) return false;
  if (d->D / d->g > 128) return false;                                // group codes a lane holds
  if (z_slices((int)(d->D / kKTile)) > kZMaxSlices) return false;     // Z partial sums per element
  if (round_up((uint64_t)d->r_c, 32) + round_up((uint64_t)d->r_r, 32) > (uint64_t)kDecMaxRank32) return false;
  // 32-bit offsets into every section, with room past the ends for the
  // dummy loads of unused slots
  const uint64_t V16 = round_up((uint64_t)d->V, 16), lim = (1ull << 32) - (1ull << 20);
  if (V16 * (uint64_t)d->D / 2 >= lim) return false;
  if (V16 * (uint64_t)(d->D / d->g) >= lim) return false;
  if (V16 * (uint64_t)(d->r_c + d->r_r) >= lim) return false;
  if ((uint64_t)(d->r_c + d->r_r) * (uint64_t)d->D >= lim) return false;
  // LDS with the most blocks per wave the launcher may choose
  const int WD = code_dwords((int)(d->D / d->g));
  bool ok = false;
  dec_layout(n_tokens, d->D, d->r_c, d->r_r, max_blocks(WD, d->r_c + d->r_r), WD, ok);
  return ok;
}

uint64_t decode_workspace_bytes(const archead_dims* d, int64_t n_tokens) {
  return (uint64_t)n_tokens * (uint64_t)(d->r_c + d->r_r) * (uint64_t)z_stride((int)(d->D / kKTile)) * 4u;
}

hipError_t launch_decode_prep(const FwdArgs& a, hipStream_t s) {
  const int r = a.r_c + a.r_r;
  if (r == 0) return hipSuccess;
  hipLaunchKernelGGL(dec_zpart_kernel, dim3((unsigned)z_slices(a.nkt), (unsigned)((r + 15) / 16)),
                     dim3(64 * kZWaves), 0, s, a, z_stride(a.nkt));
  return hipGetLastError();
}

hipError_t launch_decode(const FwdArgs& a, hipStream_t s) {
  const int zst = z_stride(a.nkt);
  switch (code_dwords(a.ng)) {
    case 1: return launch_w<1>(a, zst, s);
    case 2: return launch_w<2>(a, zst, s);
    case 4: return launch_w<4>(a, zst, s);
    default: return launch_w<8>(a, zst, s);
  }
}

}  // namespace archead
