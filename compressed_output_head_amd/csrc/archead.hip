// Host side of the C ABI: layout arithmetic, argument checks, packing and
// kernel dispatch.  See include/archead.h for the contract of every entry point.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "internal.h"

namespace archead {

int check_dims(const archead_dims* d) {
  if (!d) return ARCHEAD_E_NULL;
  if (d->V < 1 || d->D < kKTile || d->D % kKTile != 0) return ARCHEAD_E_DIMS;
  if (d->g < 2 || d->g % 2 != 0 || d->D % d->g != 0) return ARCHEAD_E_DIMS;
  if (d->r_c < 0 || d->r_r < 0) return ARCHEAD_E_DIMS;
  if (d->V > (int64_t(1) << 31) || d->D > (int64_t(1) << 20)) return ARCHEAD_E_UNSUPPORTED;
  if (d->r_c > (1 << 20) || d->r_r > (1 << 20)) return ARCHEAD_E_UNSUPPORTED;
  return ARCHEAD_OK;
}

int check_kernel_dims(const archead_dims* d) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (d->g != 32 && d->g != 64 && d->g != 128 && d->g != 256) return ARCHEAD_E_UNSUPPORTED;
  if (d->r_c % 8 || d->r_r % 8) return ARCHEAD_E_UNSUPPORTED;
  if (d->r_c > kMaxRank || d->r_r > kMaxRank) return ARCHEAD_E_UNSUPPORTED;
  return ARCHEAD_OK;
}

void compute_layout(const archead_dims* d, archead_layout* L) {
  const uint64_t V16 = round_up((uint64_t)d->V, 16);
  const uint64_t D = (uint64_t)d->D;
  const uint64_t r = (uint64_t)d->r_c + (uint64_t)d->r_r;
  const uint64_t ng = D / (uint64_t)d->g;
  const uint64_t nA = (d->r_c > 0) + (d->r_r > 0);
  memset(L, 0, sizeof(*L));
  L->format_version = ARCHEAD_FORMAT_VERSION;
  L->alignment = ARCHEAD_ALIGNMENT;
  L->header_bytes = 64;
  L->padded_rows = (int64_t)V16;
  L->header = {0, 64};
  uint64_t off = round_up(64, ARCHEAD_ALIGNMENT);
  archead_span* spans[7] = {&L->r_codes, &L->r_gcodes, &L->r_rowscale, &L->a_codes,
                            &L->a_scales, &L->b_codes, &L->b_scales};
  const uint64_t sizes[7] = {V16 * D / 2, V16 * ng, 2 * V16, V16 * r, 2 * V16 * nA, r * D, 2 * r * ng};
  uint64_t payload = 0;
  for (int i = 0; i < 7; ++i) {
    *spans[i] = {off, sizes[i]};
    payload += sizes[i];
    off = round_up(off + sizes[i], ARCHEAD_ALIGNMENT);
  }
  L->total_bytes = off;
  L->payload_bytes = payload;
}

WorkspaceLayout workspace_layout(const archead_dims* d, int64_t n_tokens, bool stats) {
  WorkspaceLayout w{};
  w.n16 = (int64_t)round_up((uint64_t)std::max<int64_t>(n_tokens, 0), 16);
  w.rc32 = (int)round_up((uint64_t)d->r_c, 32);
  w.rr32 = (int)round_up((uint64_t)d->r_r, 32);
  w.zsteps = (w.rc32 + w.rr32) / 32;
  w.n32 = (int64_t)round_up((uint64_t)std::max<int64_t>(n_tokens, 0), 32);
  const uint64_t n32 = (uint64_t)w.n32, D = (uint64_t)d->D;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = round_up(off + bytes, ARCHEAD_ALIGNMENT);
    return at;
  };
  w.hf = take(n32 * D * 2);
  w.hscale = take(n32 * 4);
  w.zf = take(n32 * (uint64_t)w.zsteps * 2 * 32 * 2);
  w.zscale = take(n32 * 4);
  const uint64_t nsmall = n_tokens <= kDecodeLdsTokens ? (uint64_t)std::max<int64_t>(n_tokens, 0) : 0;
  w.z32 = take(n32 * ((uint64_t)d->r_c + (uint64_t)d->r_r) * 4);
  w.hc = take(nsmall * D * 2);
  w.split_bytes = n_tokens > kDecodeLdsTokens ? kSplitBytes : 0;
  w.split = take(w.split_bytes);
  if (stats) {  // statistics pieces, and Y of a few-token call
    const uint64_t n = (uint64_t)std::max<int64_t>(n_tokens, 0);
    w.st_nparts = std::max<int64_t>(kStatChunks, (int64_t)(round_up((uint64_t)d->V, 16) + 255) / 256);
    w.st_part = take(n * (uint64_t)w.st_nparts * 16);
    w.st_y = take(n <= (uint64_t)kDecodeLdsTokens ? n * (uint64_t)d->V * 4 : 0);
  }
  w.total = n32 ? off : 0;
  return w;
}

namespace {

template <typename F>
void parallel_for(int64_t n, F f) {
  unsigned hw = std::thread::hardware_concurrency();
  int64_t nt = std::max<int64_t>(1, std::min<int64_t>({(int64_t)(hw ? hw : 1), 16, n}));
  if (nt <= 1 || n < 64) {
    f(0, n);
    return;
  }
  std::vector<std::thread> th;
  const int64_t chunk = (n + nt - 1) / nt;
  for (int64_t t = 0; t < nt; ++t) {
    const int64_t b = t * chunk, e = std::min(n, b + chunk);
    if (b < e) th.emplace_back([=] { f(b, e); });
  }
  for (auto& x : th) x.join();
}

}  // namespace
}  // namespace archead

using namespace archead;

extern "C" {

int archead_format_version(void) { return ARCHEAD_FORMAT_VERSION; }

const char* archead_status_string(int s) {
  switch (s) {
    case ARCHEAD_OK: return "ARCHEAD_OK";
    case ARCHEAD_E_NULL: return "ARCHEAD_E_NULL: a required pointer is NULL";
    case ARCHEAD_E_DIMS: return "ARCHEAD_E_DIMS: invalid head dimensions";
    case ARCHEAD_E_UNSUPPORTED: return "ARCHEAD_E_UNSUPPORTED: valid but unsupported configuration";
    case ARCHEAD_E_DTYPE: return "ARCHEAD_E_DTYPE: unsupported tensor dtype";
    case ARCHEAD_E_SHAPE: return "ARCHEAD_E_SHAPE: tensor shapes or strides do not match the head";
    case ARCHEAD_E_ALIGN: return "ARCHEAD_E_ALIGN: misaligned pointer or stride";
    case ARCHEAD_E_WORKSPACE: return "ARCHEAD_E_WORKSPACE: workspace too small";
    case ARCHEAD_E_HIP: return "ARCHEAD_E_HIP: kernel launch failed";
    case ARCHEAD_E_VALUE: return "ARCHEAD_E_VALUE: code out of range";
    case ARCHEAD_E_SIZE: return "ARCHEAD_E_SIZE: packed buffer too small";
    default: return "ARCHEAD: unknown status";
  }
}

int archead_pack_layout(const archead_dims* d, archead_layout* out) {
  if (!d || !out) return ARCHEAD_E_NULL;
  const int rc = check_dims(d);
  if (rc) return rc;
  compute_layout(d, out);
  return ARCHEAD_OK;
}

int archead_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes) {
  if (!d || !bytes) return ARCHEAD_E_NULL;
  const int rc = check_dims(d);
  if (rc) return rc;
  if (n_tokens < 0) return ARCHEAD_E_SHAPE;
  *bytes = workspace_layout(d, n_tokens).total;
  return ARCHEAD_OK;
}

int archead_pack(const archead_dims* d, const archead_host_components* src, void* dst,
                 uint64_t dst_bytes) {
  if (!d || !src || !dst) return ARCHEAD_E_NULL;
  int rc = check_dims(d);
  if (rc) return rc;
  if (!src->q4 || !src->c8 || !src->s_R) return ARCHEAD_E_NULL;
  if (d->r_c > 0 && (!src->A_c || !src->s_Ac || !src->B_c || !src->s_Bc)) return ARCHEAD_E_NULL;
  if (d->r_r > 0 && (!src->A_w || !src->s_Aw || !src->B_w || !src->s_Bw)) return ARCHEAD_E_NULL;
  archead_layout L;
  compute_layout(d, &L);
  if (dst_bytes < L.total_bytes) return ARCHEAD_E_SIZE;

  const int64_t V = d->V, D = d->D, g = d->g, ng = D / g, V16 = L.padded_rows;
  const int r_c = d->r_c, r_r = d->r_r, r = r_c + r_r;
  const int nA = (r_c > 0) + (r_r > 0);
  const int64_t nkt = D / kKTile, nb = V16 / 16;

  // range check of the INT4 codes first, so a failure writes nothing
  std::atomic<bool> bad{false};
  parallel_for(V, [&](int64_t b, int64_t e) {
    for (int64_t v = b; v < e && !bad.load(std::memory_order_relaxed); ++v) {
      const int8_t* row = src->q4 + v * D;
      for (int64_t k = 0; k < D; ++k)
        if (row[k] < -8 || row[k] > 7) {
          bad = true;
          break;
        }
    }
  });
  if (bad.load()) return ARCHEAD_E_VALUE;

  uint8_t* out = static_cast<uint8_t*>(dst);
  memset(out, 0, L.total_bytes);
  // header
  {
    uint32_t u32[2] = {ARCHEAD_MAGIC, ARCHEAD_FORMAT_VERSION};
    uint64_t u64[2] = {(uint64_t)V, (uint64_t)D};
    uint32_t u32b[4] = {(uint32_t)r_c, (uint32_t)r_r, (uint32_t)g, 0u};
    memcpy(out, u32, 8);
    memcpy(out + 8, u64, 16);
    memcpy(out + 24, u32b, 16);
  }
  // residual tiles, k-tile major: tile (b, kt) at (kt*nb + b)*1024; its byte
  // 16*l + 4*s + c holds row 16b + l%16, columns k = 128kt + 32s + 8(l/16) + 2c
  // (low nibble) and k + 1 (high nibble)
  uint8_t* rcodes = out + L.r_codes.offset;
  uint8_t* gcodes = out + L.r_gcodes.offset;
  parallel_for(nb, [&](int64_t b0, int64_t b1) {
    for (int64_t b = b0; b < b1; ++b) {
      for (int i = 0; i < 16; ++i) {
        const int64_t v = 16 * b + i;
        if (v >= V) break;
        const int8_t* row = src->q4 + v * D;
        for (int64_t kt = 0; kt < nkt; ++kt) {
          uint8_t* tile = rcodes + (kt * nb + b) * kTileBytes;
          for (int qq = 0; qq < 4; ++qq)
            for (int s = 0; s < 4; ++s)
              for (int c = 0; c < 4; ++c) {
                const int64_t k = kKTile * kt + 32 * s + 8 * qq + 2 * c;
                const uint8_t lo = (uint8_t)row[k] & 0xF, hi = (uint8_t)row[k + 1] & 0xF;
                tile[16 * (16 * qq + i) + 4 * s + c] = (uint8_t)(lo | (hi << 4));
              }
        }
        memcpy(gcodes + v * ng, src->c8 + v * ng, (size_t)ng);
      }
    }
  });
  memcpy(out + L.r_rowscale.offset, src->s_R, 2 * V);
  int8_t* acodes = reinterpret_cast<int8_t*>(out + L.a_codes.offset);
  uint16_t* ascales = reinterpret_cast<uint16_t*>(out + L.a_scales.offset);
  for (int64_t v = 0; v < V; ++v) {
    if (r_c) memcpy(acodes + v * r, src->A_c + v * r_c, r_c);
    if (r_r) memcpy(acodes + v * r + r_c, src->A_w + v * r_r, r_r);
    if (r_c) ascales[v * nA] = src->s_Ac[v];
    if (r_r) ascales[v * nA + nA - 1] = src->s_Aw[v];
  }
  int8_t* bcodes = reinterpret_cast<int8_t*>(out + L.b_codes.offset);
  uint16_t* bscales = reinterpret_cast<uint16_t*>(out + L.b_scales.offset);
  if (r_c) {
    memcpy(bcodes, src->B_c, (size_t)r_c * D);
    memcpy(bscales, src->s_Bc, (size_t)r_c * ng * 2);
  }
  if (r_r) {
    memcpy(bcodes + (int64_t)r_c * D, src->B_w, (size_t)r_r * D);
    memcpy(bscales + (int64_t)r_c * ng, src->s_Bw, (size_t)r_r * ng * 2);
  }
  return ARCHEAD_OK;
}

}  // extern "C"

namespace archead {
namespace {

// Checks shared by the entry points that run kernels, then every field of
// `a` except the output's.
int setup_args(const archead_tensor* H, const archead_packed_head* head, bool stats, FwdArgs& a,
               WorkspaceLayout& W) {
  if (!H || !head) return ARCHEAD_E_NULL;
  const archead_dims* d = &head->dims;
  int rc = check_kernel_dims(d);
  if (rc) return rc;
  if (H->dtype != ARCHEAD_BF16) return ARCHEAD_E_DTYPE;
  const int64_t N = H->rows;
  if (N < 0 || H->cols != d->D || H->row_stride < d->D) return ARCHEAD_E_SHAPE;
  if (N > (int64_t(1) << 22)) return ARCHEAD_E_UNSUPPORTED;
  if (N == 0) return ARCHEAD_OK;
  if (!H->data || !head->buffer || !head->workspace) return ARCHEAD_E_NULL;
  if ((uintptr_t)head->buffer % ARCHEAD_ALIGNMENT || (uintptr_t)head->workspace % ARCHEAD_ALIGNMENT)
    return ARCHEAD_E_ALIGN;
  if ((uintptr_t)H->data % 16 || (H->row_stride * 2) % 16) return ARCHEAD_E_ALIGN;
  archead_layout L;
  compute_layout(d, &L);
  if (head->buffer_bytes < L.total_bytes) return ARCHEAD_E_SIZE;
  W = workspace_layout(d, N, stats);
  if (head->workspace_bytes < W.total) return ARCHEAD_E_WORKSPACE;

  const uint8_t* buf = static_cast<const uint8_t*>(head->buffer);
  uint8_t* ws = static_cast<uint8_t*>(head->workspace);
  a = FwdArgs{};
  a.V = d->V;
  a.D = d->D;
  a.N = N;
  a.n16 = W.n16;
  a.n32 = W.n32;
  a.nb = L.padded_rows / 16;
  a.r_c = d->r_c;
  a.r_r = d->r_r;
  a.g = d->g;
  a.ng = (int)(d->D / d->g);
  a.nkt = (int)(d->D / kKTile);
  a.nks = (int)(d->D / 32);
  a.rc32 = W.rc32;
  a.rr32 = W.rr32;
  a.zsteps = W.zsteps;
  a.nA = (d->r_c > 0) + (d->r_r > 0);
  a.H = static_cast<const uint16_t*>(H->data);
  a.H_stride = H->row_stride;
  a.r_codes = buf + L.r_codes.offset;
  a.r_gcodes = buf + L.r_gcodes.offset;
  a.r_rowscale = reinterpret_cast<const uint16_t*>(buf + L.r_rowscale.offset);
  a.a_codes = reinterpret_cast<const int8_t*>(buf + L.a_codes.offset);
  a.a_scales = reinterpret_cast<const uint16_t*>(buf + L.a_scales.offset);
  a.b_codes = reinterpret_cast<const int8_t*>(buf + L.b_codes.offset);
  a.b_scales = reinterpret_cast<const uint16_t*>(buf + L.b_scales.offset);
  a.hf = reinterpret_cast<_Float16*>(ws + W.hf);
  a.hscale = reinterpret_cast<float*>(ws + W.hscale);
  a.zf = reinterpret_cast<_Float16*>(ws + W.zf);
  a.zscale = reinterpret_cast<float*>(ws + W.zscale);
  a.z32 = reinterpret_cast<float*>(ws + W.z32);
  a.hc = reinterpret_cast<_Float16*>(ws + W.hc);
  a.part = W.split_bytes ? reinterpret_cast<float*>(ws + W.split) : nullptr;
  a.part_bytes = W.split_bytes;
  if (stats) {
    a.st_part = reinterpret_cast<float*>(ws + W.st_part);
    a.st_nparts = W.st_nparts;
  }
  return ARCHEAD_OK;
}

}  // namespace
}  // namespace archead

extern "C" {

int archead_logits_events(const archead_tensor* H, const archead_packed_head* head,
                          archead_tensor* Y, int path, void* stream, void* ev_begin, void* ev_end) {
  if (!H || !head || !Y) return ARCHEAD_E_NULL;
  if (int rc0 = check_kernel_dims(&head->dims)) return rc0;
  if (path < ARCHEAD_PATH_AUTO || path > ARCHEAD_PATH_TILE) return ARCHEAD_E_UNSUPPORTED;
  if (H->dtype != ARCHEAD_BF16) return ARCHEAD_E_DTYPE;
  if (Y->dtype != ARCHEAD_F32 && Y->dtype != ARCHEAD_BF16) return ARCHEAD_E_DTYPE;
  const int64_t N = H->rows;
  if (Y->cols != head->dims.V || Y->rows != N || Y->row_stride < head->dims.V) return ARCHEAD_E_SHAPE;
  if (path == ARCHEAD_PATH_DECODE && N > kDecodeMaxTokens) return ARCHEAD_E_UNSUPPORTED;
  FwdArgs a;
  WorkspaceLayout W;
  int rc = setup_args(H, head, false, a, W);
  if (rc || N == 0) return rc;
  const int ysz = Y->dtype == ARCHEAD_F32 ? 4 : 2;
  if (!Y->data) return ARCHEAD_E_NULL;
  if ((uintptr_t)Y->data % ysz) return ARCHEAD_E_ALIGN;
  a.Y = Y->data;
  a.Y_stride = Y->row_stride;
  a.y_bf16 = Y->dtype == ARCHEAD_BF16;

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // start from a clean error state
  // auto: the LDS decode kernel for a few tokens, else the tile path.
  // decode path: the LDS kernel when it applies, else the batched kernel (the
  // 16-row decode kernel only when offsets exceed 32 bits); tile path: the
  // 32-row kernel unless offsets exceed 32 bits (launch_tile decides the same way)
  const bool small = (path == ARCHEAD_PATH_DECODE || (path == ARCHEAD_PATH_AUTO && N <= kDecodeMaxTokens)) &&
                     decode_lds_eligible(a);
  const bool decode = path == ARCHEAD_PATH_DECODE || small;
  const bool mid = decode && !small && mid_eligible(a);
  const bool rows32 = mid || (!decode && tile32_eligible(a));
  if ((small ? launch_prep_z(a, s) : launch_prep(a, rows32, s)) != hipSuccess) return ARCHEAD_E_HIP;
  if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), s) != hipSuccess) return ARCHEAD_E_HIP;
  const hipError_t e = small ? launch_decode_lds(a, s)
                       : mid ? launch_mid(a, s)
                       : decode ? launch_decode(a, s)
                                : launch_tile(a, s);
  if (e != hipSuccess) return ARCHEAD_E_HIP;
  if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), s) != hipSuccess) return ARCHEAD_E_HIP;
  return ARCHEAD_OK;
}

int archead_logits_path(const archead_tensor* H, const archead_packed_head* head,
                        archead_tensor* Y, int path, void* stream) {
  return archead_logits_events(H, head, Y, path, stream, nullptr, nullptr);
}

int archead_logits(const archead_tensor* H, const archead_packed_head* head, archead_tensor* Y,
                   void* stream) {
  return archead_logits_path(H, head, Y, ARCHEAD_PATH_AUTO, stream);
}

int archead_stats_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes) {
  if (!d || !bytes) return ARCHEAD_E_NULL;
  const int rc = check_dims(d);
  if (rc) return rc;
  if (n_tokens < 0) return ARCHEAD_E_SHAPE;
  *bytes = workspace_layout(d, n_tokens, true).total;
  return ARCHEAD_OK;
}

int archead_logits_stats(const archead_tensor* H, const archead_packed_head* head, const archead_row_stats* out,
                         void* stream) {
  if (!H || !head || !out) return ARCHEAD_E_NULL;
  if (out->row_ce && !out->targets) return ARCHEAD_E_NULL;
  for (const void* p : {(const void*)out->row_max, (const void*)out->row_argmax, (const void*)out->row_lse,
                        (const void*)out->row_ce, (const void*)out->targets})
    if ((uintptr_t)p % 4) return ARCHEAD_E_ALIGN;
  FwdArgs a;
  WorkspaceLayout W;
  int rc = setup_args(H, head, true, a, W);
  if (rc || H->rows == 0) return rc;
  a.targets = out->targets;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // start from a clean error state
  hipError_t e;
  if (decode_lds_eligible(a)) {
    // a few tokens: Y (at most 16 rows) into the workspace, then its pieces
    float* Yw = reinterpret_cast<float*>(static_cast<uint8_t*>(head->workspace) + W.st_y);
    a.Y = Yw;
    a.Y_stride = a.V;
    a.y_bf16 = 0;
    a.st_nparts = kStatChunks;
    e = launch_prep_z(a, s);
    if (e == hipSuccess) e = launch_decode_lds(a, s);
    if (e == hipSuccess) e = launch_rowstats_y(a, Yw, a.V, s);
  } else if (tile32_eligible(a)) {
    a.st_nparts = tile_stat_parts(a);
    e = launch_prep(a, true, s);
    if (e == hipSuccess) e = launch_tile_stats(a, s);
  } else {
    return ARCHEAD_E_UNSUPPORTED;
  }
  if (e == hipSuccess) e = launch_stats_reduce(a, out->row_max, out->row_argmax, out->row_lse, out->row_ce, s);
  return e == hipSuccess ? ARCHEAD_OK : ARCHEAD_E_HIP;
}

}  // extern "C"
