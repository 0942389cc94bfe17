// Host side of the C ABI: layout arithmetic, argument checks, packing and
// kernel dispatch.  See include/archead.h for the contract of every entry point.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <thread>
#include <vector>

#include "internal.h"

namespace archead {

int check_dims(const archead_dims* d) {
  if (!d) return ARCHEAD_E_NULL;
  if (d->V < 1 || d->D < kKTile || d->D % kKTile != 0) return ARCHEAD_E_DIMS;
  if (d->g < 2 || d->g % 2 != 0 || d->D % d->g != 0) return ARCHEAD_E_DIMS;
  if (d->r_c < 0 || d->r_r < 0) return ARCHEAD_E_DIMS;
  if (d->format < ARCHEAD_FMT_ARCHEAD || d->format > ARCHEAD_FMT_ROW_INT8) return ARCHEAD_E_DIMS;
  if (d->format != ARCHEAD_FMT_ARCHEAD && (d->r_c != 0 || d->r_r != 0)) return ARCHEAD_E_DIMS;
  if (d->V > (int64_t(1) << 31) || d->D > (int64_t(1) << 20)) return ARCHEAD_E_UNSUPPORTED;
  if (d->r_c > (1 << 20) || d->r_r > (1 << 20)) return ARCHEAD_E_UNSUPPORTED;
  return ARCHEAD_OK;
}

int check_archead_format(const archead_dims* d) {
  if (!d) return ARCHEAD_E_NULL;
  return d->format == ARCHEAD_FMT_ARCHEAD ? ARCHEAD_OK : ARCHEAD_E_UNSUPPORTED;
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
  uint64_t sizes[7] = {V16 * D / 2, V16 * ng, 2 * V16, V16 * r, 2 * V16 * nA, r * D, 2 * r * ng};
  if (d->format == ARCHEAD_FMT_GROUP_INT4) {  // INT4 tiles and fp16 group scales
    const uint64_t s1[7] = {V16 * D / 2, 2 * V16 * ng, 0, 0, 0, 0, 0};
    memcpy(sizes, s1, sizeof(sizes));
  } else if (d->format == ARCHEAD_FMT_ROW_INT8) {  // INT8 tiles and fp16 row scales
    const uint64_t s2[7] = {V16 * D, 0, 2 * V16, 0, 0, 0, 0};
    memcpy(sizes, s2, sizeof(sizes));
  }
  uint64_t payload = 0;
  for (int i = 0; i < 7; ++i) {
    *spans[i] = {off, sizes[i]};
    payload += sizes[i];
    off = round_up(off + sizes[i], ARCHEAD_ALIGNMENT);
  }
  L->total_bytes = off;
  L->payload_bytes = payload;
}

// Events of the archead_logits_events call running on this thread (none
// outside such a call).
MainEvents& main_events() {
  static thread_local MainEvents e;
  return e;
}

WorkspaceLayout workspace_layout(const archead_dims* d, int64_t n_tokens, bool stats, uint64_t split_cap,
                                 bool allow_decode) {
  WorkspaceLayout w{};
  const uint64_t n = (uint64_t)std::max<int64_t>(n_tokens, 0);
  // a comparison head runs the batched kernel only, up to kAltChunk tokens a launch
  const bool alt = d->format != ARCHEAD_FMT_ARCHEAD;
  const int64_t chunk = alt ? std::min<int64_t>(n_tokens, kAltChunk) : n_tokens;
  w.small = !alt && allow_decode && small_decode_fits(d, n_tokens);
  w.batch = allow_decode && !w.small && batch_fits(d, alt ? std::max<int64_t>(chunk, 1) : chunk);
  w.decode = w.small || w.batch || (!alt && allow_decode && decode_fits(d, n_tokens));
  w.rc32 = (int)round_up((uint64_t)d->r_c, 32);
  w.rr32 = (int)round_up((uint64_t)d->r_r, 32);
  w.zsteps = (w.rc32 + w.rr32) / 32;
  w.n32 = (int64_t)round_up(n, 32);
  const uint64_t n32 = (uint64_t)w.n32, D = (uint64_t)d->D;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = round_up(off + bytes, ARCHEAD_ALIGNMENT);
    return at;
  };
  if (!w.decode) {
    w.hf = take(n32 * D * 2);
    w.hscale = take(n32 * 4);
    w.zf = take(n32 * (uint64_t)w.zsteps * 2 * 32 * 2);
    w.zscale = take(n32 * 4);
    const int r = d->r_c + d->r_r;
    const uint64_t zp = r > 0 ? (uint64_t)zmm_parts((int64_t)n32, r, d->D, d->g) : 1;
    w.z32 = take(zp * n32 * (uint64_t)r * 4);  // parts of the k range, added by zsplit_kernel
  } else if (w.small || w.batch) {  // few-token and batched decode kernels: converted H, its scales, Z
    const uint64_t nc = (uint64_t)std::max<int64_t>(chunk, 0);  // rows converted per launch
    w.zsl = w.small ? small_z_slices(d->D, n_tokens) : 1;       // Z as partial sums over slices of D
    w.hc = take(nc * D * 2);
    w.hscale = take(nc * 4);
    w.z32 = take((uint64_t)w.zsl * nc * ((uint64_t)d->r_c + (uint64_t)d->r_r) * 4);
  } else {  // the decode path: partial sums of Z
    w.z32 = take(decode_workspace_bytes(d, n_tokens));
  }
  if (stats) {  // statistics pieces, and Y of a call the decode kernel takes
    w.st_nparts = std::max<int64_t>(kStatChunks, (int64_t)(round_up((uint64_t)d->V, 16) + 255) / 256);
    w.st_part = take(n * (uint64_t)w.st_nparts * 16);
    w.st_y = take(w.decode ? n * (uint64_t)d->V * 4 : 0);
  }
  // the partial sums of split tiles come last, so a caller with a fixed
  // budget can give them what is left
  w.split_bytes = w.decode ? 0 : std::min<uint64_t>(split_cap, kSplitBytes) / ARCHEAD_ALIGNMENT * ARCHEAD_ALIGNMENT;
  w.split = take(w.split_bytes);
  w.total = n ? off : 0;
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

int archead_workspace_bytes_path(const archead_dims* d, int64_t n_tokens, int path, uint64_t* bytes) {
  if (!d || !bytes) return ARCHEAD_E_NULL;
  const int rc = check_dims(d);
  if (rc) return rc;
  if (n_tokens < 0) return ARCHEAD_E_SHAPE;
  if (path < ARCHEAD_PATH_AUTO || path > ARCHEAD_PATH_TILE) return ARCHEAD_E_UNSUPPORTED;
  if (d->format != ARCHEAD_FMT_ARCHEAD && path == ARCHEAD_PATH_TILE) return ARCHEAD_E_UNSUPPORTED;
  *bytes = workspace_layout(d, n_tokens, false, kSplitBytes, path != ARCHEAD_PATH_TILE).total;
  return ARCHEAD_OK;
}

int archead_main_kernel(const archead_dims* d, int64_t n_tokens, int path, int* kernel) {
  if (!d || !kernel) return ARCHEAD_E_NULL;
  const int rc = check_dims(d);
  if (rc) return rc;
  if (n_tokens < 0) return ARCHEAD_E_SHAPE;
  if (path < ARCHEAD_PATH_AUTO || path > ARCHEAD_PATH_TILE) return ARCHEAD_E_UNSUPPORTED;
  const WorkspaceLayout w = workspace_layout(d, n_tokens, false, kSplitBytes, path != ARCHEAD_PATH_TILE);
  if (path == ARCHEAD_PATH_DECODE && !w.decode) return ARCHEAD_E_UNSUPPORTED;
  if (d->format != ARCHEAD_FMT_ARCHEAD && !w.batch) return ARCHEAD_E_UNSUPPORTED;  // batched kernel only
  *kernel = !w.decode ? ARCHEAD_KERNEL_TILE
            : w.small ? ARCHEAD_KERNEL_DECODE_FEW
            : w.batch ? ARCHEAD_KERNEL_DECODE_BATCH
                      : ARCHEAD_KERNEL_DECODE_STREAM;
  return ARCHEAD_OK;
}

int archead_workspace_bytes(const archead_dims* d, int64_t n_tokens, uint64_t* bytes) {
  return archead_workspace_bytes_path(d, n_tokens, ARCHEAD_PATH_AUTO, bytes);
}

int archead_pack(const archead_dims* d, const archead_host_components* src, void* dst,
                 uint64_t dst_bytes) {
  if (!d || !src || !dst) return ARCHEAD_E_NULL;
  int rc = check_dims(d);
  if (rc) return rc;
  const int fmt = d->format;
  if (fmt == ARCHEAD_FMT_ARCHEAD) {
    if (!src->q4 || !src->c8 || !src->s_R) return ARCHEAD_E_NULL;
    if (d->r_c > 0 && (!src->A_c || !src->s_Ac || !src->B_c || !src->s_Bc)) return ARCHEAD_E_NULL;
    if (d->r_r > 0 && (!src->A_w || !src->s_Aw || !src->B_w || !src->s_Bw)) return ARCHEAD_E_NULL;
  } else if (fmt == ARCHEAD_FMT_GROUP_INT4) {
    if (!src->q4 || !src->s_G) return ARCHEAD_E_NULL;
  } else if (!src->q8 || !src->s_R) {
    return ARCHEAD_E_NULL;
  }
  archead_layout L;
  compute_layout(d, &L);
  if (dst_bytes < L.total_bytes) return ARCHEAD_E_SIZE;

  const int64_t V = d->V, D = d->D, g = d->g, ng = D / g, V16 = L.padded_rows;
  const int r_c = d->r_c, r_r = d->r_r, r = r_c + r_r;
  const int nA = (r_c > 0) + (r_r > 0);
  const int64_t nkt = D / kKTile, nb = V16 / 16;

  // range check of the codes first, so a failure writes nothing
  std::atomic<bool> bad{false};
  parallel_for(V, [&](int64_t b, int64_t e) {
    for (int64_t v = b; v < e && !bad.load(std::memory_order_relaxed); ++v) {
      if (fmt == ARCHEAD_FMT_ROW_INT8) {
        const int8_t* row = src->q8 + v * D;
        for (int64_t k = 0; k < D; ++k)
          if (row[k] == -128) {
            bad = true;
            break;
          }
      } else {
        const int8_t* row = src->q4 + v * D;
        for (int64_t k = 0; k < D; ++k)
          if (row[k] < -8 || row[k] > 7) {
            bad = true;
            break;
          }
      }
    }
  });
  if (bad.load()) return ARCHEAD_E_VALUE;

  uint8_t* out = static_cast<uint8_t*>(dst);
  memset(out, 0, L.total_bytes);
  // header; the flags word holds the format
  {
    uint32_t u32[2] = {ARCHEAD_MAGIC, ARCHEAD_FORMAT_VERSION};
    uint64_t u64[2] = {(uint64_t)V, (uint64_t)D};
    uint32_t u32b[4] = {(uint32_t)r_c, (uint32_t)r_r, (uint32_t)g, (uint32_t)fmt};
    memcpy(out, u32, 8);
    memcpy(out + 8, u64, 16);
    memcpy(out + 24, u32b, 16);
  }
  uint8_t* rcodes = out + L.r_codes.offset;
  if (fmt == ARCHEAD_FMT_ROW_INT8) {
    // INT8 tiles, k-tile major: tile (b, kt) at (kt*nb + b)*2048; its byte
    // 32*l + 8*s + p holds row 16b + l%16, column 128kt + 32s + 8(l/16) + P[p]
    // with P = (0,1,4,5,2,3,6,7): the fp16 operand slot order of the kernels
    static const int kPerm8[8] = {0, 1, 4, 5, 2, 3, 6, 7};
    parallel_for(nb, [&](int64_t b0, int64_t b1) {
      for (int64_t b = b0; b < b1; ++b)
        for (int i = 0; i < 16; ++i) {
          const int64_t v = 16 * b + i;
          if (v >= V) break;
          const int8_t* row = src->q8 + v * D;
          for (int64_t kt = 0; kt < nkt; ++kt) {
            uint8_t* tile = rcodes + (kt * nb + b) * 2 * kTileBytes;
            for (int qq = 0; qq < 4; ++qq)
              for (int st = 0; st < 4; ++st)
                for (int pp = 0; pp < 8; ++pp)
                  tile[32 * (16 * qq + i) + 8 * st + pp] = (uint8_t)row[kKTile * kt + 32 * st + 8 * qq + kPerm8[pp]];
          }
        }
    });
    memcpy(out + L.r_rowscale.offset, src->s_R, 2 * V);
    return ARCHEAD_OK;
  }
  // INT4 tiles, k-tile major: tile (b, kt) at (kt*nb + b)*1024; its byte
  // 16*l + 4*s + c holds row 16b + l%16, columns k = 128kt + 32s + 8(l/16) + 2c
  // (low nibble) and k + 1 (high nibble)
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
        if (fmt == ARCHEAD_FMT_GROUP_INT4)  // fp16 group scales, row-major
          memcpy(gcodes + 2 * v * ng, src->s_G + v * ng, (size_t)(2 * ng));
        else
          memcpy(gcodes + v * ng, src->c8 + v * ng, (size_t)ng);
      }
    }
  });
  if (fmt == ARCHEAD_FMT_GROUP_INT4) return ARCHEAD_OK;
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

// The workspace of archead_logits_noalloc: one array per GPU (each device
// holds its own copy of this code object's data), kept until the process
// ends.  Host code reaches it only through the address hipGetSymbolAddress
// returns for the current device: on the host the array's name is not a
// device address.
namespace archead {
constexpr uint64_t kNoAllocScratchBytes = ARCHEAD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
}  // namespace archead

namespace archead {
namespace {

// Checks shared by the entry points that run kernels, then every field of
// `a` except the output's.
int setup_args(const archead_tensor* H, const archead_packed_head* head, bool stats, FwdArgs& a,
               WorkspaceLayout& W, bool allow_decode = true, uint64_t split_cap = kSplitBytes) {
  if (!H || !head) return ARCHEAD_E_NULL;
  const archead_dims* d = &head->dims;
  int rc = check_kernel_dims(d);
  if (rc) return rc;
  if (H->dtype != ARCHEAD_BF16) return ARCHEAD_E_DTYPE;
  const int64_t N = H->rows;
  if (N < 0 || H->cols != d->D || H->row_stride < d->D) return ARCHEAD_E_SHAPE;
  if (N > (int64_t(1) << 22)) return ARCHEAD_E_UNSUPPORTED;
  if (N == 0) return ARCHEAD_OK;
  if (!H->data || !head->buffer) return ARCHEAD_E_NULL;
  if ((uintptr_t)head->buffer % ARCHEAD_ALIGNMENT || (uintptr_t)head->workspace % ARCHEAD_ALIGNMENT)
    return ARCHEAD_E_ALIGN;
  if ((uintptr_t)H->data % 16 || (H->row_stride * 2) % 16) return ARCHEAD_E_ALIGN;
  archead_layout L;
  compute_layout(d, &L);
  if (head->buffer_bytes < L.total_bytes) return ARCHEAD_E_SIZE;
  W = workspace_layout(d, N, stats, split_cap, allow_decode);
  if (W.total > 0 && !head->workspace) return ARCHEAD_E_NULL;
  if (head->workspace_bytes < W.total) return ARCHEAD_E_WORKSPACE;

  const uint8_t* buf = static_cast<const uint8_t*>(head->buffer);
  uint8_t* ws = static_cast<uint8_t*>(head->workspace);
  a = FwdArgs{};
  a.V = d->V;
  a.D = d->D;
  a.N = N;
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
  a.zsl = W.zsl > 0 ? W.zsl : 1;
  a.nA = (d->r_c > 0) + (d->r_r > 0);
  a.fmt = d->format;
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

// Y = H W_hat^T on the path `path`, with the split-tile partial sums capped
// at split_cap bytes of the workspace.
// Sets the pending kernel events for one call and clears them at its end
// (whatever path the call takes), so no later launch records them.
struct EventScope {
  explicit EventScope(void* start, void* stop) {
    main_events().start = static_cast<hipEvent_t>(start);
    main_events().stop = static_cast<hipEvent_t>(stop);
  }
  ~EventScope() { main_events() = MainEvents{}; }
};

int logits_impl(const archead_tensor* H, const archead_packed_head* head, archead_tensor* Y, int path,
                void* stream, void* ev_begin, void* ev_end, uint64_t split_cap) {
  if (!H || !head || !Y) return ARCHEAD_E_NULL;
  if (int rc0 = check_kernel_dims(&head->dims)) return rc0;
  if (path < ARCHEAD_PATH_AUTO || path > ARCHEAD_PATH_TILE) return ARCHEAD_E_UNSUPPORTED;
  if (head->dims.format != ARCHEAD_FMT_ARCHEAD && path == ARCHEAD_PATH_TILE) return ARCHEAD_E_UNSUPPORTED;
  if (H->dtype != ARCHEAD_BF16) return ARCHEAD_E_DTYPE;
  if (Y->dtype != ARCHEAD_F32 && Y->dtype != ARCHEAD_BF16) return ARCHEAD_E_DTYPE;
  const int64_t N = H->rows;
  if (Y->cols != head->dims.V || Y->rows != N || Y->row_stride < head->dims.V) return ARCHEAD_E_SHAPE;
  FwdArgs a;
  WorkspaceLayout W;
  int rc = setup_args(H, head, false, a, W, path != ARCHEAD_PATH_TILE, split_cap);
  if (rc || N == 0) return rc;
  const int ysz = Y->dtype == ARCHEAD_F32 ? 4 : 2;
  if (!Y->data) return ARCHEAD_E_NULL;
  if ((uintptr_t)Y->data % ysz) return ARCHEAD_E_ALIGN;
  a.Y = Y->data;
  a.Y_stride = Y->row_stride;
  a.y_bf16 = Y->dtype == ARCHEAD_BF16;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head->dims.format != ARCHEAD_FMT_ARCHEAD) {
    // a comparison head: the batched kernel, kAltChunk tokens a launch, each
    // launch after the conversion of its own rows (the workspace holds one chunk)
    if (!W.batch) return ARCHEAD_E_UNSUPPORTED;
    const int64_t chunk = std::min<int64_t>(N, kAltChunk);
    if ((uint64_t)(chunk - 1) * (uint64_t)Y->row_stride * ysz + (uint64_t)head->dims.V * ysz >= (1ull << 32))
      return ARCHEAD_E_UNSUPPORTED;
    (void)hipGetLastError();  // start from a clean error state
    // the first batched launch records ev_begin at its start, the last one ev_end at its end
    EventScope evs(ev_begin, nullptr);
    for (int64_t c0 = 0; c0 < N; c0 += kAltChunk) {
      FwdArgs ac = a;
      ac.N = std::min<int64_t>(kAltChunk, N - c0);
      ac.H = a.H + c0 * a.H_stride;
      ac.Y = static_cast<uint8_t*>(Y->data) + (uint64_t)c0 * (uint64_t)Y->row_stride * ysz;
      if (launch_small_prep(ac, s) != hipSuccess) return ARCHEAD_E_HIP;
      if (c0 + kAltChunk >= N) main_events().stop = static_cast<hipEvent_t>(ev_end);
      if (launch_batch(ac, s) != hipSuccess) return ARCHEAD_E_HIP;
    }
    return ARCHEAD_OK;
  }
  // auto: the decode kernel when it takes the call, else the tile path; the
  // caller may force either (a forced decode path it does not take is an error)
  const bool decode = W.decode;
  if (path == ARCHEAD_PATH_DECODE && !decode) return ARCHEAD_E_UNSUPPORTED;
  // the decode kernel stores Y through 32-bit offsets
  if (decode && (uint64_t)(N - 1) * (uint64_t)Y->row_stride * ysz + (uint64_t)head->dims.V * ysz >= (1ull << 32))
    return ARCHEAD_E_UNSUPPORTED;
  if (!decode && !tile32_eligible(a)) return ARCHEAD_E_UNSUPPORTED;
  (void)hipGetLastError();  // start from a clean error state
  const hipError_t ep = !decode ? launch_prep(a, s) : (W.small || W.batch) ? launch_small_prep(a, s) : launch_decode_prep(a, s);
  if (ep != hipSuccess) return ARCHEAD_E_HIP;
  // the main kernel's launch records ev_begin at its start and ev_end at the
  // end of the forward's last kernel
  EventScope evs(ev_begin, ev_end);
  const hipError_t e = !decode ? launch_tile(a, s)
                       : W.small ? launch_small_decode(a, s)
                       : W.batch ? launch_batch(a, s)
                                 : launch_decode(a, s);
  if (e != hipSuccess) return ARCHEAD_E_HIP;
  return ARCHEAD_OK;
}

constexpr int kMaxDevices = 64;
// ---- allocation-free variant: the scratch address of each device ---------------
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch (looked up once per device).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ARCHEAD_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ARCHEAD_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ARCHEAD_OK;
}

}  // namespace
}  // namespace archead

extern "C" {

int archead_logits_events(const archead_tensor* H, const archead_packed_head* head,
                          archead_tensor* Y, int path, void* stream, void* ev_begin, void* ev_end) {
  return logits_impl(H, head, Y, path, stream, ev_begin, ev_end, kSplitBytes);
}

int archead_logits_noalloc(const archead_tensor* H, const archead_packed_head* head, archead_tensor* Y,
                           void* stream) {
  if (!H || !head || !Y) return ARCHEAD_E_NULL;
  if (int rc = check_kernel_dims(&head->dims)) return rc;
  if (int rc = check_archead_format(&head->dims)) return rc;
  if (H->rows < 0) return ARCHEAD_E_SHAPE;
  if (H->rows == 0) return ARCHEAD_OK;
  // the call's workspace without split-tile partial sums must fit; whatever
  // is left goes to them (the tile kernel splits no tile it has no room for)
  const uint64_t need = workspace_layout(&head->dims, H->rows, false, 0, true).total;
  if (need > kNoAllocScratchBytes) return ARCHEAD_E_WORKSPACE;
  void* ws = nullptr;
  if (int rc = scratch_address(&ws)) return rc;
  archead_packed_head h = *head;
  h.workspace = ws;
  h.workspace_bytes = kNoAllocScratchBytes;
  return logits_impl(H, &h, Y, ARCHEAD_PATH_AUTO, stream, nullptr, nullptr, kNoAllocScratchBytes - need);
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
  int rc = check_dims(d);
  if (rc) return rc;
  if ((rc = check_archead_format(d))) return rc;
  if (n_tokens < 0) return ARCHEAD_E_SHAPE;
  *bytes = workspace_layout(d, n_tokens, true).total;
  return ARCHEAD_OK;
}

int archead_logits_stats(const archead_tensor* H, const archead_packed_head* head, const archead_row_stats* out,
                         void* stream) {
  if (!H || !head || !out) return ARCHEAD_E_NULL;
  if (int rc0 = check_archead_format(&head->dims)) return rc0;
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
  if (W.decode) {
    // a few tokens: Y (at most 16 rows) into the workspace, then its pieces
    float* Yw = reinterpret_cast<float*>(static_cast<uint8_t*>(head->workspace) + W.st_y);
    a.Y = Yw;
    a.Y_stride = a.V;
    a.y_bf16 = 0;
    a.st_nparts = kStatChunks;
    e = (W.small || W.batch) ? launch_small_prep(a, s) : launch_decode_prep(a, s);
    if (e == hipSuccess) e = W.small ? launch_small_decode(a, s) : W.batch ? launch_batch(a, s) : launch_decode(a, s);
    if (e == hipSuccess) e = launch_rowstats_y(a, Yw, a.V, s);
  } else if (tile32_eligible(a)) {
    a.st_nparts = tile_stat_parts(a);
    e = launch_prep(a, s);
    if (e == hipSuccess) e = launch_tile_stats(a, s);
  } else {
    return ARCHEAD_E_UNSUPPORTED;
  }
  if (e == hipSuccess) e = launch_stats_reduce(a, out->row_max, out->row_argmax, out->row_lse, out->row_ce, s);
  return e == hipSuccess ? ARCHEAD_OK : ARCHEAD_E_HIP;
}

}  // extern "C"
