// Batched streaming kernel, ARCHead-format instances and the host side:
// which calls it takes (batch_fits) and the dispatch over formats and token
// tiles.  The kernel itself is in batch_kernel.h; the comparison heads'
// instances are compiled in batch_g4.hip and batch_r8.hip.
#include "batch_kernel.h"

namespace archead {

bool batch_fits(const archead_dims* d, int64_t n_tokens) {
  const bool alt = d->format != ARCHEAD_FMT_ARCHEAD;
  // ARCHead: 17 to 64 tokens (fewer go to the few-token kernel); a
  // comparison head: every call, up to kAltChunk tokens a launch
  if (alt ? (n_tokens < 1 || n_tokens > kAltChunk) : (n_tokens <= kDecodeMaxTokens || n_tokens > 16 * kBMaxTiles))
    return false;
  if ((d->D / kKTile) % 4 != 0) return false;  // whole turns of the unrolled loop (2 HK | k-tiles)
  if (d->g != 32 && d->g != 64 && d->g != 128 && d->g != 256) return false;
  if (d->format != ARCHEAD_FMT_ROW_INT8 && d->D / d->g > kBMaxGroups) return false;
  if (round_up((uint64_t)d->r_c, 32) + round_up((uint64_t)d->r_r, 32) > 32u * kBMaxSteps) return false;
  // 32-bit offsets into every section and into the converted rows
  const uint64_t V16 = round_up((uint64_t)d->V, 16), lim = (1ull << 32) - (1ull << 20);
  if (V16 * (uint64_t)d->D / (d->format == ARCHEAD_FMT_ROW_INT8 ? 1 : 2) >= lim) return false;
  if (V16 * (uint64_t)(d->D / d->g) * 2 >= lim) return false;
  if (V16 * (uint64_t)(d->r_c + d->r_r) >= lim) return false;
  if ((uint64_t)n_tokens * (uint64_t)d->D * 2 >= lim) return false;
  const int T = (int)((n_tokens + 15) / 16);
  const int occ = batch_occupancy(T);
  const int64_t nb = (int64_t)(V16 / 16), grid = batch_grid(nb, occ);
  if (batch_blocks_per_wave(nb, grid) > (occ > 1 ? kBMaxBlocks2 : kBMaxBlocks)) return false;
  return (uint64_t)occ * (batch_layout(d, n_tokens, nb, grid).total +
                         batch_ring_lds(T, batch_hk(T, (int)(d->D / kKTile)))) <= kMaxLdsBytes;
}

hipError_t launch_batch(const FwdArgs& a, hipStream_t s) {
  switch (a.fmt) {
    case ARCHEAD_FMT_ARCHEAD:
      switch ((a.N + 15) / 16) {
        case 2: return launch_t<ARCHEAD_FMT_ARCHEAD, 2>(a, s);
        case 3: return launch_t<ARCHEAD_FMT_ARCHEAD, 3>(a, s);
        case 4: return launch_t<ARCHEAD_FMT_ARCHEAD, 4>(a, s);
        default: return hipErrorInvalidValue;
      }
    case ARCHEAD_FMT_GROUP_INT4: return launch_batch_group_int4(a, s);
    case ARCHEAD_FMT_ROW_INT8: return launch_batch_row_int8(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace archead
