// Row statistics on the large-N tile kernel: its instances that reduce each
// workgroup's logits to statistics pieces instead of storing Y.
#include "tile32.h"

namespace archead {

// Statistics pieces of every (token, 256-row vocabulary tile) into
// a.st_part[token][vt]; the caller has checked tile32_eligible.
int tile_stat_parts(const FwdArgs& a) { return t32_grid(a, t32_tt(a)).vtiles; }

hipError_t launch_tile_stats(const FwdArgs& a, hipStream_t s) {
  switch (t32_tt(a)) {
    case 2: return launch_t32<2, true>(a, s);
    case 4: return launch_t32<4, true>(a, s);
    default: return launch_t32<8, true>(a, s);
  }
}

}  // namespace archead
