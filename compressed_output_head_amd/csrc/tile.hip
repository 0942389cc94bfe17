// Tile path (every call the decode kernel does not take): the 32 x 32 x 16
// MFMA tile kernel of tile32.h with the logits as output.
//
// Y = [H | Z] [R | A_c ; A_w]^T, i.e. Algorithm 1's inference step with the
// quantised core evaluated through the same (H B^T) A^T association.
#include "tile32.h"

namespace archead {

// The tile kernel serves any call whose sections fit 32-bit buffer offsets.
bool tile32_eligible(const FwdArgs& a) {
  if ((uint64_t)a.nb * 16 * (uint64_t)a.D / 2 >= (1ull << 32)) return false;
  if (((uint64_t)a.nb * 16 + kT32CB * 32) * (uint64_t)a.ng >= (1ull << 32)) return false;
  if ((uint64_t)a.nb * 16 * (uint64_t)(a.r_c + a.r_r) >= (1ull << 32)) return false;
  if ((uint64_t)a.n32 * (uint64_t)a.D * 2 >= (1ull << 32)) return false;
  if (a.ng > kT32MaxCodes) return false;
  const T32Grid G = t32_grid(a, t32_tt(a));
  return (int64_t)G.ttiles * G.vtiles < (1ll << 31);
}

hipError_t launch_tile(const FwdArgs& a, hipStream_t s) {
  switch (t32_tt(a)) {
    case 2: return launch_t32<2, false>(a, s);
    case 4: return launch_t32<4, false>(a, s);
    default: return launch_t32<8, false>(a, s);
  }
}

}  // namespace archead
