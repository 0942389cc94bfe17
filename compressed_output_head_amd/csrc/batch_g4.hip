// Instances of the batched streaming kernel for the group INT4 with fp16 group scales comparison
// head (one or two 16-token tiles: the library launches it on at most 32
// tokens at a time).
#include "batch_kernel.h"

namespace archead {

hipError_t launch_batch_group_int4(const FwdArgs& a, hipStream_t s) {
  switch ((a.N + 15) / 16) {
    case 1: return launch_t<ARCHEAD_FMT_GROUP_INT4, 1>(a, s);
    case 2: return launch_t<ARCHEAD_FMT_GROUP_INT4, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace archead
