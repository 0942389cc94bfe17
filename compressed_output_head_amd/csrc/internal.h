// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "archead.h"

namespace archead {

constexpr int kKTile = 128;        // columns per residual tile
constexpr int kTileBytes = 1024;   // 16 rows x 128 columns of INT4
constexpr int kMaxRank = 1024;     // per part (r_c, r_r)
constexpr int kDecodeMaxTokens = 64;
// Up to this many tokens the decode kernel may keep all of H in LDS.
constexpr int kDecodeLdsTokens = 16;
// LDS budget of that kernel: N*(D+8)*2 bytes of H plus N*r*4 bytes of Z.
constexpr uint64_t kDecodeLdsBytes = 48 * 1024;
// Workspace for the fp32 partial sums of tiles whose hidden dimension the
// tile kernel splits over several workgroups (calls of more than
// kDecodeLdsTokens tokens).
constexpr uint64_t kSplitBytes = 64ull << 20;

inline uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Checks shared by every entry point.  Returns ARCHEAD_OK or an error.
int check_dims(const archead_dims* d);
// Additional limits of the kernels (rank a multiple of 8, g in {32,64,128,256}).
int check_kernel_dims(const archead_dims* d);
void compute_layout(const archead_dims* d, archead_layout* L);

// Device workspace of one call (all offsets 256-byte aligned).
struct WorkspaceLayout {
  int64_t n16;          // tokens rounded up to 16
  int64_t n32;          // tokens rounded up to 32 (rows of every per-token workspace section)
  int rc32, rr32;       // ranks rounded up to 32
  int zsteps;           // (rc32 + rr32) / 32
  uint64_t hf, hscale, zf, zscale, z32, hc, split, split_bytes;
  uint64_t st_part, st_y;  // row statistics only: pieces [N][st_nparts], Y [N][V] fp32 for N <= 16
  int64_t st_nparts;
  uint64_t total;
};
WorkspaceLayout workspace_layout(const archead_dims* d, int64_t n_tokens, bool stats = false);

// Everything a kernel needs, resolved to raw device pointers.
struct FwdArgs {
  // dims
  int64_t V, D, N, n16, n32, nb;   // nb = V16/16 row blocks
  int r_c, r_r, g, ng, nkt, nks, rc32, rr32, zsteps, nA;
  // input / output
  const uint16_t* H;          // bf16 [N][H_stride]
  int64_t H_stride;
  void* Y;                    // fp32 or bf16 [N][Y_stride]
  int64_t Y_stride;
  int y_bf16;
  // packed head sections
  const uint8_t* r_codes;
  const uint8_t* r_gcodes;
  const uint16_t* r_rowscale;
  const int8_t* a_codes;
  const uint16_t* a_scales;
  const int8_t* b_codes;
  const uint16_t* b_scales;
  // workspace
  // hf/zf hold either the 16-row operand layout (16 x 16 x 32 MFMA kernels) or
  // the 32-row layout (32 x 32 x 16 MFMA kernel), whichever the chosen main
  // kernel reads:
  //   16-row: hf [n16/16][D/32][64][8],          zf [n16/16][2*zsteps][64][8]
  //   32-row: hf [n32/32][D/128][8][64][8],      zf [n32/32][4*zsteps][64][8]
  _Float16* hf;               // converted, scaled H
  float* hscale;              // [n32]
  _Float16* zf;               // hi/lo pre-projection
  float* zscale;              // [n32]
  float* z32;                 // [n32][r] fp32 pre-projection
  _Float16* hc;               // [N][D] scaled fp16 H rows in kernel k-order (small-N decode path only)
  float* part;                // fp32 partial sums of split tiles (null: no room, tiles are not split)
  uint64_t part_bytes;
  // row statistics (archead_logits_stats): pieces [N][st_nparts] of 16 bytes
  float* st_part;
  int64_t st_nparts;
  const int32_t* targets;     // [N] or null
};

hipError_t launch_prep(const FwdArgs& a, bool rows32, hipStream_t s);
bool tile32_eligible(const FwdArgs& a);
hipError_t launch_prep_z(const FwdArgs& a, hipStream_t s);
bool decode_lds_eligible(const FwdArgs& a);
hipError_t launch_decode_lds(const FwdArgs& a, hipStream_t s);
hipError_t launch_decode(const FwdArgs& a, hipStream_t s);
bool mid_eligible(const FwdArgs& a);
hipError_t launch_mid(const FwdArgs& a, hipStream_t s);
hipError_t launch_tile(const FwdArgs& a, hipStream_t s);
int tile_stat_parts(const FwdArgs& a);
hipError_t launch_tile_stats(const FwdArgs& a, hipStream_t s);
// statistics pieces of a fp32 Y already in memory, kStatChunks per token
constexpr int kStatChunks = 64;
hipError_t launch_rowstats_y(const FwdArgs& a, const float* Y, int64_t y_stride, hipStream_t s);
// merge a.st_nparts pieces per token into the outputs (null: not written)
hipError_t launch_stats_reduce(const FwdArgs& a, float* row_max, int32_t* row_argmax, float* row_lse,
                               float* row_ce, hipStream_t s);

}  // namespace archead
