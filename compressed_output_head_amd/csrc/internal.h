// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "archead.h"

namespace archead {

constexpr int kKTile = 128;        // columns per residual tile
constexpr int kTileBytes = 1024;   // 16 rows x 128 columns of INT4
constexpr int kMaxRank = 1024;     // per part (r_c, r_r)
// The decode kernel takes up to this many tokens (all of H and Z in LDS).
constexpr int kDecodeMaxTokens = 16;
// LDS one workgroup may use on gfx950.
constexpr uint32_t kMaxLdsBytes = 160 * 1024;
// Workspace for the fp32 partial sums of tiles whose hidden dimension the
// tile kernel splits over several workgroups.
constexpr uint64_t kSplitBytes = 64ull << 20;

inline uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Events a caller of archead_logits_events asked for: the start of the main
// kernel and the end of the last kernel of the forward (the main kernel, or
// the tile path's reduce kernel of split tiles).  Set for the duration of one
// call on the calling thread and consumed by launch_main.
struct MainEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
MainEvents& main_events();

// Launch a kernel of the forward; with events pending on this thread, the
// launch itself records them (AMD's launch with start and stop events: the
// dispatch's own timestamps, no separate markers on the stream).  last: no
// kernel of the forward follows this one.
template <typename F, typename... Args>
hipError_t launch_main(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, bool last, Args... args) {
  MainEvents& e = main_events();
  hipEvent_t start = e.start, stop = last ? e.stop : nullptr;
  if (start || stop) {
    e.start = nullptr;
    if (last) e.stop = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, start, stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
  return hipGetLastError();
}

// Checks shared by every entry point.  Returns ARCHEAD_OK or an error.
int check_dims(const archead_dims* d);
// Additional limits of the kernels (rank a multiple of 8, g in {32,64,128,256}).
int check_kernel_dims(const archead_dims* d);
// E_UNSUPPORTED for a comparison head (entry points that serve the ARCHead format only).
int check_archead_format(const archead_dims* d);
// Tokens per launch of the batched kernel for a comparison head.
constexpr int64_t kAltChunk = 32;
void compute_layout(const archead_dims* d, archead_layout* L);

// Whether a call with n_tokens rows of H runs the decode kernel (pure host
// arithmetic: dims, token count and the LDS the kernel would need).
bool decode_fits(const archead_dims* d, int64_t n_tokens);
// the few-token decode path (decode_small.hip) takes the call
bool small_decode_fits(const archead_dims* d, int64_t n_tokens);
// the batched decode kernel (batch.hip, 17 to 64 tokens) takes the call
bool batch_fits(const archead_dims* d, int64_t n_tokens);
// workspace of a decode-path call: partial sums of Z
uint64_t decode_workspace_bytes(const archead_dims* d, int64_t n_tokens);

// Device workspace of one call (all offsets 256-byte aligned).  The decode
// kernel needs none (its statistics call needs the pieces and Y); the tile
// path needs the converted H, Z and the partial sums of split tiles.
struct WorkspaceLayout {
  bool decode;          // the call runs the decode path
  bool small;           // ... and its few-token kernels
  bool batch;           // ... and its batched kernel (same workspace as the few-token kernels)
  int64_t n32;          // tokens rounded up to 32 (rows of every per-token workspace section)
  int rc32, rr32;       // ranks rounded up to 32
  int zsteps;           // (rc32 + rr32) / 32
  int zsl;              // few-token kernel: slices of D in the partial sums of Z (else 1)
  uint64_t hf, hscale, zf, zscale, z32, hc, split, split_bytes;
  uint64_t st_part, st_y;  // row statistics only: pieces [N][st_nparts], Y [N][V] fp32 (decode kernel)
  int64_t st_nparts;
  uint64_t total;
};
// split_cap bounds the section for partial sums of split tiles (0: none);
// allow_decode = false lays out the tile path's workspace for any call.
WorkspaceLayout workspace_layout(const archead_dims* d, int64_t n_tokens, bool stats = false,
                                 uint64_t split_cap = kSplitBytes, bool allow_decode = true);

// Everything a kernel needs, resolved to raw device pointers.
struct FwdArgs {
  // dims
  int64_t V, D, N, n32, nb;        // nb = V16/16 row blocks
  int r_c, r_r, g, ng, nkt, nks, rc32, rr32, zsteps, nA;
  int fmt;                         // archead_format of the packed head
  int zsl;                         // few-token path: slices of D whose partial sums of Z the prep writes (else 1)
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
  // workspace of the tile path: operand fragments of the 32 x 32 x 16 MFMA,
  //   hf [n32/32][D/128][8][64][8],  zf [n32/32][4*zsteps][64][8]
  _Float16* hf;               // converted, scaled H
  _Float16* hc;               // few-token decode path: H [N][D] converted in kernel k-order
  float* hscale;              // [n32]
  _Float16* zf;               // hi/lo pre-projection
  float* zscale;              // [n32]
  float* z32;                 // tile path: [n32][r] fp32 pre-projection; decode path: its partial sums
  float* part;                // fp32 partial sums of split tiles (null: no room, tiles are not split)
  uint64_t part_bytes;
  // row statistics (archead_logits_stats): pieces [N][st_nparts] of 16 bytes
  float* st_part;
  int64_t st_nparts;
  const int32_t* targets;     // [N] or null
};

// tile path: H and Z into the workspace, then the tile kernel
hipError_t launch_prep(const FwdArgs& a, hipStream_t s);
// parts of the hidden dimension in the tile path's fp32 Z ([parts][n32][r])
int zmm_parts(int64_t n32, int r, int64_t D, int g);
bool tile32_eligible(const FwdArgs& a);
hipError_t launch_tile(const FwdArgs& a, hipStream_t s);
// decode path: the partial sums of Z into the workspace, then the streaming kernel
hipError_t launch_decode_prep(const FwdArgs& a, hipStream_t s);
hipError_t launch_small_prep(const FwdArgs& a, hipStream_t s);
// slices of D over which the few-token pre-projection splits each element of Z
int small_z_slices(int64_t D, int64_t n_tokens);
hipError_t launch_small_decode(const FwdArgs& a, hipStream_t s);
hipError_t launch_decode(const FwdArgs& a, hipStream_t s);
hipError_t launch_batch(const FwdArgs& a, hipStream_t s);
int tile_stat_parts(const FwdArgs& a);
hipError_t launch_tile_stats(const FwdArgs& a, hipStream_t s);
// statistics pieces of a fp32 Y already in memory, kStatChunks per token
constexpr int kStatChunks = 64;
hipError_t launch_rowstats_y(const FwdArgs& a, const float* Y, int64_t y_stride, hipStream_t s);
// merge a.st_nparts pieces per token into the outputs (null: not written)
hipError_t launch_stats_reduce(const FwdArgs& a, float* row_max, int32_t* row_argmax, float* row_lse,
                               float* row_ce, hipStream_t s);

}  // namespace archead
