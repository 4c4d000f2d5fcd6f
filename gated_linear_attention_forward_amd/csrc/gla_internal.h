// gla_internal.h -- declarations shared by the host API and the HIP kernels
// of the gated bidirectional linear-attention mixer (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gla {

// Exact unsigned division by an invariant divisor d >= 1 for 32-bit
// numerators (multiply-high, add, shift; Granlund & Montgomery 1994):
//   t = mulhi(n, m);  n / d = (t + ((n - t) >> s1)) >> s2.
struct DivMagic {
  uint32_t m;
  int s1, s2;
};

DivMagic make_div_magic(uint32_t d);

// Everything a kernel launch needs, passed by value.
struct KArgs {
  // tensors of one call; each batch element's [N, H, D] slab is addressed with
  // 32-bit byte offsets from its own base
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  uint16_t* out;
  int N, H;
  uint32_t slab_bytes;   // N * H * D * 2
  int L;                 // tokens per block (state: chunk, output: block range)
  int C;                 // state chunks per head
  // RoPE: factorised (cos, sin) table, [T][Pt] | [Hh][Py] | [W][Px] float2
  const float2* cs;      // nullptr: RoPE off
  int T, Hh, W, Pt, Py, Px;
  DivMagic div_hw, div_w;
  int nt;                // t-rows of the table staged per block (when staged in LDS)
  // workspace
  float* part;           // [BH][C][D*D + D] fp32 chunk partials
  uint16_t* sl;          // [BH][D + 2][D] bf16: S^T rows in output order, then z hi/lo rows
  float* zf;             // [BH][D] fp32 z
  float* S_out;          // optional fp32 S [BH][D][D]
  float* z_out;          // optional fp32 z [BH][D]
};

// How one call splits its work.  Filled by make_plan on the host.
struct Plan {
  int B, N, H, D;
  int BH;
  // state kernel: C chunks per head of L tokens (L a multiple of its tile)
  int C, L;
  // output kernel: C2 blocks per head of L2 tokens (L2 a multiple of 64)
  int C2, L2;
  // workspace byte offsets and total size
  size_t off_part, off_sl, off_z, ws_bytes;
};

Plan make_plan(int B, int N, int H, int D);

// Kernel launchers (gla_kernels.hip).  Return the hipError_t of the launch.
hipError_t launch_state(const Plan& p, KArgs a, hipStream_t stream);
hipError_t launch_output(const Plan& p, KArgs a, hipStream_t stream);

// Tile sizes the plan has to respect.
constexpr int state_tile_tokens(int D) { return 8192 / D; }
constexpr int kOutputTileTokens = 64;
constexpr int kMaxChunks = 256;
// Blocks of the state kernel the plan aims for: one per compute unit (256
// compute units); a block's waves together hold a full D x D accumulator.
constexpr int state_blocks(int D) { return D > 0 ? 256 : 256; }
// Each wave of a state block should see at least this many 16-token tiles.
constexpr int kStateMinTilesPerWave = 2;
constexpr int kOutputBlocks = 2048;
// Largest RoPE table slice (bytes) a block stages in LDS; larger grids read
// the table from global memory instead.
constexpr int kMaxLdsTableBytes = 24 * 1024;

}  // namespace gla
