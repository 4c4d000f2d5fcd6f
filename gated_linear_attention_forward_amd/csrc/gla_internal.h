// gla_internal.h -- declarations shared by the host API and the HIP kernels
// of the gated bidirectional linear-attention mixer (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gla {

// RoPE description handed to the kernels by value.  cs holds (cos, sin)
// pairs laid out [T][Pt] | [Hh][Py] | [W][Px]; cs == nullptr means RoPE off.
struct RopeArgs {
  const float2* cs;
  int T, Hh, W;
  int Pt, Py, Px;
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
hipError_t launch_state(const Plan& p, const uint16_t* k, const uint16_t* v, const RopeArgs& rope,
                        void* ws, float* S_out, float* z_out, hipStream_t stream);
hipError_t launch_output(const Plan& p, const uint16_t* q, const uint16_t* g,
                         const RopeArgs& rope, const void* ws, uint16_t* out,
                         hipStream_t stream);

// Tile sizes the plan has to respect.
constexpr int state_tile_tokens(int D) { return 8192 / D; }
constexpr int kOutputTileTokens = 64;
constexpr int kMaxChunks = 256;

}  // namespace gla
