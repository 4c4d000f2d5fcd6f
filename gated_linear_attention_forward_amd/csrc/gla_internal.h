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
  // token ranges: the N tokens of a head form NB attention blocks of BT tokens
  // (the last may be shorter); a kernel's range index c covers block c / CB,
  // piece c % CB, whose L tokens start at (c / CB) * BT + (c % CB) * L and
  // end at the block's end at the latest
  int L;                 // tokens per range (state: chunk, output: block range)
  int CB;                // ranges per attention block for this kernel
  int BT, NB;            // tokens per attention block, attention blocks per head
  int C;                 // state chunks per head (NB * state CB)
  // RoPE: factorised (cos, sin) table, [T][Pt] | [Hh][Py] | [W][Px] float2
  const float2* cs;      // nullptr: RoPE off
  int T, Hh, W, Pt, Py, Px;
  DivMagic div_hw, div_w;
  int nt;                // t-rows of the table staged per block (when staged in LDS)
  // workspace
  float* part;           // [BH][C][D*D + D] fp32 chunk partials
  uint16_t* sl;          // [BH][NB][D + 2][D] bf16: per attention block, the state
                         // S^T rows in output order, then z hi/lo rows
  uint16_t* sl2;         // optional [BH][NB][D][D] bf16: the state's rows S[d][0..D)
                         // in the same row order (row R(d) holds row d)
  float* S_out;          // optional fp32 S [BH][D][D] after the last block
  float* z_out;          // optional fp32 z [BH][D] after the last block
  const float* S_in;     // optional carried fp32 S [BH][D][D] (NULL: zero)
  const float* z_in;     // optional carried fp32 z [BH][D] (NULL: zero)
};

// How one call splits its work.  Filled by make_plan on the host.
struct Plan {
  int B, N, H, D;
  int BH;
  // attention blocks: NB per head of BT tokens (one block of N tokens for the
  // bidirectional mixer)
  int BT, NB;
  // state kernel: CB chunks per attention block of L tokens (L a multiple of
  // 16), C = NB * CB chunks per head
  int CB, C, L;
  // output kernel: SUB ranges per attention block of L2 tokens (L2 a multiple
  // of 64), C2 = NB * SUB ranges per head
  int SUB, C2, L2;
  // workspace byte offsets and total size
  size_t off_part, off_sl, ws_bytes;
};

// Tile sizes the plan has to respect.
constexpr int kOutputTileTokens = 64;
constexpr int kMaxChunks = 256;
// Blocks of the state kernel the plan aims for: one per compute unit (256
// compute units); a block's waves together hold a full D x D accumulator.
constexpr int kStateBlocks = 256;
// Each wave of a state block should see at least this many 16-token tiles.
constexpr int kStateMinTilesPerWave = 2;
constexpr int kOutputBlocks = 2048;
// The persistent output kernel (one attention block per head): blocks per
// launch it aims for (one per compute unit), the LDS each block asks for (so
// that no two blocks share a compute unit) and the largest RoPE table it
// stages whole.
constexpr int kPersistBlocks = 256;
constexpr size_t kPersistLdsBytes = 90 * 1024;
constexpr size_t kMaxPersistTableBytes = 56 * 1024;
// Steps per wave below which the persistent output kernel keeps one head
// per block (staging several heads' operands would not pay).
constexpr int kGroupMinSteps = 16;
// Limits for folding the reduction into the output kernel: partial bytes
// one block reads, and all blocks together.
constexpr size_t kFoldBlockBytes = 64 * 1024;
constexpr size_t kFoldTotalBytes = 4 << 20;
constexpr int kFoldMaxChunks = 16;
// Largest N * D a one-launch pass takes (one block streams a head's tokens).
constexpr long long kInBlockMaxND = 32768;
// LDS a block may ask for on gfx950 (160 KB per compute unit).
constexpr size_t kMaxLdsPerBlock = 160 * 1024;
// The backward pass's query and key kernels (8 waves, one block per compute
// unit) take their token ranges from a plan of at most this many blocks:
// one round of long ranges, each block staging its head's operands once.
constexpr int kBackwardBlocks = 256;
// Largest RoPE table slice (bytes) a block stages in LDS; larger grids read
// the table from global memory instead.
constexpr int kMaxLdsTableBytes = 24 * 1024;

// block_tokens <= 0 or >= N: one attention block (the bidirectional mixer).
// output_blocks: the most blocks the output-side ranges (SUB, L2) may take.
Plan make_plan(int B, int N, int H, int D, int block_tokens = 0,
               int output_blocks = kOutputBlocks);

// The fixed per-device scratch of the no-allocation entry point (gla_kernels.hip):
// its size, and its device address on the current device (looked up on the
// first call per device).
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_pointer(void** out);

// Kernel launchers (gla_kernels.hip).  Return the hipError_t of the launch.
// State kernel, then (unless `reduce` is false) the cross-chunk reduction.
hipError_t launch_state(const Plan& p, KArgs a, hipStream_t stream, bool reduce = true);
// The scan alone over zero blocks: S_out/z_out = S_in/z_in (or zero).
hipError_t launch_carry(const Plan& p, KArgs a, hipStream_t stream);
// Output kernel.  With `sum_partials` its blocks sum the chunk partials
// (a.part) themselves, in place of reading the reduced operand (a.sl).
hipError_t launch_output(const Plan& p, KArgs a, hipStream_t stream, bool sum_partials = false);
// True when a bidirectional pass of this plan runs with the reduction folded
// into the output kernel's prologue: the chunk partials are small (D <= 64,
// a few KB per head and block), so re-reading them in every output block
// costs less than a launch of the reduce kernel.
bool output_sums_partials(const Plan& p);
// True when a bidirectional pass of this plan runs as one launch: one block
// per head forms the head's state from all N tokens and then its outputs
// (short sequences at D <= 64, where launches, not bytes, set the time).
bool pass_in_block(const Plan& p);
// That launch: reads a.q, a.k, a.v, a.g and a.cs, writes a.out (no workspace).
hipError_t launch_pass_in_block(const Plan& p, KArgs a, hipStream_t stream);
// Gated softmax anchor attention (gla_softmax.hip): prep (rotated, scaled q
// into qr, rotated k into kr, [B, N, H, D] bf16 each) then the flash kernel.
// Reads a.q, a.k, a.v, a.g, a.cs (nullptr: RoPE off), writes a.out.
hipError_t launch_softmax(const Plan& p, KArgs a, uint16_t* qr, uint16_t* kr, hipStream_t stream);

// Backward pass of the bidirectional mixer (gla_backward.hip).
struct BArgs {
  const uint16_t* dout;  // output gradient [B, N, H, D] bf16
  uint16_t* dq;          // gradients written [B, N, H, D] bf16
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dg;
  const float* z;        // forward z [BH][D] fp32
  float* dsp;            // [BH][C2][D*D + D] fp32 per-range partials: dS = sum rq a^T
                         // (row-major, rq features by a features), then dz
  const float* dz;       // [BH][D] fp32 dz (the reduce of dsp's last D entries)
  int C2;                // query/key kernel ranges per head
};
// Query side: reads q, g, dout and the state operands a.sl (S^T rows + z
// rows) and a.sl2 (S rows); writes dq, dg and the dS and dz partials dsp.
hipError_t launch_bwd_query(const Plan& p, KArgs a, BArgs b, hipStream_t stream);
// Key side: reads k, v, the gradient-state operands a.sl (dS^T rows) and
// a.sl2 (dS rows) and dz; writes dk, dv.
hipError_t launch_bwd_key(const Plan& p, KArgs a, BArgs b, hipStream_t stream);

// Projection prologue (gla_project.hip): q, k, v, g = x W^T per map.
struct PArgs {
  const uint16_t* x;     // hidden states [B, N, C] bf16
  const uint16_t* w;     // stacked weights [4][H * D][C] bf16 (q, k, v, g)
  int Cdim;              // hidden size C (a multiple of 64)
  uint16_t* qbuf;        // projected q [B, N, H, D] bf16 (written)
  uint16_t* gbuf;        // projected g [B, N, H, D] bf16 (written)
};
// akv: the state plan's chunks (writes a.part, as the state kernel does);
// aqg: token tiles of kProjTileTokens (one per range; writes qbuf, gbuf).
hipError_t launch_proj(const Plan& p, KArgs akv, KArgs aqg, PArgs pa, hipStream_t stream);
// The reduce kernel alone over the state partials in a.part.
hipError_t launch_reduce_state(const Plan& p, KArgs a, hipStream_t stream);
constexpr int kProjTileTokens = 256;


}  // namespace gla
