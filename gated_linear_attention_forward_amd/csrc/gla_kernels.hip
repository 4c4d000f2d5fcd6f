// gla_kernels.hip -- gfx950 kernels of the gated bidirectional linear-attention
// token mixer ("SANA-Video 2.0", NVlabs Sana docs, section Architecture:
// gated bidirectional linear attention with Wan 3D rotary embeddings).
//
// Per head (b, h), with phi = ReLU and R_n the RoPE rotation of token n:
//   S = sum_n (R_n phi(k_n)) v_n^T,  z = sum_n phi(k_n),
//   o_n = sigmoid(g_n) * ((R_n phi(q_n))^T S) / (phi(q_n).z + eps).
// "Bidirectional" means S and z sum over every token, so the work is a
// reduction over N followed by a map over N:
//   state kernel   each block reduces one chunk of one head's tokens into an
//                  fp32 partial (S_c, z_c) on bf16 MFMA (32x32x16);
//   reduce kernel  sums the chunk partials of a head in a fixed pairwise tree
//                  and stores S (bf16) and z (as a bf16 hi/lo pair) in the
//                  output kernel's operand layout;
//   output kernel  streams q and g, contracts R phi(q) with the LDS-resident S
//                  and phi(q) with z on bf16 MFMA (16x16x32), applies the
//                  normaliser and the gate, and writes bf16 out.
// All tensors are bf16 [B, N, H, D].  A head's D-vector of a token is 2D
// contiguous bytes; consecutive tokens are H*D*2 bytes apart.  Global
// traffic goes through buffer instructions with 32-bit offsets from each
// batch element's slab; a lane whose token lies outside its block's range
// uses an offset past the end of the buffer, which the hardware turns into
// zero loads and dropped stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {
namespace {
// ---------------------------------------------------------------------------
// State kernel.
//
// Block = 4 waves, one (chunk, head); the waves are independent until the
// block's end.  Each wave owns a full D x D fp32 accumulator (for D = 128,
// 256 accumulation registers per lane, one wave per SIMD) and streams the
// 16-token tiles w, w + 4, w + 8, ... of its block's chunk.  In a tile, lane
// l takes token l % 16 and the 16-byte chunks 4s + l/16 (s < D/32) of that
// token's k and v (one grid position per lane and tile; half of the RoPE
// pair slots resolve their table row at compile time).  ReLU and RoPE are
// applied to k in fp32 registers, z accumulates the unrotated features, and
// R phi(k) (bf16) and v are written to the wave's LDS tile in their natural
// token-major layout.  The MFMA operands of S += sum_n rk_n v_n^T contract
// over tokens, so they are read back with ds_read_b64_tr_b16: within each
// 16-lane group, source lane a + 4r points at 4 features of token r and
// destination lane 4a + b receives feature b of tokens 0..3; two such reads
// give a lane the 8 tokens of one feature that v_mfma_f32_32x32x16_bf16
// takes.  Row pitches are padded to 2D + 32 bytes so the four rows a 16-lane
// group touches fall on distinct banks.
//
// The loop is software-pipelined: step i issues the MFMAs of tile i - 1,
// whose operands were read from LDS in step i - 1, while it prepares tile i
// (ReLU, RoPE, LDS staging into the other of two tile buffers, operand
// reads); the global loads run PF tiles ahead in a register ring.  A tile
// past the wave's last one loads zeros (offsets outside the buffer) and adds
// exactly nothing.  At the end the four accumulators are added in wave
// order through LDS.
template <int D>
struct StateCfg {
  static constexpr int KS = D / 32;         // 16-byte chunks per lane and token
  static constexpr int TW = 16;             // tokens per wave tile
  static constexpr int RT = D / 32;         // 32x32 accumulator tiles per dimension
  static constexpr int RP = 2 * D + 32;     // LDS row pitch, bytes
  static constexpr int BUF_BYTES = 2 * TW * RP;      // k and v tiles
  static constexpr int WAVE_BYTES = 2 * BUF_BYTES;   // double-buffered
  static constexpr int TILE_BYTES = 4 * WAVE_BYTES;
  static constexpr int PF = 2;              // tiles in flight per wave
  // block-end reduction: 32x32 accumulator tiles added per round (each takes
  // 4 KB per wave), followed by the four waves' z vectors
  static constexpr int RED_FIT = (TILE_BYTES - 16 * D) / (4 * 4096);
  static constexpr int RED_TILES = RED_FIT < 1 ? 1 : (RED_FIT > RT * RT ? RT * RT : RED_FIT);
  static constexpr int ZW_OFF = 4 * RED_TILES * 4096;
  static constexpr int LDS_BYTES = TILE_BYTES > ZW_OFF + 16 * D ? TILE_BYTES : ZW_OFF + 16 * D;
};

template <int D, bool ROPE>
struct StateWave {
  using Cf = StateCfg<D>;
  static constexpr int KS = Cf::KS;
  const KArgs& a;
  const TabView& tv;
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t tokstride, headoff;
  int n_begin, n_end, wave, nit, lane, m, col;
  unsigned char* buf;  // this wave's two tile buffers
  u32x4 kr[Cf::PF][KS], vr[Cf::PF][KS];
  bf16x8 A[2][Cf::RT], Bv[2][Cf::RT];
  float2 cs[KS][4];    // RoPE factors of the tile being prepared
  float zacc[KS][8];
  f32x16 acc[Cf::RT][Cf::RT];

  __device__ __forceinline__ int token(int it) const {
    return n_begin + Cf::TW * (wave + 4 * it) + col;
  }

  __device__ __forceinline__ void issue(int st, int it) {
    const int n = token(it);
    const uint32_t off = (it < nit && n < n_end) ? (uint32_t)n * tokstride + headoff : kOob;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      kr[st][s2] = load16_nt(rk, off + 64u * s2);
      vr[st][s2] = load16_nt(rv, off + 64u * s2);
    }
  }

  // LDS reads of tile `it`'s RoPE factors (they complete while the step
  // issues its operand reads and MFMAs)
  __device__ __forceinline__ void load_factors(int it) {
    if (!ROPE) return;
    int t, y, x;
    grid_pos(a, (uint32_t)min(token(it), n_end - 1), t, y, x);
    const RowOff ro = row_offsets<D>(a, tv, t, y, x);
    static_for<KS>([&](auto S2) {
      constexpr int s2 = decltype(S2)::value;
      rope_factors<D, s2>(tv, ro, m, cs[s2]);
    });
  }

  // ReLU, z and RoPE of tile `it` (ring slot ST), staged into tile buffer PB;
  // then the loads of tile it + PF go into the freed ring slot
  template <int ST, int PB>
  __device__ __forceinline__ void stage(int it) {
    unsigned char* ktile = buf + PB * Cf::BUF_BYTES;
    unsigned char* vtile = ktile + Cf::TW * Cf::RP;
    u32x4 rkw[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      u32x4 fq;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        fq[u] = relu2(kr[ST][s2][u]);
        zacc[s2][2 * u] += bf_lo(fq[u]);
        zacc[s2][2 * u + 1] += bf_hi(fq[u]);
      }
      rkw[s2] = ROPE ? rotate_chunk(fq, cs[s2]) : fq;
    }
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      *reinterpret_cast<u32x4*>(ktile + col * Cf::RP + 16 * (4 * s2 + m)) = rkw[s2];
      *reinterpret_cast<u32x4*>(vtile + col * Cf::RP + 16 * (4 * s2 + m)) = vr[ST][s2];
    }
    issue(ST, it + Cf::PF);
  }

  // MFMA operands of the tile staged in buffer PB.  The LDS executes one
  // wave's instructions in order, so these reads see that wave's staging
  // writes of an earlier step without a wait; the compiler barrier keeps
  // the program order.
  template <int PB>
  __device__ __forceinline__ void read_operands() {
    asm volatile("" ::: "memory");
    const unsigned char* ktile = buf + PB * Cf::BUF_BYTES;
    const unsigned char* vtile = ktile + Cf::TW * Cf::RP;
#pragma unroll
    for (int i = 0; i < Cf::RT; ++i) A[PB][i] = frag_tr(ktile, Cf::RP, i, lane);
#pragma unroll
    for (int j = 0; j < Cf::RT; ++j) Bv[PB][j] = frag_tr(vtile, Cf::RP, j, lane);
  }

  template <int PB>
  __device__ __forceinline__ void contract() {
#pragma unroll
    for (int i = 0; i < Cf::RT; ++i)
#pragma unroll
      for (int j = 0; j < Cf::RT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[PB][i], Bv[PB][j], acc[i][j], 0, 0, 0);
  }

  // step `it` (parity P = it % 2): factors of tile it, operands of tile
  // it - 1, MFMAs of tile it - 2, staging of tile it
  template <int P>
  __device__ __forceinline__ void step(int it) {
    load_factors(it);
    read_operands<1 - P>();
    contract<P>();
    asm volatile("" ::: "memory");
    stage<P, P>(it);
  }

  __device__ __forceinline__ void run() {
#pragma unroll
    for (int i = 0; i < Cf::RT; ++i)
#pragma unroll
      for (int j = 0; j < Cf::RT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int j = 0; j < 8; ++j) zacc[s2][j] = 0.f;
    static_assert(Cf::PF == 2, "the ring, the buffers and the operand sets alternate together");
    issue(0, 0);
    issue(1, 1);
    load_factors(0);
    stage<0, 0>(0);
    load_factors(1);
    read_operands<0>();
    asm volatile("" ::: "memory");
    stage<1, 1>(1);
    // tile j is contracted in step j + 2; tiles past the wave's last are
    // zero, so the loop runs whole pairs of steps up to step nit + 1
    for (int it = 2; it < nit + 2; it += 2) {
      step<0>(it);
      step<1>(it + 1);
    }
  }
};

template <int D, bool ROPE, bool TLDS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void state_kernel(KArgs a) {
  using Cf = StateCfg<D>;
  constexpr int KS = Cf::KS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float2* ltab = reinterpret_cast<float2*>(smem + Cf::LDS_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int m = lane >> 4;
  const int col = lane & 15;
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  int n_begin, n_end;
  range_of(a, c, n_begin, n_end);

  TabView tv{};
  if (ROPE) tv = stage_table<D>(a, ltab, TLDS, n_begin, n_end);
  __syncthreads();

  const size_t boff = (size_t)b * a.N * a.H * D;
  const int ntile = (n_end - n_begin + Cf::TW - 1) / Cf::TW;
  StateWave<D, ROPE> w{a,
                       tv,
                       make_rsrc(a.k + boff, a.slab_bytes),
                       make_rsrc(a.v + boff, a.slab_bytes),
                       (uint32_t)a.H * D * 2,
                       (uint32_t)h * D * 2 + 16u * m,
                       n_begin,
                       n_end,
                       wave,
                       (ntile - wave + 3) / 4,
                       lane,
                       m,
                       col,
                       smem + wave * Cf::WAVE_BYTES};
  w.run();

  // z of this wave: the 16 lanes of a lane group hold the same features
#pragma unroll
  for (int msk = 1; msk < 16; msk *= 2)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int j = 0; j < 8; ++j) w.zacc[s2][j] += __shfl_xor(w.zacc[s2][j], msk);

  __syncthreads();  // every wave is done with its tiles; they become scratch
  float* red = reinterpret_cast<float*>(smem);
  float* dst = a.part + ((size_t)bh * a.C + c) * (size_t)(D * D + D);
  float* zw = reinterpret_cast<float*>(smem + Cf::ZW_OFF);
  if (col == 0) {
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int j = 0; j < 8; ++j) zw[wave * D + 8 * (4 * s2 + m) + j] = w.zacc[s2][j];
  }
  __syncthreads();
  if (tid < D) dst[D * D + tid] = ((zw[tid] + zw[D + tid]) + zw[2 * D + tid]) + zw[3 * D + tid];
  __syncthreads();

  // S: add the four waves' accumulators, RED_TILES 32x32 tiles per round
  constexpr int NT = Cf::RT * Cf::RT;
  constexpr int WSTRIDE = Cf::RED_TILES * 1024;  // floats per wave per round
#pragma unroll
  for (int t0 = 0; t0 < NT; t0 += Cf::RED_TILES) {
#pragma unroll
    for (int q = 0; q < Cf::RED_TILES; ++q) {
      if (t0 + q < NT) {
        const int ti = (t0 + q) / Cf::RT, tj = (t0 + q) % Cf::RT;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          red[wave * WSTRIDE + (q * 16 + r) * 64 + lane] = w.acc[ti][tj][r];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < WSTRIDE; idx += 256) {
      const int q = idx / 1024, r = (idx / 64) % 16, l = idx % 64;
      if (t0 + q < NT) {
        const int ti = (t0 + q) / Cf::RT, tj = (t0 + q) % Cf::RT;
        const float sum = ((red[idx] + red[WSTRIDE + idx]) + red[2 * WSTRIDE + idx]) +
                          red[3 * WSTRIDE + idx];
        const int d = 32 * ti + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        const int e = 32 * tj + (l & 31);
        dst[d * D + e] = sum;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Half-state kernel (D = 64, 128).
//
// A full D x D accumulator per wave allows one wave per SIMD at D = 128, and
// one wave alone leaves the SIMD idle while it waits on its own loads, LDS
// round trips and MFMA results.  Here a block has 8 waves in 4 pairs; both
// waves of pair p work on the pair's 16-token tiles p, p + 4, p + 8, ... and
// wave half hf accumulates rows [hf D/2, hf D/2 + D/2) of S (D = 128: 128
// accumulation registers, two waves per SIMD).  Each wave loads its half of
// the features of k and of v, so every byte is fetched once: ReLU, z and
// RoPE of its k half go to its own LDS tile (its A operand), its v half to
// the pair's shared v tile (both waves' B operand), and one barrier per
// step publishes the v tile.  The v tile alternates between two slots, so
// the writes of step i + 1 never meet the reads of step i.  With CH
// 16-byte chunks in a half row, lane l takes chunk l % CH of tile rows
// l / CH, l / CH + 64 / CH, ...: one load instruction covers 64 / CH whole
// half rows, which streams faster than sixteen partial rows.  Row pitches
// are 16 or 48 (mod 64) dwords: the four rows one 16-lane group of a
// transposing read touches then start 16 banks apart, and the two token rows
// eight lanes write together never share a bank.  At the block's end the
// four pairs' accumulators are added in pair order through LDS.
template <int D>
struct HalfCfg {
  static constexpr int HALF = D / 2;          // rows of S per wave
  static constexpr int CH = HALF / 8;         // 16-byte chunks in a half row
  static constexpr int TPI = 64 / CH;         // tokens per load instruction
  static constexpr int TW = 16;               // tokens per tile
  static constexpr int NI = TW / TPI;         // tokens per lane and tile (k and v each)
  static constexpr int RA = D / 64;           // 32-row blocks of a wave's S rows
  static constexpr int RB = D / 32;           // 32-column blocks
  static constexpr int KP = tile_pitch(HALF * 2);
  static constexpr int VP = tile_pitch(D * 2);
  static constexpr int KTILE = TW * KP;       // per wave
  static constexpr int VTILE = TW * VP;       // per pair and slot
  static constexpr int V_OFF = 8 * KTILE;
  static constexpr int TILE_BYTES = V_OFF + 4 * 2 * VTILE;
  static constexpr int PF = 2;                // tiles in flight per wave
  // block-end reduction: per round each wave stores RED 32x32 tiles (4 KB)
  static constexpr int NT = RA * RB;
  static constexpr int RED_FIT = TILE_BYTES / (8 * 4096);
  static constexpr int RED = RED_FIT < 1 ? 1 : (RED_FIT > NT ? NT : RED_FIT);
  static constexpr int ZW_OFF = 8 * RED * 4096;
  static constexpr int LDS_BYTES = TILE_BYTES > ZW_OFF + 16 * D ? TILE_BYTES : ZW_OFF + 16 * D;
  static_assert(CH >= 4 && NI >= 1 && RA >= 1, "half-state layout needs D >= 64");
};

template <int D, bool ROPE, int HF>
struct HalfWave {
  using Cf = HalfCfg<D>;
  static constexpr int NI = Cf::NI, RA = Cf::RA, RB = Cf::RB, PF = Cf::PF, TPI = Cf::TPI;
  const KArgs& a;
  const TabView& tv;
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t tokstride, hoff;
  int n_begin, n_end, pair, nit, lane, cl, tl;
  unsigned char* kbuf;  // this wave's R phi(k) tile, TW rows of KP bytes
  unsigned char* vbuf;  // the pair's two v tile slots, TW rows of VP bytes each
  u32x4 kr[PF][NI], vr[PF][NI];
  bf16x8 A[RA], Bv[RB];
  float2 cs[NI][4];
  float zacc[8];
  f32x16 acc[RA][RB];

  // token of the lane's i-th row in tile `it`
  __device__ __forceinline__ int token(int it, int i) const {
    return n_begin + Cf::TW * (pair + 4 * it) + TPI * i + tl;
  }

  __device__ __forceinline__ void issue(int st, int it) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = token(it, i);
      const uint32_t off = (it < nit && n < n_end) ? (uint32_t)n * tokstride + hoff : kOob;
      kr[st][i] = load16_nt(rk, off);
      vr[st][i] = load16_nt(rv, off);
    }
  }

  // (cos, sin) of the lane's 4 pairs for each of its tokens in tile `it`:
  // chunk cl of this half is chunk CH HF + cl of the row
  __device__ __forceinline__ void load_factors(int it) {
    if (!ROPE) return;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int t, y, x;
      grid_pos(a, (uint32_t)min(token(it, i), n_end - 1), t, y, x);
      const RowOff ro = row_offsets<D>(a, tv, t, y, x);
      static_for<4>([&](auto U) {
        constexpr int u = decltype(U)::value;
        constexpr int pmin = 4 * Cf::CH * HF + u;
        cs[i][u] = rope_factor<D, pmin, pmin + 4 * (Cf::CH - 1)>(tv, ro, pmin + 4 * cl);
      });
    }
  }

  template <int ST>
  __device__ __forceinline__ void stage(int it) {
    asm volatile("" ::: "memory");
    unsigned char* vt = vbuf + ST * Cf::VTILE + Cf::HALF * 2 * HF + 16 * cl;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      u32x4 fq;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        fq[u] = relu2(kr[ST][i][u]);
        zacc[2 * u] += bf_lo(fq[u]);
        zacc[2 * u + 1] += bf_hi(fq[u]);
      }
      const u32x4 w = ROPE ? rotate_chunk(fq, cs[i]) : fq;
      const int row = TPI * i + tl;
      *reinterpret_cast<u32x4*>(kbuf + row * Cf::KP + 16 * cl) = w;
      *reinterpret_cast<u32x4*>(vt + row * Cf::VP) = vr[ST][i];
    }
    issue(ST, it + PF);
  }

  // After the barrier: the wave's own k tile (the LDS executes one wave's
  // instructions in order, so its own writes need no wait) and the pair's v
  // slot ST.
  template <int ST>
  __device__ __forceinline__ void contract() {
#pragma unroll
    for (int i = 0; i < RA; ++i) A[i] = frag_tr(kbuf, Cf::KP, i, lane);
#pragma unroll
    for (int j = 0; j < RB; ++j) Bv[j] = frag_tr(vbuf + ST * Cf::VTILE, Cf::VP, j, lane);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < RA; ++i)
#pragma unroll
      for (int j = 0; j < RB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], Bv[j], acc[i][j], 0, 0, 0);
  }

  // Every wave's LDS writes of this step are complete before any wave passes
  // (no wait on the global loads in flight).
  __device__ __forceinline__ void publish() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // Steps are kept apart in the schedule: overlapping one step's factor
  // reads with the previous step's operands would overflow the register
  // budget of two waves per SIMD, and a spill reload (a memory load like the
  // prefetches) would make the loop wait for every load in flight.
  template <int ST>
  __device__ __forceinline__ void step(int it) {
    __builtin_amdgcn_sched_barrier(0);
    load_factors(it);
    stage<ST>(it);
    publish();
    contract<ST>();
  }

  // nsteps: the block's common step count (even, >= every pair's tiles);
  // steps past a pair's last tile load and add zeros
  __device__ __forceinline__ void run(int nsteps) {
#pragma unroll
    for (int i = 0; i < RA; ++i)
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) zacc[j] = 0.f;
    static_assert(PF == 2, "the load ring and the v slots alternate together");
    // Loads return in issue order and the loop waits for slot 0 while slot 1
    // is still in flight; the entry must issue the slots in the same order as
    // the loop body, or the wait at the loop head becomes a wait for all.
    issue(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int it = 0; it < nsteps; it += 2) {
      step<0>(it);
      step<1>(it + 1);
    }
  }
};

// Runs one half's waves and the block-end reduction.  Both halves execute the
// same sequence of barriers.
template <int D, bool ROPE, int HF>
__device__ __forceinline__ void half_main(const KArgs& a, const TabView& tv, unsigned char* smem,
                                          int tid, int wave, int pair, int lane, int b, int h,
                                          int bh, int c, int n_begin, int n_end) {
  using Cf = HalfCfg<D>;
  const int cl = lane % Cf::CH, tl = lane / Cf::CH;
  const size_t boff = (size_t)b * a.N * a.H * D;
  const int ntile = (n_end - n_begin + Cf::TW - 1) / Cf::TW;
  const int nsteps = 2 * ((ntile + 7) / 8);  // pair 0's tiles, rounded up to even
  HalfWave<D, ROPE, HF> w{a,
                          tv,
                          make_rsrc(a.k + boff, a.slab_bytes),
                          make_rsrc(a.v + boff, a.slab_bytes),
                          (uint32_t)a.H * D * 2,
                          (uint32_t)h * D * 2 + (uint32_t)(Cf::HALF * 2 * HF) + 16u * cl,
                          n_begin,
                          n_end,
                          pair,
                          (ntile - pair + 3) / 4,
                          lane,
                          cl,
                          tl,
                          smem + wave * Cf::KTILE,
                          smem + Cf::V_OFF + pair * 2 * Cf::VTILE};
  w.run(nsteps);

  // z of this wave: lanes with the same l % CH hold the same features
#pragma unroll
  for (int msk = Cf::CH; msk < 64; msk *= 2)
#pragma unroll
    for (int j = 0; j < 8; ++j) w.zacc[j] += __shfl_xor(w.zacc[j], msk);

  __syncthreads();  // every wave is done with its tiles; they become scratch
  float* red = reinterpret_cast<float*>(smem);
  float* dst = a.part + ((size_t)bh * a.C + c) * (size_t)(D * D + D);
  float* zw = reinterpret_cast<float*>(smem + Cf::ZW_OFF);
  if (tl == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) zw[pair * D + Cf::HALF * HF + 8 * cl + j] = w.zacc[j];
  }
  __syncthreads();
  if (tid < D) dst[D * D + tid] = ((zw[tid] + zw[D + tid]) + zw[2 * D + tid]) + zw[3 * D + tid];

  // S: add the four pairs' accumulators, RED 32x32 tiles per wave per round
  constexpr int WSTRIDE = Cf::RED * 1024;  // floats per wave per round
#pragma unroll
  for (int t0 = 0; t0 < Cf::NT; t0 += Cf::RED) {
#pragma unroll
    for (int q = 0; q < Cf::RED; ++q) {
      if (t0 + q < Cf::NT) {
        const int ti = (t0 + q) / Cf::RB, tj = (t0 + q) % Cf::RB;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          red[wave * WSTRIDE + (q * 16 + r) * 64 + lane] = w.acc[ti][tj][r];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < 2 * WSTRIDE; idx += 512) {
      const int hf = idx / WSTRIDE, rem = idx - hf * WSTRIDE;
      const int q = rem / 1024, r = (rem / 64) % 16, l = rem % 64;
      if (t0 + q < Cf::NT) {
        const int ti = (t0 + q) / Cf::RB, tj = (t0 + q) % Cf::RB;
        const float* src = red + 4 * hf * WSTRIDE + rem;
        const float sum = ((src[0] + src[WSTRIDE]) + src[2 * WSTRIDE]) + src[3 * WSTRIDE];
        const int d = Cf::HALF * hf + 32 * ti + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        const int e = 32 * tj + (l & 31);
        dst[d * D + e] = sum;
      }
    }
    __syncthreads();
  }
}

template <int D, bool ROPE, bool TLDS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void state_half_kernel(KArgs a) {
  using Cf = HalfCfg<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float2* ltab = reinterpret_cast<float2*>(smem + Cf::LDS_BYTES);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int pair = wave & 3, hf = wave >> 2;
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  int n_begin, n_end;
  range_of(a, c, n_begin, n_end);

  TabView tv{};
  if (ROPE) tv = stage_table<D, 512>(a, ltab, TLDS, n_begin, n_end);
  __syncthreads();
  if (hf == 0)
    half_main<D, ROPE, 0>(a, tv, smem, tid, wave, pair, lane, b, h, bh, c, n_begin, n_end);
  else
    half_main<D, ROPE, 1>(a, tv, smem, tid, wave, pair, lane, b, h, bh, c, n_begin, n_end);
}

// ---------------------------------------------------------------------------
// Reduce kernel: per head and attention block b, the state up to the end of
// block b: S_<=b = S_in + sum over chunks c of blocks <= b of S_c (likewise
// z), accumulated block after block (for the bidirectional mixer: one block,
// no carried state, S = sum_c S_c).  A block takes a tile of S (16 rows x 64
// columns at D = 128);
// each thread loads, for its 4 consecutive columns e of a row d, the P (a power of two
// >= C, at most 32) chunk values at once -- loads past the head's C partials
// fall outside the buffer and read as zero -- and adds them in a fixed
// pairwise tree, so the result does not depend on which block finished
// first.  More than 32 chunks are summed 32 at a time, groups in order.  The
// tile is transposed through LDS so the bf16 operand rows go out in 16-byte
// runs.  The first tile's block also reduces z.
// Outputs per head and attention block, in the output kernel's operand
// layout (D + 2 rows of D bf16): row R(e) holds S_<=b[0..D)[e] (see
// out_row_of); row D holds bf16(z), row D + 1 holds bf16(z - bf16(z)).
// Optionally also the row-major operand (D rows: row R(d) holds S[d][0..D),
// which the backward pass contracts over the value index).  The fp32 state
// after the last block optionally goes to the caller.

// Output-kernel operand row of value column e: with MB = D/16 column blocks,
// row 16 j + c holds column MB c + j, so that lane column c of block j owns
// the MB contiguous columns MB c .. MB c + MB - 1 across the blocks.
template <int D>
__device__ __forceinline__ int out_row_of(int e) {
  constexpr int MB = D / 16;
  return 16 * (e % MB) + e / MB;
}

// Fixed-order sum over chunks of R 16-byte vectors at off0 + r * rstride.
template <int P, int R>
__device__ __forceinline__ void tree_sum4(__amdgpu_buffer_rsrc_t rs, uint32_t off0,
                                          uint32_t cstride, uint32_t rstride, int C,
                                          f32x4 (&out)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) out[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < C; g0 += P) {
    f32x4 x[R][P];
#pragma unroll
    for (int cc = 0; cc < P; ++cc)
#pragma unroll
      for (int r = 0; r < R; ++r)
        x[r][cc] = __builtin_bit_cast(
            f32x4, load16(rs, off0 + (uint32_t)(g0 + cc) * cstride + r * rstride));
#pragma unroll
    for (int w = P / 2; w >= 1; w /= 2)
#pragma unroll
      for (int cc = 0; cc < w; ++cc)
#pragma unroll
        for (int r = 0; r < R; ++r) x[r][cc] = x[r][2 * cc] + x[r][2 * cc + 1];
#pragma unroll
    for (int r = 0; r < R; ++r) out[r] = (g0 == 0) ? x[r][0] : out[r] + x[r][0];
  }
}

// The P chunk vectors of one column group (loads past the window read zero).
template <int P>
__device__ __forceinline__ void load_chunks(__amdgpu_buffer_rsrc_t rs, uint32_t off0,
                                            uint32_t cstride, f32x4 (&x)[P]) {
#pragma unroll
  for (int cc = 0; cc < P; ++cc)
    x[cc] = __builtin_bit_cast(f32x4, load16(rs, off0 + (uint32_t)cc * cstride));
}

// Their fixed pairwise tree sum (the same order tree_sum4 uses for one group).
template <int P>
__device__ __forceinline__ f32x4 sum_chunks(f32x4 (&x)[P]) {
#pragma unroll
  for (int w = P / 2; w >= 1; w /= 2)
#pragma unroll
    for (int cc = 0; cc < w; ++cc) x[cc] = x[2 * cc] + x[2 * cc + 1];
  return x[0];
}

template <int D>
struct RedCfg {
  static constexpr int TE = D < 64 ? D : 64;   // tile columns (e)
  static constexpr int EQ = TE / 4;            // threads per tile row (4 columns each)
  static constexpr int TR = 256 / EQ < D ? 256 / EQ : D;  // tile rows (d), one per thread group
  static constexpr int NTE = D / TE;           // tiles across e
  static constexpr int NTILE = NTE * (D / TR); // tiles per head
  static constexpr int TP = TR + 1;            // LDS pitch (floats) of the transposed tile
  static_assert(EQ * TR == 256 && TR % 8 == 0, "one tile element group per thread");
};

template <int D, int P>
__global__ __launch_bounds__(256) void reduce_kernel(KArgs a) {
  using Rc = RedCfg<D>;
  __shared__ float tile[Rc::TE * Rc::TP];     // [e][d]
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int d0 = Rc::TR * (blockIdx.x / Rc::NTE), e0 = Rc::TE * (blockIdx.x % Rc::NTE);
  const uint32_t pstride = (uint32_t)(D * D + D) * 4u;  // bytes per chunk partial
  // attention block blk's chunks: blk * CB .. blk * CB + CB - 1; loads past the
  // block's last chunk must read zero, so each block gets its own window
  const uint32_t bstride = (uint32_t)a.CB * pstride;

  // row d0 + t / EQ, columns e0 + 4 (t % EQ) .. + 3
  const int dl = t / Rc::EQ, el = 4 * (t % Rc::EQ);
  const size_t sidx = (size_t)bh * D * D + (size_t)(d0 + dl) * D + e0 + el;
  f32x4 acc = a.S_in ? *reinterpret_cast<const f32x4*>(a.S_in + sidx) : f32x4{0.f, 0.f, 0.f, 0.f};
  const bool zt = blockIdx.x == 0 && t < D / 4;  // threads that also carry z
  f32x4 zacc = (zt && a.z_in) ? *reinterpret_cast<const f32x4*>(a.z_in + (size_t)bh * D + 4 * t)
                              : f32x4{0.f, 0.f, 0.f, 0.f};

  // Block blk + 1's partials are loaded while block blk is summed, written
  // and transposed (when a block has at most PF_MAX chunks: one group).
  constexpr int PF_MAX = 16;
  auto window = [&](int blk) {
    return make_rsrc(reinterpret_cast<const char*>(a.part + ((size_t)bh * a.C +
                                                             (size_t)blk * a.CB) * (D * D + D)),
                     bstride);
  };
  const uint32_t soff = (uint32_t)((d0 + dl) * D + e0 + el) * 4u;
  const uint32_t zoff = (uint32_t)(D * D + 4 * t) * 4u;
  f32x4 xs[P <= PF_MAX ? P : 1], xz[P <= PF_MAX ? P : 1];
  if constexpr (P <= PF_MAX) {
    if (a.NB > 0) {
      load_chunks<P>(window(0), soff, pstride, xs);
      if (zt) load_chunks<P>(window(0), zoff, pstride, xz);
    }
  }
  for (int blk = 0; blk < a.NB; ++blk) {
    f32x4 s_blk, z_blk = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (P <= PF_MAX) {
      s_blk = sum_chunks<P>(xs);
      if (zt) z_blk = sum_chunks<P>(xz);
      if (blk + 1 < a.NB) {
        load_chunks<P>(window(blk + 1), soff, pstride, xs);
        if (zt) load_chunks<P>(window(blk + 1), zoff, pstride, xz);
      }
    } else {
      f32x4 s4[1];
      tree_sum4<P, 1>(window(blk), soff, pstride, 0u, a.CB, s4);
      s_blk = s4[0];
      if (zt) {
        tree_sum4<P, 1>(window(blk), zoff, pstride, 0u, a.CB, s4);
        z_blk = s4[0];
      }
    }
    acc = acc + s_blk;
    if (a.sl2) {
      // the row-major operand: row R(d) holds S[d][0..D), 4 columns per thread
      typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
      uint16_t* r2 = a.sl2 + ((size_t)bh * a.NB + blk) * D * D;
      *reinterpret_cast<u32x2v*>(r2 + (size_t)out_row_of<D>(d0 + dl) * D + e0 + el) =
          u32x2v{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) tile[(el + k) * Rc::TP + dl] = acc[k];
    __syncthreads();
    // operand rows: for each tile column e, TR values over d in runs of 8 (16 bytes)
    uint16_t* slh = a.sl + ((size_t)bh * a.NB + blk) * (D + 2) * D;
    for (int item = t; item < Rc::TE * (Rc::TR / 8); item += 256) {
      const int e = item / (Rc::TR / 8), dc = 8 * (item % (Rc::TR / 8));
      const float* src = tile + e * Rc::TP + dc;
      u32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = pack_bf16(src[2 * k], src[2 * k + 1]);
      *reinterpret_cast<u32x4*>(slh + (size_t)out_row_of<D>(e0 + e) * D + d0 + dc) = w;
    }
    if (zt) {
      zacc = zacc + z_blk;
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const __bf16 h0 = (__bf16)zacc[2 * k], h1 = (__bf16)zacc[2 * k + 1];
        const __bf16 l0 = (__bf16)(zacc[2 * k] - (float)h0);
        const __bf16 l1 = (__bf16)(zacc[2 * k + 1] - (float)h1);
        hi[k] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        lo[k] = (uint32_t)__builtin_bit_cast(uint16_t, l0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
      typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2v*>(slh + (size_t)D * D + 4 * t) = u32x2v{hi[0], hi[1]};
      *reinterpret_cast<u32x2v*>(slh + (size_t)(D + 1) * D + 4 * t) = u32x2v{lo[0], lo[1]};
    }
    __syncthreads();  // the tile is rewritten by the next block
  }
  // the state after the last block (each element is read above and written
  // here by the same thread, so S_out may be S_in)
  if (a.S_out) *reinterpret_cast<f32x4*>(a.S_out + sidx) = acc;
  if (zt && a.z_out) *reinterpret_cast<f32x4*>(a.z_out + (size_t)bh * D + 4 * t) = zacc;
}

// ---------------------------------------------------------------------------
// Output kernel.
//
// Block = 256 threads (4 waves), one (token range, head).  The head's S^T
// (bf16, D rows of D) and the two z rows are staged in LDS once per block,
// as a swizzled row tile (row_tile_offset).  Each wave computes 16 tokens per step as
// num = (R phi(q)) S on v_mfma_f32_16x16x32_bf16 with the tokens as the A
// operand: lane l holds token l % 16 and, for k-step s, features
// 32 s + 8 (l / 16) .. + 7 of it (one 16-byte global load).  The B operand
// of column block j is LDS row 16 j + c for lane column c, which holds value
// column MB c + j (MB = D / 16 blocks).  The accumulator of block j then
// holds, in lane l, tokens 4 (l / 16) + i (i < 4) at value column
// MB (l % 16) + j: across the MB blocks a lane owns MB contiguous columns of
// four tokens (16 bytes at D = 128).  g is read and out written in that
// layout, so one instruction covers four whole token rows.  The denominator
// phi(q).z uses the unrotated features, exact in bf16, against B columns
// that alternate bf16(z) and bf16(z - bf16(z)); adding the neighbouring
// lane's value gives phi(q).z in fp32 for the same four tokens.
template <int D, bool ROPE, bool TLDS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8)))
void output_kernel(KArgs a) {
  constexpr int KS = D / 32;       // k-steps of 32 features
  constexpr int MB = D / 16;       // 16-column blocks of the value dimension
  constexpr int OB = 2 * MB;       // output bytes per lane and token
  constexpr int OW = OB / 4;       // ... in dwords
  constexpr int ROWS = D + 2;
  using OChunk = typename Chunk<OB>::T;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* sS = smem;
  float2* ltab = reinterpret_cast<float2*>(smem + ROWS * 2 * D);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int m = lane >> 4;
  const int col = lane & 15;
  // heads vary fastest over the grid: the blocks resident at once cover every
  // head of a few token ranges (whole token rows are read together), and with
  // a head count divisible by the 8 XCDs each head's blocks share one L2
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  int n_begin, n_end;
  range_of(a, blockIdx.y, n_begin, n_end);
  const int blk = blockIdx.y / a.CB;  // attention block of the range
  TabView tv{};                       // the RoPE table view, set when staged

  const size_t boff = (size_t)b * a.N * a.H * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + boff, a.slab_bytes);
  const uint32_t tokstride = (uint32_t)a.H * D * 2;
  const uint32_t qoff = (uint32_t)h * D * 2 + 16u * m;     // A operand chunk of q
  const uint32_t goff = (uint32_t)h * D * 2 + (uint32_t)OB * col;  // owned output columns

  // q: token base + col; g and out: token base + 4 m + i
  auto q_offset = [&](int base) -> uint32_t {
    const int n = base + col;
    return (n < n_end) ? (uint32_t)n * tokstride + qoff : kOob;
  };
  auto g_offset = [&](int base, int i) -> uint32_t {
    const int n = base + 4 * m + i;
    return (n < n_end) ? (uint32_t)n * tokstride + goff : kOob;
  };
  auto load_qg = [&](int base, u32x4 (&qv)[KS], OChunk (&gv)[4]) {
    const uint32_t toff = q_offset(base);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) qv[s2] = load16(rq, toff + 64u * s2);
#pragma unroll
    for (int i = 0; i < 4; ++i) gv[i] = load_chunk_nt<OB>(rg, g_offset(base, i));
  };

  // one 16-token step of this wave: tokens base .. base + 15
  auto step = [&](int base, const u32x4 (&qv)[KS], const OChunk (&gv)[4]) {
    // the S fragments stay in LDS: reading them in the loop costs LDS
    // bandwidth but leaves registers for more waves in flight
    asm volatile("" ::: "memory");
    RowOff rof{};
    if (ROPE) {
      int t, y, x;
      grid_pos(a, (uint32_t)min(base + col, n_end - 1), t, y, x);
      rof = row_offsets<D>(a, tv, t, y, x);
    }
    // phi(q) first, against z: phi(q).z_hi in even lane columns, phi(q).z_lo
    // in odd ones; the rotated operand is built afterwards from the same
    // registers, so the two copies are never live together
    u32x4 fq[KS];
    f32x4 accd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
#pragma unroll
      for (int u = 0; u < 4; ++u) fq[s2][u] = relu2(qv[s2][u]);
      const bf16x8 Bz = *reinterpret_cast<const bf16x8*>(
          sS + row_tile_offset<D>(D + (col & 1), 16 * (4 * s2 + m)));
      accd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fq[s2]), Bz, accd,
                                                    0, 0, 0);
    }
    bf16x8 Aq[KS];
    static_for<KS>([&](auto S2) {
      constexpr int s2 = decltype(S2)::value;
      Aq[s2] = __builtin_bit_cast(bf16x8, ROPE ? rope_chunk<D, s2>(fq[s2], tv, rof, m) : fq[s2]);
    });
    // S fragments of column block j + 1 are read while block j multiplies;
    // the fences keep the compiler from reading further ahead (each block
    // is KS fragments of 4 registers)
    f32x4 acc[MB];
    bf16x8 Bf[2][KS];
    auto read_b = [&](int j, bf16x8 (&dst)[KS]) {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        dst[s2] = *reinterpret_cast<const bf16x8*>(sS + row_tile_offset<D>(16 * j + col, 16 * (4 * s2 + m)));
    };
    read_b(0, Bf[0]);
    static_for<MB>([&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (j + 1 < MB) read_b(j + 1, Bf[(j + 1) & 1]);
      asm volatile("" ::: "memory");
      acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aq[s2], Bf[j & 1][s2], acc[j], 0, 0, 0);
    });

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // quad_perm [1, 0, 3, 2]: the neighbouring lane column's term
      const float other = __int_as_float(
          __builtin_amdgcn_mov_dpp(__float_as_int(accd[i]), 0xB1, 0xF, 0xF, false));
      const float den = (accd[i] + other) + kEps;
      OChunk ow;
#pragma unroll
      for (int w = 0; w < OW; ++w) {
        float o2[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int j = 2 * w + hlf;  // column block = element of the owned chunk
          const float gval = hlf ? bf_hi(gv[i][w]) : bf_lo(gv[i][w]);
          // sigmoid(g) / den = 1 / (den * (1 + exp(-g)))
          const float e = __expf(-gval);
          o2[hlf] = acc[j][i] * __builtin_amdgcn_rcpf(__builtin_fmaf(den, e, den));
        }
        ow[w] = pack_bf16(o2[0], o2[1]);
      }
      store_chunk_nt<OB>(ro, g_offset(base, i), ow);
    }
  };

  // two register sets: the next step's q and g are in flight during a step.
  // The first step's loads go out before the staging below, so the two wait
  // for memory together.
  u32x4 qa[KS], qb[KS];
  OChunk ga[4], gb[4];
  int base = n_begin + 16 * wave;
  if (base < n_end) load_qg(base, qa, ga);

  // stage the block's S^T rows and z rows
  {
    RowStage<D, D, 256> st_s;
    RowStage<D, 2, 256, D> st_z;
    const uint16_t* sl = a.sl + ((size_t)bh * a.NB + blk) * ROWS * D;
    st_s.load(sl);
    st_z.load(sl);
    if (ROPE) tv = stage_table<D>(a, ltab, TLDS, n_begin, n_end);
    st_s.store(sS);
    st_z.store(sS);
  }
  __syncthreads();

  for (; base < n_end; base += 128) {
    load_qg(base + 64, qb, gb);
    step(base, qa, ga);
    if (base + 64 >= n_end) break;
    load_qg(base + 128, qa, ga);
    step(base + 64, qb, gb);
  }
}

// ---------------------------------------------------------------------------
// Tile state kernel (D = 128).
//
// Block = 8 waves (512 threads), one (chunk, head), one block per compute
// unit.  A step takes 64 tokens.  Thread t loads chunk t % 16 of token rows
// t / 16 and t / 16 + 32 of k and of v (one load instruction covers four whole
// 256-byte rows), PF steps ahead in a register ring.  The thread applies
// ReLU, z and RoPE to its k chunks and writes R phi(k) and v token-major into
// one of two LDS tile buffers.  Each wave owns two of the sixteen 32 x 32
// blocks of S (row block w / 2, column blocks 2 (w % 2) and 2 (w % 2) + 1)
// and contracts a step's 64 tokens into them with four
// v_mfma_f32_32x32x16_bf16 k-steps, the operands read back transposed with
// ds_read_b64_tr_b16.  The contraction of step t - 1 runs in step t, after
// its operand reads and beside step t's ReLU and RoPE arithmetic, so the
// matrix unit and the vector ALU work at the same time; one LDS barrier per
// step both publishes step t's tiles and frees step t - 1's buffer.  No two
// waves share an accumulator, so the block writes its fp32 partial straight
// from the accumulators, with no cross-wave reduction.
struct TileCfg {
  static constexpr int D = 128;
  static constexpr int NT = 512;               // threads
  static constexpr int TT = 64;                // tokens per step
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPI = NT / CPR;         // rows one load instruction per thread covers
  static constexpr int LPT = TT / RPI;         // loads per thread, tensor and step
  static constexpr int P = tile_pitch(2 * D);  // LDS row pitch (bytes)
  static constexpr int TILE = TT * P;
  static constexpr int BUF = 2 * TILE;         // R phi(k) tile + v tile
  static constexpr int LDS_BYTES = 2 * BUF;    // two buffers
  static constexpr int RT = D / 32;
  static constexpr int TPW = RT * RT / 8;      // accumulator blocks per wave
  static constexpr int KSTEP = TT / 16;
  static constexpr int PF = 2;                 // steps of loads in flight
  static_assert(LPT == 2 && TPW == 2 && PF % 2 == 0, "tile state layout");
};

template <bool ROPE, bool TLDS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void state_tile_kernel(KArgs a) {
  using Cf = TileCfg;
  constexpr int D = Cf::D, LPT = Cf::LPT, TPW = Cf::TPW, P = Cf::P, PF = Cf::PF;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float2* ltab = reinterpret_cast<float2*>(smem + Cf::LDS_BYTES);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  int n_begin, n_end;
  range_of(a, c, n_begin, n_end);

  TabView tv{};  // the RoPE table view, set once staged (after the first loads)
  const size_t boff = (size_t)b * a.N * a.H * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + boff, a.slab_bytes);
  const uint32_t tokstride = (uint32_t)a.H * D * 2;
  const int cc = tid % Cf::CPR, r0 = tid / Cf::CPR;
  const uint32_t hoff = (uint32_t)h * D * 2 + 16u * cc;
  const int ntile = (n_end - n_begin + Cf::TT - 1) / Cf::TT;
  const int nsteps = (ntile + PF - 1) / PF * PF;
  // axis block of each of the thread's four rotation pairs 4 cc + u (the
  // thread's chunk never changes)
  using X = Axes<D>;
  bool in_y[4], in_x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = 4 * cc + u;
    in_y[u] = p >= X::Pt && p < X::Pt + X::Py;
    in_x[u] = p >= X::Pt + X::Py;
  }

  // grid positions of the thread's rows in the tile being transformed
  GridWalk gw[LPT];
  if (ROPE) {
#pragma unroll
    for (int j = 0; j < LPT; ++j)
      gw[j].init(a, (uint32_t)min(n_begin + r0 + Cf::RPI * j, a.N - 1), (uint32_t)Cf::TT);
  }

  u32x4 kr[PF][LPT], vr[PF][LPT];
  f32x16 acc[TPW];
  float zacc[8];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) zacc[j] = 0.f;

  auto issue = [&](auto S, int t) {
    constexpr int s = decltype(S)::value;
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int n = n_begin + Cf::TT * t + r0 + Cf::RPI * j;
      const uint32_t off = n < n_end ? (uint32_t)n * tokstride + hoff : kOob;
      kr[s][j] = load16_nt(rk, off);
      vr[s][j] = load16_nt(rv, off);
    }
  };
  // ReLU, z and RoPE of the tile in ring slot s, into LDS buffer s % 2
  auto transform = [&](auto S, int t) {
    constexpr int s = decltype(S)::value;
    unsigned char* kt = smem + (s % 2) * Cf::BUF;
    unsigned char* vt = kt + Cf::TILE;
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int row = r0 + Cf::RPI * j;
      u32x4 fq;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        fq[u] = relu2(kr[s][j][u]);
        zacc[2 * u] += bf_lo(fq[u]);
        zacc[2 * u + 1] += bf_hi(fq[u]);
      }
      u32x4 w = fq;
      if (ROPE) {
        const RowOff ro = row_offsets<D>(a, tv, gw[j].t, gw[j].y, gw[j].x);
        gw[j].advance(a);
        float2 cs[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int base = in_x[u] ? ro.ox : (in_y[u] ? ro.oy : ro.ot);
          cs[u] = tv.tab[base + 4 * cc + u];
        }
        w = rotate_chunk(fq, cs);
      }
      *reinterpret_cast<u32x4*>(kt + row * P + 16 * cc) = w;
      *reinterpret_cast<u32x4*>(vt + row * P + 16 * cc) = vr[s][j];
    }
  };
  // operands of the tile in LDS buffer B, then its MFMAs
  const int ti = wave >> 1, tj = 2 * (wave & 1);
  auto read_ops = [&](int B, bf16x8 (&A)[Cf::KSTEP], bf16x8 (&Bv)[Cf::KSTEP][TPW]) {
    const unsigned char* kt = smem + B * Cf::BUF;
    const unsigned char* vt = kt + Cf::TILE;
#pragma unroll
    for (int ks = 0; ks < Cf::KSTEP; ++ks) {
      A[ks] = frag_tr(kt + 16 * ks * P, P, ti, lane);
#pragma unroll
      for (int u = 0; u < TPW; ++u) Bv[ks][u] = frag_tr(vt + 16 * ks * P, P, tj + u, lane);
    }
  };
  auto contract = [&](const bf16x8 (&A)[Cf::KSTEP], const bf16x8 (&Bv)[Cf::KSTEP][TPW]) {
#pragma unroll
    for (int ks = 0; ks < Cf::KSTEP; ++ks)
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ks], Bv[ks][u], acc[u], 0, 0, 0);
  };

  // Loads return in issue order and a step waits for its own slot while the
  // later slots are in flight; the entry issues the slots in the loop's order,
  // before the table staging, so the two wait for memory together.
  static_for<PF>([&](auto S) {
    issue(S, decltype(S)::value);
    __builtin_amdgcn_sched_barrier(0);
  });
  if (ROPE) tv = stage_table<D, 512>(a, ltab, TLDS, n_begin, n_end);
  __syncthreads();
  for (int it = 0; it < nsteps; it += PF) {
    static_for<PF>([&](auto S) {
      constexpr int s = decltype(S)::value;
      const int t = it + s;
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 A[Cf::KSTEP], Bv[Cf::KSTEP][TPW];
      const bool prev = t > 0;  // uniform
      if (prev) read_ops(1 - s % 2, A, Bv);
      transform(S, t);
      if (prev) contract(A, Bv);
      issue(S, t + PF);
      // every wave's tile writes of this step are done, and every wave is
      // done reading the other buffer (no wait on the loads in flight)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    });
  }
  if (nsteps > 0) {
    bf16x8 A[Cf::KSTEP], Bv[Cf::KSTEP][TPW];
    read_ops(1, A, Bv);  // nsteps is even: the last tile sits in buffer 1
    contract(A, Bv);
  }

  // z: lanes l, l + 16, l + 32, l + 48 hold the same features; then the
  // eight waves in wave order through LDS (buffer 0, which no wave reads now)
#pragma unroll
  for (int msk = Cf::CPR; msk < 64; msk *= 2)
#pragma unroll
    for (int j = 0; j < 8; ++j) zacc[j] += __shfl_xor(zacc[j], msk);
  float* zw = reinterpret_cast<float*>(smem);
  if (lane < Cf::CPR) {
#pragma unroll
    for (int j = 0; j < 8; ++j) zw[wave * D + 8 * cc + j] = zacc[j];
  }
  __syncthreads();
  // The partial goes out with agent-scope stores, written through the L2:
  // nothing is left dirty there for the end of the kernel to write back
  // before the reduce kernel can start (5B 480p/81f: state half 21.4 ->
  // 20.7 us; the same at the longer shapes).
  float* dst = a.part + ((size_t)bh * a.C + c) * (size_t)(D * D + D);
  if (tid < D) {
    float z = zw[tid];
#pragma unroll
    for (int w = 1; w < 8; ++w) z += zw[w * D + tid];
    __hip_atomic_store(dst + D * D + tid, z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * ti + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int e = 32 * (tj + u) + (lane & 31);
      __hip_atomic_store(dst + d * D + e, acc[u][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent output kernel (one attention block per head: the bidirectional
// mixer).  Block = 4 waves (256 threads), one per compute unit: the launch
// asks for enough LDS that two blocks never share a compute unit.  A block
// serves G consecutive heads of one batch element (G = 1, 2 or 4): it keeps
// their S operands (and the whole RoPE table when it fits: fp32 pairs, or
// fp16 pairs beside several operands) in LDS for its whole life and walks
// the group's (64 / G)-token ranges s, s + NS, s + 2 NS, ... (NS blocks per
// group); wave w takes head G g + w % G and tokens 16 (w / G) .. + 15 of each
// range.  The blocks of all groups then read and write a compact window of
// the sequence at any time, in runs of G heads' whole rows per token, which
// measured faster than the per-range blocks of output_kernel (that restage
// S for every range), than long contiguous ranges per block, and (G = 4)
// than one head's rows.  A step is output_kernel's step (same arithmetic,
// same result).  At D <= 64 the block can instead take its head's operand
// from the chunk partials, or form the head's whole state itself first
// (the SRC template argument), so that short passes need fewer launches.
//
// Where a block's state operand comes from (the SRC template argument).
constexpr int kSrcReduced = 0;   // the reduce kernel's operand rows (a.sl)
constexpr int kSrcPartials = 1;  // the head's chunk partials, summed here
constexpr int kSrcInBlock = 2;   // the head's state, formed here from all N tokens

// Register budget: the RoPE forms allocate about 220 VGPRs either way, and
// keep the allocation of a one-wave-per-SIMD target.  Without RoPE that
// target let the grouped kernels grow past 256 and shuttle values through
// the accumulation registers (about 8% slower); the two-wave target keeps
// them in 256.
template <int D, bool ROPE, bool TLDS, int G, bool T16, bool QROWS, int SRC = kSrcReduced>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ROPE ? 1 : 2, 2)))
void output_persist_kernel(KArgs a, int nsub) {
  // QROWS: whole-row q loads (four rows of 16 chunks) through a per-wave LDS
  // tile (D = 128)
  static_assert(!QROWS || D == 128, "whole-row q tiles");
  constexpr int QT = 16 * 2 * D;    // per-wave q tile in LDS
  constexpr int KS = D / 32;
  constexpr int MB = D / 16;
  constexpr int OB = 2 * MB;
  constexpr int OW = OB / 4;
  constexpr int ROWS = D + 2;
  constexpr int OPB = ROWS * 2 * D;  // one head's S operand and z rows
  constexpr int RANGE = 64 / G;      // tokens of a head per block and step
  static_assert(G == 1 || ((G == 2 || G == 4) && D == 128), "heads per block");
  static_assert(!T16 || (TLDS && G > 1), "fp16 pairs only in a grouped block's LDS table");
  static_assert(SRC == kSrcReduced || (G == 1 && !QROWS && D <= 64),
                "partials or the state are summed by one-head blocks (D <= 64)");
  using OChunk = typename Chunk<OB>::T;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane >> 4;
  const int col = lane & 15;
  unsigned char* sS = smem + (wave % G) * OPB;
  unsigned char* myq = smem + G * OPB + wave * QT;
  // kSrcInBlock: the state kernel's tiles and reduction scratch follow the
  // operand
  constexpr int SCR = SRC == kSrcInBlock ? StateCfg<D>::LDS_BYTES : 0;
  float2* ltab = reinterpret_cast<float2*>(smem + G * OPB + (QROWS ? 4 * QT : 0) + SCR);
  // grid (head group, range, batch element): wave w takes head G g + w % G,
  // and tokens 16 (w / G) .. of each range.  (A batch index divided out of
  // one grid dimension can land in vector registers; the compiler then
  // wraps buffer loads in loops over the lanes.)
  const int b = blockIdx.z;
  const int h = (int)blockIdx.x * G + wave % G;
  const int bh = b * a.H + h;
  // attention block ab of the block-causal form: grid.y = NB x nsub, and the
  // block walks only ab's tokens [n0, N) with ab's state operand.  The
  // bidirectional mixer is one attention block: ab = 0, tokens [0, a.N).
  const int ab = __builtin_amdgcn_readfirstlane((int)blockIdx.y / nsub);
  const int s = (int)blockIdx.y - ab * nsub;
  const int n0 = ab * a.BT;
  const int N = min(n0 + a.BT, a.N);  // end of the block's window
  const int bhb = bh * a.NB + ab;     // (head, attention block) operand
  TabView tv{};

  const size_t boff = (size_t)b * a.N * a.H * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + boff, a.slab_bytes);
  const uint32_t tokstride = (uint32_t)a.H * D * 2;
  const uint32_t qoff = (uint32_t)h * D * 2 + 16u * m;
  const uint32_t goff = (uint32_t)h * D * 2 + (uint32_t)OB * col;

  auto g_offset = [&](int base, int i) -> uint32_t {
    const int n = base + 4 * m + i;
    return (n < N) ? (uint32_t)n * tokstride + goff : kOob;
  };
  // QROWS: qv[i] holds chunk col of token base + 4 i + m (four whole rows per
  // load instruction); the step turns them into the operand layout through the
  // wave's LDS tile.  Otherwise qv[s2] is chunk 4 s2 + m of token base + col.
  auto load_qg = [&](int base, u32x4 (&qv)[KS], OChunk (&gv)[4]) {
    if constexpr (QROWS) {
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const int n = base + 4 * i + m;
        qv[i] = load16(rq, n < N ? (uint32_t)n * tokstride + (uint32_t)h * D * 2 + 16u * col : kOob);
      }
    } else {
      const int n = base + col;
      const uint32_t toff = (n < N) ? (uint32_t)n * tokstride + qoff : kOob;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) qv[s2] = load16(rq, toff + 64u * s2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) gv[i] = load_chunk_nt<OB>(rg, g_offset(base, i));
  };

  GridWalk gw;  // grid position of the lane's token (base + col) in the next step
  auto step = [&](int base, const u32x4 (&qv)[KS], const OChunk (&gv)[4]) {
    asm volatile("" ::: "memory");
    RowOff rof{};
    if (ROPE) {
      rof = row_offsets<D>(a, tv, gw.t, gw.y, gw.x);
      gw.advance(a);
    }
    u32x4 fq[KS];
    if constexpr (QROWS) {
      // the wave's own tile: its LDS instructions execute in order, so the
      // reads see the writes and the next step's writes follow these reads
#pragma unroll
      for (int i = 0; i < KS; ++i)
        *reinterpret_cast<u32x4*>(myq + row_tile_offset<D>(4 * i + m, 16 * col)) = qv[i];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        fq[s2] = *reinterpret_cast<const u32x4*>(myq + row_tile_offset<D>(col, 16 * (4 * s2 + m)));
    } else {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) fq[s2] = qv[s2];
    }
    f32x4 accd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
#pragma unroll
      for (int u = 0; u < 4; ++u) fq[s2][u] = relu2(fq[s2][u]);
      const bf16x8 Bz = *reinterpret_cast<const bf16x8*>(
          sS + row_tile_offset<D>(D + (col & 1), 16 * (4 * s2 + m)));
      accd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fq[s2]), Bz, accd,
                                                    0, 0, 0);
    }
    bf16x8 Aq[KS];
    static_for<KS>([&](auto S2) {
      constexpr int s2 = decltype(S2)::value;
      Aq[s2] = __builtin_bit_cast(bf16x8, ROPE ? rope_chunk<D, s2, T16>(fq[s2], tv, rof, m) : fq[s2]);
    });
    f32x4 acc[MB];
    bf16x8 Bf[2][KS];
    auto read_b = [&](int j, bf16x8 (&dst)[KS]) {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        dst[s2] = *reinterpret_cast<const bf16x8*>(sS + row_tile_offset<D>(16 * j + col, 16 * (4 * s2 + m)));
    };
    read_b(0, Bf[0]);
    static_for<MB>([&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (j + 1 < MB) read_b(j + 1, Bf[(j + 1) & 1]);
      asm volatile("" ::: "memory");
      acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aq[s2], Bf[j & 1][s2], acc[j], 0, 0, 0);
    });
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float other = __int_as_float(
          __builtin_amdgcn_mov_dpp(__float_as_int(accd[i]), 0xB1, 0xF, 0xF, false));
      const float den = (accd[i] + other) + kEps;
      OChunk ow;
#pragma unroll
      for (int w = 0; w < OW; ++w) {
        float o2[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int j = 2 * w + hlf;
          const float gval = hlf ? bf_hi(gv[i][w]) : bf_lo(gv[i][w]);
          const float e = __expf(-gval);
          o2[hlf] = acc[j][i] * __builtin_amdgcn_rcpf(__builtin_fmaf(den, e, den));
        }
        ow[w] = pack_bf16(o2[0], o2[1]);
      }
      store_chunk_nt<OB>(ro, g_offset(base, i), ow);
    }
  };

  // the wave's steps: tokens RANGE r + 16 (wave / G) .. for ranges
  // r = s + k nsub
  const int stride = RANGE * nsub;
  int base = n0 + RANGE * s + 16 * (wave / G);
  if (ROPE) gw.init(a, (uint32_t)min(base + col, N - 1), (uint32_t)stride);
  u32x4 qa[KS], qb[KS];
  OChunk ga[4], gb[4];
  if (base < N) load_qg(base, qa, ga);
  if constexpr (G > 1) {
    // the waves of head slot w % G (4 / G of them) stage that head's operand
    // together: every chunk a lane copies is loaded before any is written
    // (33 chunks per lane at G = 4), and the table's loads are issued right
    // behind them, so the staging costs one memory round trip where chunks
    // issued eight at a time cost five
    constexpr int CH = ROWS * D / 8;            // 16-byte chunks of one operand
    constexpr int WPH = 4 / G;                  // waves per head
    constexpr int LPH = 64 * WPH;               // lanes per head
    constexpr int NCH = (CH + LPH - 1) / LPH;   // chunks per lane
    const int li = (wave / G) * 64 + lane;
    const __amdgpu_buffer_rsrc_t rsl =
        make_rsrc(a.sl + (size_t)bhb * ROWS * D, (uint32_t)CH * 16u);  // past CH: zero
    u32x4 v[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) v[k] = load16(rsl, (uint32_t)(k * LPH + li) * 16u);
    if (ROPE) {
      const int pairs = a.T * a.Pt + a.Hh * a.Py + a.W * a.Px;
      if (T16) {
        uint32_t* lt16 = reinterpret_cast<uint32_t*>(ltab);
        copy_table_to_lds<256, 8, true>(lt16, a.cs, pairs);
        tv.tab16 = lt16;
        tv.tab = nullptr;
      } else if (TLDS) {
        copy_table_to_lds<256, 8, false>(ltab, a.cs, pairs);
        tv.tab = ltab;
      } else {
        tv.tab = a.cs;
      }
      tv.tbase = 0;
      tv.ntr = a.T;
      tv.t_last = a.T - 1;
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int i = k * LPH + li;
      if ((k + 1) * LPH <= CH || i < CH)
        *reinterpret_cast<u32x4*>(sS + row_tile_offset<D>(i / (D / 8), 16 * (i % (D / 8)))) = v[k];
    }
  } else if constexpr (SRC == kSrcInBlock) {
    // the whole pass in one block per head: the table, then the state over
    // all N tokens (the state kernel's waves, one 16-token tile each in turn),
    // the four waves' sums added in wave order through LDS and written into
    // the operand layout
    using Cf = StateCfg<D>;
    constexpr int KS2 = Cf::KS;
    unsigned char* scr = smem + OPB;
    if (ROPE) {
      if (TLDS) {
        copy_table_to_lds<256, 8, false>(ltab, a.cs, a.T * a.Pt + a.Hh * a.Py + a.W * a.Px);
        tv.tab = ltab;
      } else {
        tv.tab = a.cs;
      }
      tv.tbase = 0;
      tv.ntr = a.T;
      tv.t_last = a.T - 1;
    }
    __syncthreads();
    const int ntile = (N + Cf::TW - 1) / Cf::TW;
    StateWave<D, ROPE> sw{a,
                          tv,
                          make_rsrc(a.k + boff, a.slab_bytes),
                          make_rsrc(a.v + boff, a.slab_bytes),
                          tokstride,
                          (uint32_t)h * D * 2 + 16u * m,
                          0,
                          N,
                          wave,
                          (ntile - wave + 3) / 4,
                          lane,
                          m,
                          col,
                          scr + wave * Cf::WAVE_BYTES};
    sw.run();
#pragma unroll
    for (int msk = 1; msk < 16; msk *= 2)
#pragma unroll
      for (int s2 = 0; s2 < KS2; ++s2)
#pragma unroll
        for (int j = 0; j < 8; ++j) sw.zacc[s2][j] += __shfl_xor(sw.zacc[s2][j], msk);
    __syncthreads();  // every wave is done with its tiles; they become scratch
    float* red = reinterpret_cast<float*>(scr);
    float* zw = reinterpret_cast<float*>(scr + Cf::ZW_OFF);
    if (col == 0) {
#pragma unroll
      for (int s2 = 0; s2 < KS2; ++s2)
#pragma unroll
        for (int j = 0; j < 8; ++j) zw[wave * D + 8 * (4 * s2 + m) + j] = sw.zacc[s2][j];
    }
    __syncthreads();
    if (tid < D) {
      const float zs = ((zw[tid] + zw[D + tid]) + zw[2 * D + tid]) + zw[3 * D + tid];
      const uint32_t hl = pack_bf16(zs, 0.f) & 0xffffu;
      *reinterpret_cast<uint16_t*>(sS + row_tile_offset<D>(D, 2 * tid)) = (uint16_t)hl;
      *reinterpret_cast<uint16_t*>(sS + row_tile_offset<D>(D + 1, 2 * tid)) =
          (uint16_t)(pack_bf16(zs - __uint_as_float(hl << 16), 0.f) & 0xffffu);
    }
    constexpr int NTI = Cf::RT * Cf::RT;
    constexpr int WSTRIDE = Cf::RED_TILES * 1024;
#pragma unroll
    for (int t0 = 0; t0 < NTI; t0 += Cf::RED_TILES) {
      __syncthreads();  // the previous round's reads (and the z reads) are done
#pragma unroll
      for (int qq = 0; qq < Cf::RED_TILES; ++qq) {
        if (t0 + qq < NTI) {
          const int ti = (t0 + qq) / Cf::RT, tj = (t0 + qq) % Cf::RT;
#pragma unroll
          for (int r = 0; r < 16; ++r) red[wave * WSTRIDE + (qq * 16 + r) * 64 + lane] = sw.acc[ti][tj][r];
        }
      }
      __syncthreads();
      for (int idx = tid; idx < WSTRIDE; idx += 256) {
        const int qq = idx / 1024, r = (idx / 64) % 16, l = idx % 64;
        if (t0 + qq < NTI) {
          const int ti = (t0 + qq) / Cf::RT, tj = (t0 + qq) % Cf::RT;
          const float sum = ((red[idx] + red[WSTRIDE + idx]) + red[2 * WSTRIDE + idx]) +
                            red[3 * WSTRIDE + idx];
          const int d = 32 * ti + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
          const int e = 32 * tj + (l & 31);
          *reinterpret_cast<uint16_t*>(sS + row_tile_offset<D>(out_row_of<D>(e), 2 * d)) =
              (uint16_t)(pack_bf16(sum, 0.f) & 0xffffu);
        }
      }
    }
  } else if constexpr (SRC == kSrcPartials) {
    // the reduction folded in: S and z are the sums of the head's C <= 16
    // chunk partials in the reduce kernel's pairwise tree (so the same
    // values), written straight into the operand layout (row out_row_of(e)
    // holds column e of S; rows D and D + 1 the hi and lo halves of z)
    const float* pp = a.part + (size_t)bh * a.C * (D * D + D);
    constexpr int GR = (D * D + D) / 4;  // groups of four floats
    for (int gi = tid; gi < GR; gi += 256) {
      f32x4 x[kFoldMaxChunks];
#pragma unroll
      for (int c = 0; c < kFoldMaxChunks; ++c)
        x[c] = c < a.C ? *reinterpret_cast<const f32x4*>(pp + (size_t)c * (D * D + D) + 4 * gi)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 acc = sum_chunks<kFoldMaxChunks>(x);
      if (gi < D * D / 4) {
        const int d = gi / (D / 4), e0 = 4 * (gi % (D / 4));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint16_t*>(sS + row_tile_offset<D>(out_row_of<D>(e0 + j), 2 * d)) =
              (uint16_t)(pack_bf16(acc[j], 0.f) & 0xffffu);
      } else {
        const int z0 = 4 * (gi - D * D / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t hl = pack_bf16(acc[j], 0.f) & 0xffffu;
          const float hi = __uint_as_float(hl << 16);
          *reinterpret_cast<uint16_t*>(sS + row_tile_offset<D>(D, 2 * (z0 + j))) = (uint16_t)hl;
          *reinterpret_cast<uint16_t*>(sS + row_tile_offset<D>(D + 1, 2 * (z0 + j))) =
              (uint16_t)(pack_bf16(acc[j] - hi, 0.f) & 0xffffu);
        }
      }
    }
    if (ROPE) {
      if (TLDS) {
        copy_table_to_lds<256, 8, false>(ltab, a.cs, a.T * a.Pt + a.Hh * a.Py + a.W * a.Px);
        tv.tab = ltab;
      } else {
        tv.tab = a.cs;
      }
      tv.tbase = 0;
      tv.ntr = a.T;
      tv.t_last = a.T - 1;
    }
  } else {
    RowStage<D, D, 256> st_s;
    RowStage<D, 2, 256, D> st_z;
    const uint16_t* sl = a.sl + (size_t)bhb * ROWS * D;
    st_s.load(sl);
    st_z.load(sl);
    if (ROPE) {
      if (TLDS) {
        copy_table_to_lds<256, 8, false>(ltab, a.cs, a.T * a.Pt + a.Hh * a.Py + a.W * a.Px);
        tv.tab = ltab;
      } else {
        tv.tab = a.cs;
      }
      tv.tbase = 0;
      tv.ntr = a.T;
      tv.t_last = a.T - 1;
    }
    st_s.store(sS);
    st_z.store(sS);
  }
  __syncthreads();

  // three register sets: the loads of the next two steps are in flight
  // during a step
  // At D = 128 the loop runs whole rounds of three steps with no exit inside
  // a round, and the last one or two steps follow it: with an exit after
  // every step, the compiler merges the exits' state into the loop head,
  // which then waits for the next step's loads as well (3.5% of the kernel
  // at 5B 720p/60s, 4% at 5B 480p/81f).  With four heads' q tiles, or at
  // D <= 64, the whole-round form needs more registers than it saves, and
  // the loop keeps its exits.
  u32x4 qc[KS];
  OChunk gc[4];
  if (base < N) {
    load_qg(base + stride, qb, gb);
    if constexpr ((QROWS && G == 4) || D < 128) {
      for (;;) {
        load_qg(base + 2 * stride, qc, gc);
        step(base, qa, ga);
        if (base + stride >= N) break;
        load_qg(base + 3 * stride, qa, ga);
        step(base + stride, qb, gb);
        if (base + 2 * stride >= N) break;
        load_qg(base + 4 * stride, qb, gb);
        step(base + 2 * stride, qc, gc);
        if (base + 3 * stride >= N) break;
        base += 3 * stride;
      }
    } else {
      for (; base + 2 * stride < N; base += 3 * stride) {
        load_qg(base + 2 * stride, qc, gc);
        step(base, qa, ga);
        load_qg(base + 3 * stride, qa, ga);
        step(base + stride, qb, gb);
        load_qg(base + 4 * stride, qb, gb);
        step(base + 2 * stride, qc, gc);
      }
      if (base < N) step(base, qa, ga);
      if (base + stride < N) step(base + stride, qb, gb);
    }
  }
}

// D = 32 keeps the one-wave-per-tile kernel (its accumulator is small);
// D = 64 uses the half-state kernel and D = 128 the tile state kernel.
template <int D>
constexpr bool use_half() {
  return D >= 64;
}
template <int D>
constexpr int state_lds_bytes() {
  if constexpr (use_half<D>())
    return HalfCfg<D>::LDS_BYTES;
  else
    return StateCfg<D>::LDS_BYTES;
}
template <int D>
constexpr int output_lds_bytes() {
  return (D + 2) * D * 2;
}



template <int D, int P>
void launch_reduce(const Plan& p, const KArgs& a, hipStream_t stream) {
  const dim3 g2(RedCfg<D>::NTILE, p.BH);
  hipLaunchKernelGGL((reduce_kernel<D, P>), g2, dim3(256), 0, stream, a);
}


template <int D>
hipError_t launch_reduce_d(const Plan& p, const KArgs& a, hipStream_t stream) {
  if (p.CB <= 8)
    launch_reduce<D, 8>(p, a, stream);
  else if (p.CB <= 16)
    launch_reduce<D, 16>(p, a, stream);
  else
    launch_reduce<D, 32>(p, a, stream);
  return hipGetLastError();
}

template <int D, bool ROPE, bool TLDS>
hipError_t launch_state_k(const Plan& p, const KArgs& a, size_t lds, hipStream_t stream) {
  const dim3 g1(p.C, p.BH);
  if constexpr (D == 128) {
    const size_t lds_t = lds - state_lds_bytes<D>() + TileCfg::LDS_BYTES;
    hipError_t e = allow_lds<state_tile_kernel<ROPE, TLDS>>(lds_t);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((state_tile_kernel<ROPE, TLDS>), g1, dim3(512), lds_t, stream, a);
  } else if constexpr (use_half<D>()) {
    hipError_t e = allow_lds<state_half_kernel<D, ROPE, TLDS>>(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((state_half_kernel<D, ROPE, TLDS>), g1, dim3(512), lds, stream, a);
  } else {
    hipError_t e = allow_lds<state_kernel<D, ROPE, TLDS>>(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((state_kernel<D, ROPE, TLDS>), g1, dim3(256), lds, stream, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_state_d(const Plan& p, KArgs a, hipStream_t stream, bool reduce) {
  const bool tl = a.cs && table_lds_bytes(a) <= kMaxLdsTableBytes;
  const size_t lds = state_lds_bytes<D>() + (tl ? table_lds_bytes(a) : 0);
  hipError_t e0;
  if (!a.cs)
    e0 = launch_state_k<D, false, false>(p, a, lds, stream);
  else if (tl)
    e0 = launch_state_k<D, true, true>(p, a, lds, stream);
  else
    e0 = launch_state_k<D, true, false>(p, a, lds, stream);
  if (e0 != hipSuccess) return e0;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !reduce) return e;
  return launch_reduce_d<D>(p, a, stream);
}

// A kernel as a type, so one generic launch helper can take any of them.
template <auto K>
struct KernelTag {
  static constexpr auto value = K;
};

size_t persist_table_pairs(const KArgs& a) {
  return (size_t)a.T * a.Pt + (size_t)a.Hh * a.Py + (size_t)a.W * a.Px;
}
// LDS of a persistent output block besides the table: G heads' S operands
// and, with whole-row q loads, the four waves' q tiles.
template <int D, int G, bool QR>
constexpr size_t persist_fixed_lds() {
  return G * output_lds_bytes<D>() + (QR ? 4 * 16 * 2 * D : 0);
}

// Persistent output launch with G heads per block: about kPersistBlocks
// blocks, one per compute unit (the LDS request keeps a second block off).
// The RoPE table goes into LDS as fp32 pairs when it fits, else (grouped
// blocks only) as fp16 pairs, else it is read from global memory.
// Blocks per head group of the persistent output launch: about
// kPersistBlocks in all, but no more per group than it has ranges.
// A group is G heads of one attention block (the whole sequence for the
// bidirectional mixer), so a block-causal pass has NB times as many.
long long persist_groups(const Plan& p, int G) { return (long long)(p.BH / G) * p.NB; }
int persist_nsub(const Plan& p, int G) {
  const long long groups = persist_groups(p, G);
  const int ranges = (p.BT + 64 / G - 1) / (64 / G);
  const int nsub = kPersistBlocks / groups > 0 ? (int)(kPersistBlocks / groups) : 1;
  return nsub < ranges ? nsub : ranges;
}

template <int D, int G, bool QR, int SRC = kSrcReduced>
hipError_t launch_output_persist(const Plan& p, KArgs a, hipStream_t stream) {
  // kSrcInBlock: one block per head, which forms the state itself
  const int nsub = SRC == kSrcInBlock ? 1 : persist_nsub(p, G);
  const size_t pairs = persist_table_pairs(a);
  const size_t fixed =
      persist_fixed_lds<D, G, QR>() + (SRC == kSrcInBlock ? StateCfg<D>::LDS_BYTES : 0);
  const bool t32 = a.cs && 8 * pairs <= kMaxPersistTableBytes && fixed + 8 * pairs <= kMaxLdsPerBlock;
  const bool t16 = G > 1 && a.cs && !t32 && fixed + 4 * pairs <= kMaxLdsPerBlock;
  size_t lds = fixed + (t32 ? 8 * pairs : (t16 ? 4 * pairs : 0));
  if (lds < kPersistLdsBytes) lds = kPersistLdsBytes;
  const dim3 g(p.H / G, nsub * p.NB, p.B);
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = allow_lds<decltype(kern)::value>(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decltype(kern)::value, g, dim3(256), lds, stream, a, nsub);
    return hipGetLastError();
  };
  if (!a.cs) return go(KernelTag<output_persist_kernel<D, false, false, G, false, QR, SRC>>{});
  if (t32) return go(KernelTag<output_persist_kernel<D, true, true, G, false, QR, SRC>>{});
  if constexpr (G > 1) {
    if (t16) return go(KernelTag<output_persist_kernel<D, true, true, G, true, QR>>{});
  }
  return go(KernelTag<output_persist_kernel<D, true, false, G, false, QR, SRC>>{});
}

template <int D>
hipError_t launch_output_d(const Plan& p, KArgs a, hipStream_t stream, int src) {
  if constexpr (D <= 64) {
    if (src == kSrcPartials) return launch_output_persist<D, 1, false, kSrcPartials>(p, a, stream);
    if (src == kSrcInBlock) return launch_output_persist<D, 1, false, kSrcInBlock>(p, a, stream);
  }
  if constexpr (D == 128) {
    // as many heads per block (4, then 2) as divide H with the table in LDS
    // (fp16 pairs at least; whole-row q tiles if they fit beside it): the
    // blocks of a group read whole contiguous runs of the group's heads,
    // which streams faster than one head's rows.  A block stages G heads'
    // operands, so this pays only where each wave then runs at least
    // kGroupMinSteps steps (5B 480p/81f, with about 5, measured 19.5 us
    // per output pass with one head per block and 22.7 with four).
    // Block-causal passes (NB > 1) take the persistent kernel too while
    // their groups, one per (attention block, G heads), fill at least 7/8
    // of the chip's rounds of blocks; other lists of attention blocks keep
    // output_kernel (5B 720p/60s in 5-frame blocks: 185 persistent blocks
    // measured 825 us per pass against 820 with it).
    const size_t tb16 = a.cs ? 4 * persist_table_pairs(a) : 0;
    auto fits = [&](int G) {
      if (p.NB == 1) return true;
      const long long groups = persist_groups(p, G);
      if (groups > kPersistBlocks) {
        // one block per group (nsub = 1) in several rounds, with the rounds
        // 7/8 full on average, and grouped heads only: 5B 720p/60s in
        // 1-frame blocks (905 four-head groups) 1,047 -> 1,016 us per pass,
        // but 14B 480p in 1-frame blocks (1,600 one-head groups) 248 -> 258
        if (G == 1) return false;
        const long long rounds = (groups + kPersistBlocks - 1) / kPersistBlocks;
        return groups * 8 >= rounds * kPersistBlocks * 7;
      }
      return groups * persist_nsub(p, G) >= kPersistBlocks * 7 / 8;
    };
    auto steps = [&](int G) {
      const long long groups = persist_groups(p, G);
      const int nsub = kPersistBlocks / groups > 0 ? (int)(kPersistBlocks / groups) : 1;
      return (p.BT + 64 / G * nsub - 1) / (64 / G * nsub);
    };
    if (p.H % 4 == 0 && fits(4) && steps(4) >= kGroupMinSteps) {
      if (persist_fixed_lds<D, 4, true>() + tb16 <= kMaxLdsPerBlock)
        return launch_output_persist<D, 4, true>(p, a, stream);
      if (persist_fixed_lds<D, 4, false>() + tb16 <= kMaxLdsPerBlock)
        return launch_output_persist<D, 4, false>(p, a, stream);
    }
    if (p.H % 2 == 0 && fits(2) && steps(2) >= kGroupMinSteps &&
        persist_fixed_lds<D, 2, true>() + tb16 <= kMaxLdsPerBlock)
      return launch_output_persist<D, 2, true>(p, a, stream);
    if (fits(1)) return launch_output_persist<D, 1, true>(p, a, stream);
  } else {
    if (p.NB == 1) return launch_output_persist<D, 1, false>(p, a, stream);
  }
  const dim3 g3(p.BH, p.C2);
  const bool tl = a.cs && table_lds_bytes(a) <= kMaxLdsTableBytes;
  const size_t lds = output_lds_bytes<D>() + (tl ? table_lds_bytes(a) : 0);
  if (!a.cs)
    hipLaunchKernelGGL((output_kernel<D, false, false>), g3, dim3(256), lds, stream, a);
  else if (tl)
    hipLaunchKernelGGL((output_kernel<D, true, true>), g3, dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL((output_kernel<D, true, false>), g3, dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// Fixed scratch for the entry point that allocates nothing: the forward
// workspace (chunk partials and the bf16 state operand) of any call that fits
// in kScratchBytes.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code the array's name is only a stand-in for the
// device address; that address is looked up once per device, with the device
// current, and kept.
namespace {
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t scratch_pointer(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_state(const Plan& p, KArgs a, hipStream_t stream, bool reduce) {
  switch (p.D) {
    case 32: return launch_state_d<32>(p, a, stream, reduce);
    case 64: return launch_state_d<64>(p, a, stream, reduce);
    case 128: return launch_state_d<128>(p, a, stream, reduce);
    default: return hipErrorInvalidValue;
  }
}

bool output_sums_partials(const Plan& p) {
  if (p.NB != 1 || p.D > 64 || p.BH == 0 || p.N == 0) return false;
  const size_t per_block = (size_t)p.C * (size_t)(p.D * p.D + p.D) * sizeof(float);
  const size_t blocks = (size_t)p.BH * (size_t)persist_nsub(p, 1);
  return p.C <= kFoldMaxChunks && per_block <= kFoldBlockBytes &&
         per_block * blocks <= kFoldTotalBytes;
}

hipError_t launch_reduce_state(const Plan& p, KArgs a, hipStream_t stream) {
  switch (p.D) {
    case 32: return launch_reduce_d<32>(p, a, stream);
    case 64: return launch_reduce_d<64>(p, a, stream);
    case 128: return launch_reduce_d<128>(p, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_carry(const Plan& p, KArgs a, hipStream_t stream) {
  a.NB = 0;
  switch (p.D) {
    case 32: launch_reduce<32, 8>(p, a, stream); break;
    case 64: launch_reduce<64, 8>(p, a, stream); break;
    case 128: launch_reduce<128, 8>(p, a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_output(const Plan& p, KArgs a, hipStream_t stream, bool sum_partials) {
  const int src = sum_partials ? kSrcPartials : kSrcReduced;
  switch (p.D) {
    case 32: return launch_output_d<32>(p, a, stream, src);
    case 64: return launch_output_d<64>(p, a, stream, src);
    case 128: return launch_output_d<128>(p, a, stream, src);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pass_in_block(const Plan& p, KArgs a, hipStream_t stream) {
  switch (p.D) {
    case 32: return launch_output_d<32>(p, a, stream, kSrcInBlock);
    case 64: return launch_output_d<64>(p, a, stream, kSrcInBlock);
    default: return hipErrorInvalidValue;
  }
}

bool pass_in_block(const Plan& p) {
  return p.NB == 1 && p.D <= 64 && p.BH > 0 && (long long)p.N * p.D <= kInBlockMaxND;
}

}  // namespace gla
