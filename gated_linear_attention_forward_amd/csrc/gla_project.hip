// gla_project.hip -- gfx950 kernels of the projection prologue: q, k, v and
// g as linear maps of the hidden states ("SANA-Video 2.0", NVlabs Sana docs,
// section Architecture: hidden size 2,560 with 20 heads x 128 at 5B, 4,096
// with 32 heads x 128 at 14B), fused with the mixer's state contraction so
// that k and v never go to memory.
//
// x is bf16 [B, N, C]; the weights are bf16 [4][H*D][C] (maps q, k, v, g;
// row j of a map is output feature j, contiguous over C).  Each map is
// y = x W^T, rounded to bf16 as a BF16 model stores it.
//
// Both kernels run the same GEMM main loop on a tile of TM = 256 tokens of
// one batch element and the 2 D output features of one head in two maps
// (k and v, or q and g) on v_mfma_f32_32x32x16_bf16 (A = x rows, B = W rows:
// both operands are contiguous over C).  At D >= 64 a block has 8 waves, two
// per SIMD, each computing 128 tokens x 2D/4 features (128 accumulation
// registers at D = 128); at D = 32, 4 waves of 128 x 32.  Per K-step of 64
// the x tile (256 x 64) and the W tile (2 D x 64) load straight into one of
// two LDS stages while the other stage is multiplied.
//
//   kv kernel  one block per (state chunk, head), looping over the chunk's
//              tiles; after each tile's GEMM: bf16(k) with ReLU and bf16(v)
//              to feature-major LDS tiles, the rotation applied in place
//              (each thread owns four tokens and every PGS-th pair) while z
//              accumulates the unrotated features, then S += rk^T v over the
//              tile's tokens on MFMA (each wave owns an eighth of S's 32x32
//              tiles at D = 128); at the end the block writes the same fp32 (S_c, z_c)
//              partial the state kernel writes, for the same reduce kernel;
//   qg kernel  one block per (token tile, head): q and g through a
//              token-major LDS tile to 16-byte row stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {
namespace {

// Token tiles per group of the qg kernel's XCD-aware block numbering.
constexpr int kQgGroupTiles = 4;

template <int D>
struct ProjCfg {
  static constexpr int TM = kProjTileTokens;  // tokens per tile
  static constexpr int KT = 64;               // K per stage (128 bytes of a row)
  // A stage holds the x tile (TM rows) and the W tile (2 D rows) in 1 KB
  // load groups of 8 rows of 128 bytes, each group padded by 64 bytes; row q
  // of a group stores its 16-byte chunk c at position c ^ (q / 2).  The 16
  // rows a 16-lane fragment read touches then fall in 16 distinct bank
  // groups, and one buffer-load-to-LDS instruction fills one group.
  static constexpr int GP = 1024 + 64;
  static constexpr int AG = TM / 8;           // x groups per stage
  static constexpr int BG = 2 * D / 8;        // W groups per stage
  static constexpr int A_BYTES = AG * GP;
  static constexpr int STAGE = (AG + BG) * GP;
  // 8 waves (two per SIMD) where a wave still gets 32 columns, else 4
  static constexpr int NW = D >= 64 ? 8 : 4;
  static constexpr int NT = 64 * NW;
  static constexpr int WN = NW / 2;           // column groups (two row groups of TM / 2 tokens)
  static constexpr int WC = 2 * D / WN;       // columns per wave
  static constexpr int WT = TM / 2;           // tokens per wave
  static constexpr int MI = WT / 32;          // 32-row subtiles per wave
  static constexpr int NI = WC / 32;          // 32-column subtiles per wave
  static constexpr int GPW = (AG + BG) / NW;  // load groups per wave and stage
  // kv epilogue: feature-major tiles [D][TM] of R phi(k) and v
  static constexpr int FP = TM * 2 + 16;
  static constexpr int KV_BYTES = 2 * D * FP;
  static constexpr int ST = (D / 32) * (D / 32);        // 32x32 tiles of S
  static constexpr int STW = (ST + NW - 1) / NW;        // per wave
  static constexpr int TQ = TM / 4;                     // token quads of the rotation pass
  static constexpr int PGS = NT / TQ;                   // pair groups of the rotation pass
  // qg epilogue: token-major tile [TM][2 D]
  static constexpr int QP = 4 * D + 16;
  static constexpr int QG_BYTES = TM * QP;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(KV_BYTES <= LDS_BYTES && QG_BYTES <= LDS_BYTES, "epilogue tiles fit the stages");
  static_assert((AG + BG) % NW == 0, "whole load groups per wave");
  static_assert(NI >= 1 && MI >= 1 && D % 8 == 0, "a 32-column subtile, whole groups per map");
  static_assert(TQ <= 64 && NT % TQ == 0 && D / 2 % PGS == 0, "pairs split evenly over the pair groups");
  static_assert(LDS_BYTES + kMaxLdsTableBytes <= 160 * 1024, "stages and the RoPE table fit the LDS");
};

struct Gemm {
  __amdgpu_buffer_rsrc_t rx, rw;
  uint32_t x_row;      // bytes per x row (C * 2)
  int n_tile_end;      // tokens at or past this one load zeros
  int wrow0, wrow1;    // first W row of the two maps' head slices
};

typedef __attribute__((address_space(3))) void lds_void;

// The main loop: acc[mi][ni] += x[tile rows] W[cols]^T over the whole of C.
// Wave (wm, wn) computes tokens WT wm .. + WT and columns WC wn .. + WC of
// the tile's 2 D columns (the first D are map 0, the rest map 1).  The next
// stage's groups load straight into LDS while this stage is multiplied
// (spread over its 16-wide k-steps); past the last K-step the offsets lie
// outside the buffers and load zeros, and an odd step count runs one extra
// step over a zero stage, which adds exactly nothing.
template <int D>
__device__ __forceinline__ void gemm_tile(const Gemm& gm, int tile0, int Cdim, unsigned char* smem,
                                          f32x16 (&acc)[ProjCfg<D>::MI][ProjCfg<D>::NI]) {
  using Cf = ProjCfg<D>;
  constexpr int MI = Cf::MI, NI = Cf::NI, GP = Cf::GP;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // load side: lane i fills row q = i / 8 of a group with chunk (i % 8) ^ (q / 2)
  const int lq = lane >> 3;
  const uint32_t lchunk = 16u * (uint32_t)((lane & 7) ^ (lq >> 1));
  // the lane's offset of its chunk at K = 0 in each of the wave's groups
  // (rows past the tile's end lie outside the buffer)
  uint32_t goff[Cf::GPW];
#pragma unroll
  for (int i = 0; i < Cf::GPW; ++i) {
    const int g = wave * Cf::GPW + i;
    const int n = tile0 + 8 * g + lq;
    const int row = 8 * (g - Cf::AG) + lq;
    const int wr = (row < D ? gm.wrow0 : gm.wrow1 - D) + row;
    const uint32_t xo = n < gm.n_tile_end ? (uint32_t)n * gm.x_row : kOob;
    goff[i] = (g < Cf::AG ? xo : (uint32_t)wr * gm.x_row) + lchunk;
  }
  auto issue = [&](int i, int k0, bool valid, unsigned char* stg) {
    const int g = wave * Cf::GPW + i;  // wave-uniform
    const uint32_t off = valid ? goff[i] + (uint32_t)k0 * 2u : kOob;
    const __amdgpu_buffer_rsrc_t r = g < Cf::AG ? gm.rx : gm.rw;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(stg + g * GP), 16, off, 0, 0, 0);
  };
  // read side: row r, chunk c at (r / 8) GP + (r % 8) 128 + 16 (c ^ (r % 8 / 2)).
  // The lane's rows have r % 8 = l % 8; its chunk is 2 ks + l / 32, so the
  // swizzle moves it by +-2 chunks depending on the parity of ks: two bases.
  const int q = lane & 7, sw = q >> 1, kh = lane >> 5;
  const int lo = kh ^ (sw & 1), hi = sw >> 1;
  const int rbase = q * 128 + 16 * lo;
  const int base_even = rbase + 32 * hi, base_odd = rbase - 32 * hi;
  const int arow = Cf::WT * wm + (lane & 31), brow = Cf::WC * wn + (lane & 31);
  const int a_grp = (arow >> 3) * GP, b_grp = Cf::A_BYTES + (brow >> 3) * GP;

  const int nk = Cdim / Cf::KT;
#pragma unroll
  for (int i = 0; i < Cf::GPW; ++i) issue(i, 0, true, smem);
  __syncthreads();
  // step kt (P = kt % 2): multiply stage P while stage 1 - P loads step kt + 1
  auto step = [&](auto PAR, int kt) {
    constexpr int P = decltype(PAR)::value;
    const unsigned char* st = smem + P * Cf::STAGE;
    unsigned char* nx = smem + (1 - P) * Cf::STAGE;
    const bool valid = kt + 1 < nk;
    static_for<Cf::KT / 16>([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      constexpr int g0 = ks * Cf::GPW / (Cf::KT / 16), g1 = (ks + 1) * Cf::GPW / (Cf::KT / 16);
#pragma unroll
      for (int i = g0; i < g1; ++i) issue(i, (kt + 1) * Cf::KT, valid, nx);
      const int kbase = ((ks & 1) ? base_odd : base_even) + 32 * ks;
      bf16x8 A[MI], Bm[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        A[mi] = *reinterpret_cast<const bf16x8*>(st + a_grp + 4 * mi * GP + kbase);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        Bm[ni] = *reinterpret_cast<const bf16x8*>(st + b_grp + 4 * ni * GP + kbase);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[mi], Bm[ni], acc[mi][ni], 0, 0, 0);
    });
    // the next stage has landed and every wave is done with this one
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
  }
}

// ---------------------------------------------------------------------------
// kv kernel
template <int D, bool ROPE, bool TLDS>
__global__ __launch_bounds__(64 * ProjCfg<D>::NW)
__attribute__((amdgpu_waves_per_eu(ProjCfg<D>::NW / 4, ProjCfg<D>::NW / 4)))
void proj_kv_kernel(KArgs a, PArgs pa) {
  using Cf = ProjCfg<D>;
  constexpr int TM = Cf::TM, FP = Cf::FP, PGS = Cf::PGS, NPG = D / 2 / PGS;  // pairs per thread
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float2* ltab = reinterpret_cast<float2*>(smem + Cf::LDS_BYTES);
  unsigned char* ktile = smem;
  unsigned char* vtile = smem + D * FP;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // heads vary fastest: with B*H a multiple of the 8 XCDs, each XCD's L2
  // serves a fixed handful of heads' weight slices
  const int bh = blockIdx.x, c = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  int n_begin, n_end;
  range_of(a, c, n_begin, n_end);
  TabView tv{};
  if (ROPE) tv = stage_table<D, Cf::NT>(a, ltab, TLDS, n_begin, n_end);
  __syncthreads();

  const int HD = a.H * D;
  Gemm gm;
  gm.rx = make_rsrc(pa.x + (size_t)b * a.N * pa.Cdim, (uint32_t)((size_t)a.N * pa.Cdim * 2));
  gm.rw = make_rsrc(pa.w, (uint32_t)((size_t)4 * HD * pa.Cdim * 2));
  gm.x_row = (uint32_t)pa.Cdim * 2u;
  gm.n_tile_end = n_end;
  gm.wrow0 = 1 * HD + h * D;  // k
  gm.wrow1 = 2 * HD + h * D;  // v

  f32x16 accS[Cf::STW];
#pragma unroll
  for (int u = 0; u < Cf::STW; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) accS[u][r] = 0.f;
  float zacc[NPG][2];
#pragma unroll
  for (int i = 0; i < NPG; ++i) zacc[i][0] = zacc[i][1] = 0.f;
  const int tq = tid % Cf::TQ, pg = tid / Cf::TQ;
  // this wave's columns: map (0: k, 1: v) and first feature
  const int wmap = (Cf::WC * wn) / D, wf0 = (Cf::WC * wn) % D;

  for (int tile0 = n_begin; tile0 < n_end; tile0 += TM) {
    f32x16 acc[Cf::MI][Cf::NI];
    gemm_tile<D>(gm, tile0, pa.Cdim, smem, acc);
    // bf16 phi(k) and bf16 v, feature-major: lane column = feature, four
    // consecutive tokens per accumulator quarter
    unsigned char* dst = wmap ? vtile : ktile;
#pragma unroll
    for (int mi = 0; mi < Cf::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < Cf::NI; ++ni)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int f = wf0 + 32 * ni + (lane & 31);
          const int t = Cf::WT * wm + 32 * mi + 8 * rg + 4 * (lane >> 5);
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float val = acc[mi][ni][4 * rg + j];
            y[j] = wmap ? val : fmaxf(val, 0.f);
          }
          typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
          *reinterpret_cast<u32x2v*>(dst + f * FP + 2 * t) =
              u32x2v{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
        }
    __syncthreads();
    // z and the rotation: thread (tq, pg) owns tokens 4 tq .. + 3 and pairs
    // pg, pg + PGS, ...
    {
      RowOff ro[4];
      if (ROPE) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int t, y, x;
          grid_pos(a, (uint32_t)min(tile0 + 4 * tq + j, n_end - 1), t, y, x);
          ro[j] = row_offsets<D>(a, tv, t, y, x);
        }
      }
#pragma unroll
      for (int i = 0; i < NPG; ++i) {
        const int p = pg + PGS * i;
        typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
        u32x2v* r0 = reinterpret_cast<u32x2v*>(ktile + (2 * p) * FP + 8 * tq);
        u32x2v* r1 = reinterpret_cast<u32x2v*>(ktile + (2 * p + 1) * FP + 8 * tq);
        const u32x2v w0 = *r0, w1 = *r1;
        float e0[4] = {bf_lo(w0[0]), bf_hi(w0[0]), bf_lo(w0[1]), bf_hi(w0[1])};
        float e1[4] = {bf_lo(w1[0]), bf_hi(w1[0]), bf_lo(w1[1]), bf_hi(w1[1])};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          zacc[i][0] += e0[j];
          zacc[i][1] += e1[j];
        }
        if (ROPE) {
          float o0[4], o1[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float2 f = rope_factor<D, 0, D / 2 - 1>(tv, ro[j], p);
            o0[j] = e0[j] * f.x - e1[j] * f.y;
            o1[j] = e0[j] * f.y + e1[j] * f.x;
          }
          *r0 = u32x2v{pack_bf16(o0[0], o0[1]), pack_bf16(o0[2], o0[3])};
          *r1 = u32x2v{pack_bf16(o1[0], o1[1]), pack_bf16(o1[2], o1[3])};
        }
      }
    }
    __syncthreads();
    // S += rk^T v over the tile's tokens (k-steps of 16 tokens)
#pragma unroll
    for (int u = 0; u < Cf::STW; ++u) {
      const int q = wave + Cf::NW * u;
      if (q < Cf::ST) {
        const int ti = q / (D / 32), tj = q % (D / 32);
        const unsigned char* ar = ktile + (32 * ti + (lane & 31)) * FP + 16 * (lane >> 5);
        const unsigned char* br = vtile + (32 * tj + (lane & 31)) * FP + 16 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < TM / 16; ++ks) {
          const bf16x8 A = *reinterpret_cast<const bf16x8*>(ar + 32 * ks);
          const bf16x8 Bv = *reinterpret_cast<const bf16x8*>(br + 32 * ks);
          accS[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bv, accS[u], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the tiles are the next GEMM's stages
  }

  float* dstp = a.part + ((size_t)bh * a.C + c) * (size_t)(D * D + D);
#pragma unroll
  for (int u = 0; u < Cf::STW; ++u) {
    const int q = wave + Cf::NW * u;
    if (q < Cf::ST) {
      const int ti = q / (D / 32), tj = q % (D / 32);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * ti + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int e = 32 * tj + (lane & 31);
        dstp[d * D + e] = accS[u][r];
      }
    }
  }
  // z: the TQ threads of a pair group hold the same features
#pragma unroll
  for (int i = 0; i < NPG; ++i)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float s = zacc[i][hf];
#pragma unroll
      for (int msk = 1; msk < Cf::TQ; msk *= 2) s += __shfl_xor(s, msk);
      if (tq == 0) dstp[D * D + 2 * (pg + PGS * i) + hf] = s;
    }
}

// ---------------------------------------------------------------------------
// qg kernel
template <int D>
__global__ __launch_bounds__(64 * ProjCfg<D>::NW)
__attribute__((amdgpu_waves_per_eu(ProjCfg<D>::NW / 4, ProjCfg<D>::NW / 4)))
void proj_qg_kernel(KArgs a, PArgs pa) {
  using Cf = ProjCfg<D>;
  constexpr int TM = Cf::TM, QP = Cf::QP;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // Blocks go to the 8 XCDs in turn (block i to XCD i % 8), and each XCD has
  // its own L2.  The 1-D grid is renumbered so that XCD x takes a contiguous
  // run of logical tiles, ordered in groups of kQgGroupTiles token tiles
  // across all heads, token tiles fastest.  The blocks an XCD holds at once
  // then cover a few token tiles (x rows) times a few heads (weight rows),
  // and both are reused from its L2.
  int bh, tile;
  {
    const int T = gridDim.x, BHn = T / a.CB, pb = blockIdx.x;
    const int xcd = pb & 7, per = T >> 3, rem = T & 7;
    const int lg = xcd * per + min(xcd, rem) + (pb >> 3);
    const int grp = lg / (kQgGroupTiles * BHn), first = grp * kQgGroupTiles;
    const int gsz = min(a.CB - first, kQgGroupTiles);
    const int r = lg - grp * kQgGroupTiles * BHn;
    tile = first + r % gsz;
    bh = r / gsz;
  }
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  int n_begin, n_end;
  range_of(a, tile, n_begin, n_end);

  const int HD = a.H * D;
  Gemm gm;
  gm.rx = make_rsrc(pa.x + (size_t)b * a.N * pa.Cdim, (uint32_t)((size_t)a.N * pa.Cdim * 2));
  gm.rw = make_rsrc(pa.w, (uint32_t)((size_t)4 * HD * pa.Cdim * 2));
  gm.x_row = (uint32_t)pa.Cdim * 2u;
  gm.n_tile_end = n_end;
  gm.wrow0 = 0 * HD + h * D;  // q
  gm.wrow1 = 3 * HD + h * D;  // g

  f32x16 acc[Cf::MI][Cf::NI];
  gemm_tile<D>(gm, n_begin, pa.Cdim, smem, acc);
  // token-major tile: row t holds q (D bf16) then g (D bf16)
#pragma unroll
  for (int mi = 0; mi < Cf::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < Cf::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = Cf::WT * wm + 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int f = Cf::WC * wn + 32 * ni + (lane & 31);
        const __bf16 y = (__bf16)acc[mi][ni][r];
        *reinterpret_cast<__bf16*>(smem + t * QP + 2 * f) = y;
      }
  __syncthreads();
  const size_t boff = (size_t)b * a.N * a.H * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(pa.qbuf + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(pa.gbuf + boff, a.slab_bytes);
  const uint32_t tokstride = (uint32_t)a.H * D * 2;
  constexpr int CPR = D / 8;  // 16-byte chunks per map row
  for (int cidx = tid; cidx < TM * 2 * CPR; cidx += Cf::NT) {
    const int t = cidx / (2 * CPR), part = (cidx / CPR) & 1, u = cidx % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + t * QP + 2 * (part * D + 8 * u));
    const int n = n_begin + t;
    const uint32_t off =
        n < n_end ? (uint32_t)n * tokstride + (uint32_t)h * D * 2 + 16u * u : kOob;
    __builtin_amdgcn_raw_buffer_store_b128(v, part ? rg : rq, off, 0, 0);
  }
}

template <int D>
hipError_t launch_proj_d(const Plan& p, const KArgs& akv, const KArgs& aqg, const PArgs& pa,
                         hipStream_t s) {
  using Cf = ProjCfg<D>;
  // k, v and the state partials
  const bool tl = akv.cs && table_lds_bytes(akv) <= kMaxLdsTableBytes;
  const size_t lds = Cf::LDS_BYTES + (tl ? table_lds_bytes(akv) : 0);
  const dim3 g1(p.BH, p.C);
  hipError_t e;
  if (!akv.cs) {
    if ((e = allow_lds<proj_kv_kernel<D, false, false>>(lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((proj_kv_kernel<D, false, false>), g1, dim3(Cf::NT), lds, s, akv, pa);
  } else if (tl) {
    if ((e = allow_lds<proj_kv_kernel<D, true, true>>(lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((proj_kv_kernel<D, true, true>), g1, dim3(Cf::NT), lds, s, akv, pa);
  } else {
    if ((e = allow_lds<proj_kv_kernel<D, true, false>>(lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((proj_kv_kernel<D, true, false>), g1, dim3(Cf::NT), lds, s, akv, pa);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // q and g
  if ((e = allow_lds<proj_qg_kernel<D>>(Cf::LDS_BYTES)) != hipSuccess) return e;
  const dim3 g2(p.BH * aqg.CB);  // renumbered in the kernel (XCD groups)
  hipLaunchKernelGGL((proj_qg_kernel<D>), g2, dim3(Cf::NT), Cf::LDS_BYTES, s, aqg, pa);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj(const Plan& p, KArgs akv, KArgs aqg, PArgs pa, hipStream_t stream) {
  switch (p.D) {
    case 32: return launch_proj_d<32>(p, akv, aqg, pa, stream);
    case 64: return launch_proj_d<64>(p, akv, aqg, pa, stream);
    case 128: return launch_proj_d<128>(p, akv, aqg, pa, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gla
