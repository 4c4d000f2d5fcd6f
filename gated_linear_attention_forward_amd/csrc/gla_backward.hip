// gla_backward.hip -- gfx950 kernels of the backward pass of the gated
// bidirectional linear-attention mixer: the gradients of q, k, v and the
// gate logits g, given the gradient dout of the output (the hybrid's linear
// layers are trained from scratch: "SANA-Video 2.0: Hybrid Linear Attention
// with Attention Residuals for Efficient Video Generation", Abstract).
//
// Per head, with fq = phi(q_n), rq = R_n fq, den = fq.z + eps, s = sigmoid(g_n)
// and num = S^T rq (the forward's quantities), the chain rule gives
//   a_n  = dout_n * s / den,          dg_n = dout_n * o_n * (1 - s),
//   dden = -(dout_n . o_n) / den,
//   dq_n = [q_n > 0] * (R_n^T (S a_n) + dden z),
//   dS   = sum_n rq a_n^T,            dz = sum_n dden fq,
//   dv_m = dS^T (R_m phi(k_m)),       dk_m = [k_m > 0] * (R_m^T (dS v_m) + dz).
// The pass runs as:
//   1. the forward's state and reduce kernels on (k, v): S and z, with S in
//      two bf16 operand layouts (rows of S^T, as the output kernel takes it,
//      and rows of S) and z in fp32 (or the reduce kernel alone on a state
//      the caller saved from the forward);
//   2. the query kernel here: per token num and den as in the output kernel,
//      then dg, a, dden, S a on MFMA, and dq; each block also contracts its
//      tokens' rq a^T into a dS partial and sums their dden fq into a dz
//      partial;
//   3. the reduce kernel on those partials: dS in the same two operand
//      layouts, and dz in fp32;
//   4. the key kernel here: dv and dS v on MFMA per token, dk.
// Steps 2 and 4 use the output kernel's MFMA orientation (16x16x32, tokens
// as the A operand, lane l holding token l % 16 and features
// 32 s + 8 (l / 16) .. + 7); their accumulators give lane l the MB = D / 16
// contiguous features MB (l % 16) .. of tokens 4 (l / 16) + i, i < 4, so
// each gradient store covers whole token rows and the inverse rotation of a
// pair (2p, 2p + 1) stays inside one lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {
namespace {

constexpr int kQueryWaves = 8;
constexpr int kKeyWaves = 4;

template <int D>
struct BwdCfg {
  static constexpr int KS = D / 32;   // k-steps of 32 features
  static constexpr int MB = D / 16;   // 16-column blocks
  static constexpr int OB = 2 * MB;   // bytes a lane owns of one token row
  static constexpr int PU = D / 32;   // rotation pairs in those bytes
  static constexpr int PITCH = 2 * D;  // row tiles are unpadded and swizzled (row_tile_offset)
  // query kernel LDS: S^T rows + z rows, S rows, fp32 z, then two
  // token-major tiles of the block's 16 NW tokens per step, rq = R phi(q)
  // and a, at a row pitch the transposing reads take without bank conflicts
  static constexpr int TP = tile_pitch(2 * D);
  static constexpr int Q_SR = (D + 2) * PITCH;
  static constexpr int Q_ZF = Q_SR + D * PITCH;
  static constexpr int Q_AT = Q_ZF + 4 * D;
  static constexpr int Q_RQ = Q_AT + 16 * kQueryWaves * TP;
  static constexpr int Q_BYTES = Q_RQ + 16 * kQueryWaves * TP;
  // dS tiles of 32 x 32: wave w owns tiles w, w + NW, ... (row block
  // t / (D / 32) of rq features, column block t % (D / 32) of a features)
  static constexpr int NTI = (D / 32) * (D / 32);
  static constexpr int TPW = (NTI + kQueryWaves - 1) / kQueryWaves;
  // key kernel LDS: dS^T rows, dS rows, fp32 dz
  static constexpr int K_SR = D * PITCH;
  static constexpr int K_ZF = 2 * D * PITCH;
  static constexpr int K_BYTES = K_ZF + 4 * D;
  // key kernel whole-row k and v (D = 128): a 16-token tile of each per wave
  static constexpr int K_TILE = 16 * 2 * D;
  static constexpr int K_TILES = kKeyWaves * 2 * K_TILE;
  static_assert(Q_AT % 16 == 0 && Q_RQ % 16 == 0 && K_ZF % 16 == 0, "16-byte aligned sections");
  static_assert(kQueryWaves * D * 4 <= 16 * kQueryWaves * TP, "dz scratch fits the a tile");
};

// (cos, sin) of the PU rotation pairs PU col + u (u < PU) of token n: the
// pairs of the MB contiguous features the accumulator layout gives lane
// column col.
template <int D>
__device__ __forceinline__ void acc_factors(const KArgs& a, const TabView& tv, int n, int col,
                                            float2 (&cs)[BwdCfg<D>::PU]) {
  constexpr int PU = BwdCfg<D>::PU;
  int t, y, x;
  grid_pos(a, (uint32_t)n, t, y, x);
  const RowOff ro = row_offsets<D>(a, tv, t, y, x);
  static_for<PU>([&](auto U) {
    constexpr int u = decltype(U)::value;
    cs[u] = rope_factor<D, u, PU * 15 + u>(tv, ro, PU * col + u);
  });
}

// Sum over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15); every lane
// gets the same value, added in the same order.
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// acc[j] = sum over k-steps s of A[s] x (LDS rows 16 j + col of `op`, chunk
// 4 s + m): one 16-token step of a token-major contraction against a
// staged operand.  B fragments of block j + 1 are read while block j
// multiplies (fences keep the compiler from reading further ahead).
template <int D>
__device__ __forceinline__ void contract_rows(const unsigned char* op, const bf16x8 (&A)[D / 32],
                                              int col, int m, f32x4 (&acc)[D / 16]) {
  constexpr int KS = D / 32, MB = D / 16;
  bf16x8 Bf[2][KS];
  auto read_b = [&](int j, bf16x8 (&dst)[KS]) {
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      dst[s2] = *reinterpret_cast<const bf16x8*>(op + row_tile_offset<D>(16 * j + col, 16 * (4 * s2 + m)));
  };
  read_b(0, Bf[0]);
  static_for<MB>([&](auto J) {
    constexpr int j = decltype(J)::value;
    if constexpr (j + 1 < MB) read_b(j + 1, Bf[(j + 1) & 1]);
    asm volatile("" ::: "memory");
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s2], Bf[j & 1][s2], acc[j], 0, 0, 0);
  });
}

// ---------------------------------------------------------------------------
// Query kernel.  Block = 8 waves, one (token range, head); grid (B H, C2).
// LDS holds the head's S^T operand and z rows (as in the output kernel), the
// S rows operand, fp32 z, and two token-major tiles of the block's 128
// tokens per step: rq = R phi(q) and a.  Per block step, each wave takes 16
// tokens:
//   - phi(q) against the z rows gives den, R phi(q) against S^T gives num;
//     R phi(q) goes to the rq tile;
//   - per owned column: s = sigmoid(g), o = s num / den, a = dout s / den,
//     dg = dout o (1 - s) (1 - s = e^-g s), and the row sums of dout o;
//   - dg is stored and a (bf16) goes to the a tile;
//   - dden = -(dout . o) / den from a 16-lane DPP sum;
//   - S a on MFMA from the a tile and the S rows operand, rotated back by
//     R^T, plus dden z, masked by q > 0: dq;
//   - dden phi(q) accumulates into the lane's dz partial.
// After an LDS barrier every wave adds the block step's rq a^T to the 32 x 32
// tiles of dS it owns (v_mfma_f32_32x32x16_bf16 over the 128 tokens, both
// operands read with transposing LDS reads as in the state kernel), and a
// second barrier frees the tiles for the next step.  At the end the block
// writes its dS partial and its dz partial, which the reduce kernel sums.
// The loads form a ring: each class (q in the A layout, g and dout, q in the
// row layout) is refilled for the next step as soon as this step is done with
// it.  The barriers wait for LDS only, so those loads stay in flight.
// Every wave runs every block step; tokens past the range load zeros and add
// nothing (rq and a are zero there).
template <int D, bool ROPE, bool TLDS>
__global__ __launch_bounds__(64 * kQueryWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_query_kernel(KArgs a, BArgs bw) {
  using Cf = BwdCfg<D>;
  constexpr int KS = Cf::KS, MB = Cf::MB, OB = Cf::OB, PU = Cf::PU, TP = Cf::TP;
  constexpr int NW = kQueryWaves, NT = 64 * NW;
  using OChunk = typename Chunk<OB>::T;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* sS = smem;
  unsigned char* sR = smem + Cf::Q_SR;
  float* zf = reinterpret_cast<float*>(smem + Cf::Q_ZF);
  unsigned char* atile = smem + Cf::Q_AT;
  unsigned char* rqtile = smem + Cf::Q_RQ;
  float2* ltab = reinterpret_cast<float2*>(smem + Cf::Q_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int m = lane >> 4;
  const int col = lane & 15;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int c = blockIdx.y;
  // strided walk: ranges of 16 NW tokens c, c + nsub, ...
  const int nsub = gridDim.y;
  const int n_begin = 16 * NW * c, n_end = a.N, wstride = 16 * NW * nsub;

  TabView tv{};
  {
    RowStage<D, D, NT> st_s;      // S^T rows
    RowStage<D, 2, NT, D> st_z;   // z hi and lo rows
    RowStage<D, D, NT> st_r;      // S rows
    const uint16_t* sl = a.sl + (size_t)bh * (D + 2) * D;
    st_s.load(sl);
    st_z.load(sl);
    st_r.load(a.sl2 + (size_t)bh * D * D);
    const float zv = tid < D ? bw.z[(size_t)bh * D + tid] : 0.f;
    if (ROPE) {
      if (TLDS) {
        copy_table_to_lds<NT, 8, false>(ltab, a.cs, a.T * a.Pt + a.Hh * a.Py + a.W * a.Px);
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
    st_r.store(sR);
    if (tid < D) zf[tid] = zv;
  }
  __syncthreads();
  // the lane's own z features, for dden z (registers: the masked sums below
  // then compile to selects instead of a branch around each LDS read)
  float zl[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) zl[j] = zf[MB * col + j];

  const size_t boff = (size_t)b * a.N * a.H * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(bw.dout + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(bw.dq + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rdg = make_rsrc(bw.dg + boff, a.slab_bytes);
  const uint32_t tokstride = (uint32_t)a.H * D * 2;
  const uint32_t qoff = (uint32_t)h * D * 2 + 16u * m;            // A operand chunk
  const uint32_t roff = (uint32_t)h * D * 2 + (uint32_t)OB * col;  // owned row bytes

  auto q_offset = [&](int base) -> uint32_t {
    const int n = base + col;
    return (n < n_end) ? (uint32_t)n * tokstride + qoff : kOob;
  };
  auto r_offset = [&](int base, int i) -> uint32_t {
    const int n = base + 4 * m + i;
    return (n < n_end) ? (uint32_t)n * tokstride + roff : kOob;
  };

  u32x4 qv[KS];
  OChunk gv[4], dv[4], qc[4];
  auto issue_q = [&](int base) {
    const uint32_t o = q_offset(base);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) qv[s2] = load16(rq, o + 64u * s2);
  };
  auto issue_gd = [&](int base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = r_offset(base, i);
      gv[i] = load_chunk<OB>(rg, o);
      dv[i] = load_chunk<OB>(rdo, o);
    }
  };
  auto issue_qc = [&](int base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) qc[i] = load_chunk<OB>(rq, r_offset(base, i));
  };

  float dzacc[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) dzacc[j] = 0.f;
  f32x16 dsacc[Cf::TPW];
#pragma unroll
  for (int t = 0; t < Cf::TPW; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dsacc[t][r] = 0.f;

  // this wave's rows of the two tiles
  unsigned char* my_a = atile + 16 * wave * TP;
  unsigned char* my_rq = rqtile + 16 * wave * TP;

  // QR (D = 128): q is loaded as whole rows only; its A operand comes from
  // the rows through the wave's a-tile rows (free until this step writes a),
  // which also keep the row chunks for the dq mask and dz until then
  constexpr bool QR = D == 128;
  int base = n_begin + 16 * wave;
  if (!QR) issue_q(base);
  issue_gd(base);
  issue_qc(base);
  wait_vmem_all();
  for (int bs = n_begin; bs < n_end; bs += wstride, base += wstride) {
    const int next = base + wstride;
    __builtin_amdgcn_sched_barrier(0);
    RowOff rof{};
    if (ROPE) {
      int t, y, x;
      grid_pos(a, (uint32_t)min(base + col, n_end - 1), t, y, x);
      rof = row_offsets<D>(a, tv, t, y, x);
    }
    if constexpr (QR) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<OChunk*>(my_a + (4 * m + i) * TP + OB * col) = qc[i];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        qv[s2] = *reinterpret_cast<const u32x4*>(my_a + col * TP + 16 * (4 * s2 + m));
      issue_qc(next);
    }
    // den: phi(q) against z_hi (even lane columns) and z_lo (odd ones)
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
    if (!QR) issue_q(next);
    // R phi(q) of token col, features 32 s + 8 m .. + 7, into the rq tile
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      *reinterpret_cast<bf16x8*>(my_rq + col * TP + 16 * (4 * s2 + m)) = Aq[s2];
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[MB];
    contract_rows<D>(sS, Aq, col, m, acc);

    // QR: the q row chunks back from the a tile before a overwrites them
    OChunk qk[4];
    if constexpr (QR) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qk[i] = *reinterpret_cast<const OChunk*>(my_a + (4 * m + i) * TP + OB * col);
    }
    // dg, a and the row sums of dout o
    float rden[4], part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float other = __int_as_float(
          __builtin_amdgcn_mov_dpp(__float_as_int(accd[i]), 0xB1, 0xF, 0xF, false));
      rden[i] = __builtin_amdgcn_rcpf((accd[i] + other) + kEps);
      part[i] = 0.f;
      OChunk wa, wg;
#pragma unroll
      for (int w = 0; w < OB / 4; ++w) {
        float av[2], gvv[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int j = 2 * w + hlf;
          const float gval = hlf ? bf_hi(gv[i][w]) : bf_lo(gv[i][w]);
          const float dval = hlf ? bf_hi(dv[i][w]) : bf_lo(dv[i][w]);
          const float e = __expf(-gval);
          const float s = __builtin_amdgcn_rcpf(1.f + e);
          const float ai = dval * s * rden[i];
          const float t = ai * acc[j][i];  // dout * o
          part[i] += t;
          av[hlf] = ai;
          gvv[hlf] = t * (e * s);           // dout * o * (1 - s)
        }
        wa[w] = pack_bf16(av[0], av[1]);
        wg[w] = pack_bf16(gvv[0], gvv[1]);
      }
      store_chunk_nt<OB>(rdg, r_offset(base, i), wg);
      *reinterpret_cast<OChunk*>(my_a + (4 * m + i) * TP + OB * col) = wa;
    }
    issue_gd(next);
    __builtin_amdgcn_sched_barrier(0);

    float dden[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dden[i] = -row_sum16(part[i]) * rden[i];

    // a in the A-operand layout (the LDS runs one wave's accesses in order)
    asm volatile("" ::: "memory");
    bf16x8 Aa[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      Aa[s2] = *reinterpret_cast<const bf16x8*>(my_a + col * TP + 16 * (4 * s2 + m));
    f32x4 acc2[MB];
    contract_rows<D>(sR, Aa, col, m, acc2);

    // dq = [q > 0] (R^T (S a) + dden z); dz += dden phi(q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float2 cs[PU];
      if (ROPE) acc_factors<D>(a, tv, min(base + 4 * m + i, n_end - 1), col, cs);
      OChunk wq;
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const float x = acc2[2 * u][i], y = acc2[2 * u + 1][i];
        float xr = x, yr = y;
        if (ROPE) {
          xr = x * cs[u].x + y * cs[u].y;
          yr = y * cs[u].x - x * cs[u].y;
        }
        const float q0 = bf_lo(QR ? qk[i][u] : qc[i][u]), q1 = bf_hi(QR ? qk[i][u] : qc[i][u]);
        const float g0 = q0 > 0.f ? xr + dden[i] * zl[2 * u] : 0.f;
        const float g1 = q1 > 0.f ? yr + dden[i] * zl[2 * u + 1] : 0.f;
        dzacc[2 * u] += dden[i] * fmaxf(q0, 0.f);
        dzacc[2 * u + 1] += dden[i] * fmaxf(q1, 0.f);
        wq[u] = pack_bf16(g0, g1);
      }
      store_chunk_nt<OB>(rdq, r_offset(base, i), wq);
    }
    if (!QR) issue_qc(next);
    __builtin_amdgcn_sched_barrier(0);

    // dS += rq a^T over the block step's 16 NW tokens
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < NW; ++ks) {
      const unsigned char* rt = rqtile + 16 * ks * TP;
      const unsigned char* at = atile + 16 * ks * TP;
#pragma unroll
      for (int t = 0; t < Cf::TPW; ++t) {
        const int ti = wave + NW * t;
        if (Cf::NTI % NW == 0 || ti < Cf::NTI) {
          const bf16x8 A = frag_tr(rt, TP, ti / (D / 32), lane);
          const bf16x8 B = frag_tr(at, TP, ti % (D / 32), lane);
          dsacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, dsacc[t], 0, 0, 0);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // the block's dS partial: element (d, e) of tile ti at row 32 (ti / (D/32)) + d
  float* dst = bw.dsp + ((size_t)bh * bw.C2 + c) * (size_t)(D * D + D);
#pragma unroll
  for (int t = 0; t < Cf::TPW; ++t) {
    const int ti = wave + NW * t;
    if (Cf::NTI % NW == 0 || ti < Cf::NTI) {
      const int ib = ti / (D / 32), jb = ti % (D / 32);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * ib + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        dst[d * D + 32 * jb + (lane & 31)] = dsacc[t][r];
      }
    }
  }
  // dz of the block: lanes of one column hold the same features; then the
  // waves in order
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    dzacc[j] += __shfl_xor(dzacc[j], 16);
    dzacc[j] += __shfl_xor(dzacc[j], 32);
  }
  float* zw = reinterpret_cast<float*>(atile);  // free after the last barrier
  if (m == 0) {
#pragma unroll
    for (int j = 0; j < MB; ++j) zw[wave * D + MB * col + j] = dzacc[j];
  }
  __syncthreads();
  if (tid < D) {
    float sum = zw[tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += zw[w * D + tid];
    dst[D * D + tid] = sum;
  }
}

// Key kernel.  Block = 4 waves, one (head, c) of grid (B H, C2): the two
// operands, the k and v tiles and the table take most of the LDS, so one block per
// compute unit, one wave per SIMD (measured faster than 8 waves, two per
// SIMD: 500.7 against 519.1 us per backward pass at 5B 720p/193f).  The block
// walks the head's 64-token ranges c, c + C2, ...
// LDS holds the head's dS^T and dS row operands and fp32 dz.  Per 16-token
// step: R phi(k) against dS^T gives dv; v (as loaded) against dS rows gives
// dS v, rotated back by R^T, plus dz, masked by k > 0: dk.
template <int D, bool ROPE, bool TLDS>
__global__ __launch_bounds__(64 * kKeyWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_key_kernel(KArgs a, BArgs bw) {
  using Cf = BwdCfg<D>;
  constexpr int KS = Cf::KS, MB = Cf::MB, OB = Cf::OB, PU = Cf::PU;
  constexpr int NW = kKeyWaves, NT = 64 * NW;
  using OChunk = typename Chunk<OB>::T;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // KROWS: k and v are loaded as whole token rows only (four rows per load
  // instruction) and turned into the A-operand layout through a per-wave LDS
  // tile, so k is read once and no load covers partial rows
  constexpr bool KROWS = D == 128;
  unsigned char* sD = smem;
  unsigned char* sR = smem + Cf::K_SR;
  float* zf = reinterpret_cast<float*>(smem + Cf::K_ZF);
  float2* ltab = reinterpret_cast<float2*>(smem + Cf::K_BYTES + (KROWS ? Cf::K_TILES : 0));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int m = lane >> 4;
  const int col = lane & 15;
  unsigned char* myk = smem + Cf::K_BYTES + wave * 2 * Cf::K_TILE;  // KROWS: the wave's tiles
  unsigned char* myv = myk + Cf::K_TILE;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int nsub = gridDim.y;
  const int n_begin = 16 * NW * blockIdx.y, n_end = a.N, wstride = 16 * NW * nsub;

  TabView tv{};
  {
    RowStage<D, D, NT> st_d;   // dS^T rows
    RowStage<D, D, NT> st_r;   // dS rows
    st_d.load(a.sl + (size_t)bh * (D + 2) * D);
    st_r.load(a.sl2 + (size_t)bh * D * D);
    const float zv = tid < D ? bw.dz[(size_t)bh * D + tid] : 0.f;
    if (ROPE) {
      if (TLDS) {
        copy_table_to_lds<NT, 8, false>(ltab, a.cs, a.T * a.Pt + a.Hh * a.Py + a.W * a.Px);
        tv.tab = ltab;
      } else {
        tv.tab = a.cs;
      }
      tv.tbase = 0;
      tv.ntr = a.T;
      tv.t_last = a.T - 1;
    }
    st_d.store(sD);
    st_r.store(sR);
    if (tid < D) zf[tid] = zv;
  }
  __syncthreads();
  // the lane's own dz features (registers, as in the query kernel)
  float zl[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) zl[j] = zf[MB * col + j];

  const size_t boff = (size_t)b * a.N * a.H * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rdk = make_rsrc(bw.dk + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rdv = make_rsrc(bw.dv + boff, a.slab_bytes);
  const uint32_t tokstride = (uint32_t)a.H * D * 2;
  const uint32_t koff = (uint32_t)h * D * 2 + 16u * m;
  const uint32_t roff = (uint32_t)h * D * 2 + (uint32_t)OB * col;

  auto a_offset = [&](int base) -> uint32_t {
    const int n = base + col;
    return (n < n_end) ? (uint32_t)n * tokstride + koff : kOob;
  };
  auto r_offset = [&](int base, int i) -> uint32_t {
    const int n = base + 4 * m + i;
    return (n < n_end) ? (uint32_t)n * tokstride + roff : kOob;
  };

  if constexpr (KROWS) {
    OChunk kc[4], vc[4];
    auto issue_rows = [&](int base) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t o = r_offset(base, i);
        kc[i] = load_chunk<OB>(rk, o);
        vc[i] = load_chunk<OB>(rv, o);
      }
    };
    int base = n_begin + 16 * wave;
    issue_rows(base);
    wait_vmem_all();
    for (; base < n_end; base += wstride) {
      const int next = base + wstride;
      __builtin_amdgcn_sched_barrier(0);
      // rows 4 m + i into the wave's tiles, then token col's operand chunks
      // back (the wave's LDS accesses execute in order)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<OChunk*>(myk + row_tile_offset<D>(4 * m + i, OB * col)) = kc[i];
        *reinterpret_cast<OChunk*>(myv + row_tile_offset<D>(4 * m + i, OB * col)) = vc[i];
      }
      u32x4 kv[KS], vv[KS];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        kv[s2] = *reinterpret_cast<const u32x4*>(myk + row_tile_offset<D>(col, 16 * (4 * s2 + m)));
        vv[s2] = *reinterpret_cast<const u32x4*>(myv + row_tile_offset<D>(col, 16 * (4 * s2 + m)));
      }
      issue_rows(next);
      __builtin_amdgcn_sched_barrier(0);
      RowOff rof{};
      if (ROPE) {
        int t, y, x;
        grid_pos(a, (uint32_t)min(base + col, n_end - 1), t, y, x);
        rof = row_offsets<D>(a, tv, t, y, x);
      }
      bf16x8 Ak[KS];
      static_for<KS>([&](auto S2) {
        constexpr int s2 = decltype(S2)::value;
        u32x4 fk;
#pragma unroll
        for (int u = 0; u < 4; ++u) fk[u] = relu2(kv[s2][u]);
        Ak[s2] = __builtin_bit_cast(bf16x8, ROPE ? rope_chunk<D, s2>(fk, tv, rof, m) : fk);
      });
      f32x4 acc[MB];
      contract_rows<D>(sD, Ak, col, m, acc);
      bf16x8 Av[KS];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) Av[s2] = __builtin_bit_cast(bf16x8, vv[s2]);
      f32x4 acc2[MB];
      contract_rows<D>(sR, Av, col, m, acc2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        OChunk wv;
#pragma unroll
        for (int w = 0; w < OB / 4; ++w) wv[w] = pack_bf16(acc[2 * w][i], acc[2 * w + 1][i]);
        store_chunk_nt<OB>(rdv, r_offset(base, i), wv);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the row chunk of k again, from the tile, for the k > 0 mask
        const OChunk kr = *reinterpret_cast<const OChunk*>(myk + row_tile_offset<D>(4 * m + i, OB * col));
        float2 cs[PU];
        if (ROPE) acc_factors<D>(a, tv, min(base + 4 * m + i, n_end - 1), col, cs);
        OChunk wk;
#pragma unroll
        for (int u = 0; u < PU; ++u) {
          const float x = acc2[2 * u][i], y = acc2[2 * u + 1][i];
          float xr = x, yr = y;
          if (ROPE) {
            xr = x * cs[u].x + y * cs[u].y;
            yr = y * cs[u].x - x * cs[u].y;
          }
          const float k0 = bf_lo(kr[u]), k1 = bf_hi(kr[u]);
          const float g0 = k0 > 0.f ? xr + zl[2 * u] : 0.f;
          const float g1 = k1 > 0.f ? yr + zl[2 * u + 1] : 0.f;
          wk[u] = pack_bf16(g0, g1);
        }
        store_chunk_nt<OB>(rdk, r_offset(base, i), wk);
      }
    }
    return;
  } else {
  u32x4 kv[KS], vv[KS];
  OChunk kc[4];
  auto issue_k = [&](int base) {
    const uint32_t o = a_offset(base);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) kv[s2] = load16(rk, o + 64u * s2);
  };
  auto issue_v = [&](int base) {
    const uint32_t o = a_offset(base);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) vv[s2] = load16(rv, o + 64u * s2);
  };
  auto issue_kc = [&](int base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kc[i] = load_chunk<OB>(rk, r_offset(base, i));
  };

  int base = n_begin + 16 * wave;
  issue_k(base);
  issue_v(base);
  issue_kc(base);
  wait_vmem_all();
  for (; base < n_end; base += wstride) {
    const int next = base + wstride;
    __builtin_amdgcn_sched_barrier(0);
    RowOff rof{};
    if (ROPE) {
      int t, y, x;
      grid_pos(a, (uint32_t)min(base + col, n_end - 1), t, y, x);
      rof = row_offsets<D>(a, tv, t, y, x);
    }
    bf16x8 Ak[KS];
    static_for<KS>([&](auto S2) {
      constexpr int s2 = decltype(S2)::value;
      u32x4 fk;
#pragma unroll
      for (int u = 0; u < 4; ++u) fk[u] = relu2(kv[s2][u]);
      Ak[s2] = __builtin_bit_cast(bf16x8, ROPE ? rope_chunk<D, s2>(fk, tv, rof, m) : fk);
    });
    issue_k(next);
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[MB];
    contract_rows<D>(sD, Ak, col, m, acc);
    bf16x8 Av[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) Av[s2] = __builtin_bit_cast(bf16x8, vv[s2]);
    f32x4 acc2[MB];
    contract_rows<D>(sR, Av, col, m, acc2);
    issue_v(next);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      OChunk wv;
#pragma unroll
      for (int w = 0; w < OB / 4; ++w) wv[w] = pack_bf16(acc[2 * w][i], acc[2 * w + 1][i]);
      store_chunk_nt<OB>(rdv, r_offset(base, i), wv);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float2 cs[PU];
      if (ROPE) acc_factors<D>(a, tv, min(base + 4 * m + i, n_end - 1), col, cs);
      OChunk wk;
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        const float x = acc2[2 * u][i], y = acc2[2 * u + 1][i];
        float xr = x, yr = y;
        if (ROPE) {
          xr = x * cs[u].x + y * cs[u].y;
          yr = y * cs[u].x - x * cs[u].y;
        }
        const float k0 = bf_lo(kc[i][u]), k1 = bf_hi(kc[i][u]);
        const float g0 = k0 > 0.f ? xr + zl[2 * u] : 0.f;
        const float g1 = k1 > 0.f ? yr + zl[2 * u + 1] : 0.f;
        wk[u] = pack_bf16(g0, g1);
      }
      store_chunk_nt<OB>(rdk, r_offset(base, i), wk);
    }
    issue_kc(next);
  }
  }
}

template <auto K>
hipError_t launch_rows_kernel(const Plan& p, const KArgs& a, const BArgs& b, int threads,
                              size_t lds, hipStream_t stream) {
  hipError_t e = allow_lds<K>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(K, dim3(p.BH, p.C2), dim3(threads), lds, stream, a, b);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_query_d(const Plan& p, const KArgs& a, const BArgs& b, hipStream_t s) {
  // the table goes to LDS when it fits beside the operands and the two tiles
  // (160 KB per compute unit); otherwise the kernel reads it from memory
  const size_t tbw = 8 * ((size_t)a.T * a.Pt + (size_t)a.Hh * a.Py + (size_t)a.W * a.Px);
  const bool tl = a.cs && BwdCfg<D>::Q_BYTES + tbw <= 160 * 1024;
  const size_t lds = BwdCfg<D>::Q_BYTES + (tl ? tbw : 0);
  constexpr int T = 64 * kQueryWaves;
  if (!a.cs) return launch_rows_kernel<bwd_query_kernel<D, false, false>>(p, a, b, T, lds, s);
  if (tl) return launch_rows_kernel<bwd_query_kernel<D, true, true>>(p, a, b, T, lds, s);
  return launch_rows_kernel<bwd_query_kernel<D, true, false>>(p, a, b, T, lds, s);
}

template <int D>
hipError_t launch_bwd_key_d(const Plan& p, const KArgs& a, const BArgs& b, hipStream_t s) {
  const size_t tbw = 8 * ((size_t)a.T * a.Pt + (size_t)a.Hh * a.Py + (size_t)a.W * a.Px);
  const size_t fixed = BwdCfg<D>::K_BYTES + (D == 128 ? BwdCfg<D>::K_TILES : 0);
  const bool tl = a.cs && fixed + tbw <= 160 * 1024;
  const size_t lds = fixed + (tl ? tbw : 0);
  constexpr int T = 64 * kKeyWaves;
  if (!a.cs) return launch_rows_kernel<bwd_key_kernel<D, false, false>>(p, a, b, T, lds, s);
  if (tl) return launch_rows_kernel<bwd_key_kernel<D, true, true>>(p, a, b, T, lds, s);
  return launch_rows_kernel<bwd_key_kernel<D, true, false>>(p, a, b, T, lds, s);
}

}  // namespace

hipError_t launch_bwd_query(const Plan& p, KArgs a, BArgs b, hipStream_t stream) {
  switch (p.D) {
    case 32: return launch_bwd_query_d<32>(p, a, b, stream);
    case 64: return launch_bwd_query_d<64>(p, a, b, stream);
    case 128: return launch_bwd_query_d<128>(p, a, b, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_key(const Plan& p, KArgs a, BArgs b, hipStream_t stream) {
  switch (p.D) {
    case 32: return launch_bwd_key_d<32>(p, a, b, stream);
    case 64: return launch_bwd_key_d<64>(p, a, b, stream);
    case 128: return launch_bwd_key_d<128>(p, a, b, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gla
