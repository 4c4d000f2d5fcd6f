// gla_softmax.hip -- gfx950 kernels of the gated softmax anchor attention
// ("SANA-Video 2.0", NVlabs Sana docs, section Architecture: a quarter of
// the layers are dense softmax anchors, 10 heads x 256 at 5B and 16 x 256 at
// 14B, with Wan 3D rotary embeddings; "SANA-Video 2.0: Hybrid Linear
// Attention with Attention Residuals for Efficient Video Generation"
// (mlsanity index), Abstract: periodic gated-softmax anchors).  Per head,
// with no mask:
//     o_n = sigmoid(g_n) * sum_m softmax_m(R_n q_n . R_m k_m / sqrt(D)) v_m
//
//   prep kernel   rotates q (scaled by log2(e) / sqrt(D), so that the
//                 softmax runs on exp2) and k once, into bf16 copies;
//   flash kernel  streams 64-key tiles of the rotated keys and the values
//                 through LDS for blocks of 128 queries, with an online
//                 softmax in fp32, and applies the gate at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {
namespace {

// ---------------------------------------------------------------------------
// Prep kernel: one thread per 16-byte chunk (4 rotation pairs) of one
// (b, n, h) row of q and of k.  The table is read from global memory (it is
// small and stays in the caches); rope == nullptr copies (q scaled).
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void softmax_prep_kernel(KArgs a, uint16_t* qr, uint16_t* kr,
                                                           float qscale, long long chunks) {
  using X = Axes<D>;
  constexpr int CPR = D / 8;  // chunks per row
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= chunks) return;
  const long long unit = idx / CPR;      // (b * N + n) * H + h
  const int c = (int)(idx - unit * CPR);
  const int n = (int)((unit / a.H) % a.N);
  const size_t off = (size_t)unit * D + 8 * c;
  const u32x4 qv = *reinterpret_cast<const u32x4*>(a.q + off);
  const u32x4 kv = *reinterpret_cast<const u32x4*>(a.k + off);
  float2 cs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) cs[u] = make_float2(1.f, 0.f);
  if (ROPE) {
    int t, y, x;
    grid_pos(a, (uint32_t)n, t, y, x);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = 4 * c + u;
      int at;
      if (p < X::Pt)
        at = t * X::Pt + p;
      else if (p < X::Pt + X::Py)
        at = a.T * X::Pt + y * X::Py + (p - X::Pt);
      else
        at = a.T * X::Pt + a.Hh * X::Py + x * X::Px + (p - X::Pt - X::Py);
      cs[u] = a.cs[at];
    }
  }
  u32x4 qo, ko;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float q0 = bf_lo(qv[u]), q1 = bf_hi(qv[u]);
    const float k0 = bf_lo(kv[u]), k1 = bf_hi(kv[u]);
    qo[u] = pack_bf16((q0 * cs[u].x - q1 * cs[u].y) * qscale, (q0 * cs[u].y + q1 * cs[u].x) * qscale);
    ko[u] = pack_bf16(k0 * cs[u].x - k1 * cs[u].y, k0 * cs[u].y + k1 * cs[u].x);
  }
  *reinterpret_cast<u32x4*>(qr + off) = qo;
  *reinterpret_cast<u32x4*>(kr + off) = ko;
}

// ---------------------------------------------------------------------------
// Flash kernel.
//
// Block = 4 waves, 128 consecutive queries of one head (32 per wave).  For
// each 64-key tile (K and V loaded straight into LDS, double-buffered, the
// next tile's loads in flight during the current one):
//   scores    S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with the keys as the A
//             operand (K rows read straight from LDS) and the wave's queries
//             as the B operand (held in registers for the whole block).  The
//             accumulator then gives each lane one query (l % 32) and 16 of
//             the 32 keys of a sub-tile (rows 8 (r/4) + 4 (l/32) + r % 4),
//             so a query's maximum and sum need one cross-lane step (l^32);
//   softmax   online in fp32 on exp2 (q carries the log2(e) / sqrt(D) scale),
//             with a running maximum that may trail the true one by up to
//             kLazyMax (the same stale maximum scales the weights and their
//             sum, so the result is the same softmax);
//   values    O^T += V^T P^T with P^T as the B operand straight from the
//             score registers: in k-step s the lane's 8 keys are
//             16 s + 8 (k / 4) + 4 (l / 32) + k % 4, and the V operand is
//             read with ds_read_b64_tr_b16 from exactly those rows.  O^T's
//             accumulator again gives each lane one query, so the softmax
//             rescale is one scalar per lane.
//
// LDS layout of a 64-key tile.  One buffer-load-to-LDS instruction fills
// 1 KB: RPG whole rows (RPG = 64 lanes / (D / 8) 16-byte chunks per row).
// Such a group of rows is padded, and row q of a group stores its chunk c at
// position c ^ (SW q), so that the reads below hit distinct banks:
//   K  (16-byte reads of 16 consecutive rows, one chunk):  groups padded by
//      16 bytes, SW = 16 / RPG;
//   V  (transposing 8-byte reads of 4 consecutive rows, 64 bytes each):
//      SW = 4, groups padded to 128 (mod 256) bytes when a group is 2 rows.
// The XOR keeps every read offset a compile-time constant from one of RPG
// per-lane bases (the swizzled bits of c are known at compile time).
template <int D>
struct FaCfg {
  static constexpr int QB = 128;   // queries per block
  static constexpr int KT = 64;    // keys per tile
  static constexpr int KS = D / 16;  // k-steps of the scores
  static constexpr int ND = D / 32;  // 32-dim tiles of O^T
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static constexpr int RPG = 64 / CPR;  // rows per 1 KB load group
  static constexpr int GROUPS = KT / RPG;
  static constexpr int GPW = GROUPS / 4;  // load groups per wave and tensor
  static constexpr int KSW = 16 / RPG;
  static constexpr int VSW = 4;
  static constexpr int KG = RPG * 2 * D + 16;
  static constexpr int VG = RPG * 2 * D + (RPG == 2 ? 128 : 0);
  static constexpr int K_BYTES = GROUPS * KG;
  static constexpr int V_BYTES = GROUPS * VG;
  static_assert(GROUPS % 4 == 0 && KG % 16 == 0 && VG % 16 == 0, "load groups");
  // a running maximum that trails a tile's maximum by at most this much (in
  // log2 units) is kept: the weights stay below 2^8, and the accumulators
  // are rescaled only when the maximum really moves
  static constexpr int KPF = 2;    // k-steps the K fragment reads run ahead
  static constexpr float kLazyMax = 8.f;
  // how far (log2 units) a tile's maximum may pass the fixed reference of
  // the main pass: weights up to 2^64, sums over < 2^31 keys stay far below
  // the fp32 range
  static constexpr float kFixedSpan = 64.f;
};

typedef __attribute__((address_space(3))) void lds_void;

// This lane's part of the global offset of the chunk it loads in every group:
// row q = lane / CPR of the group, chunk (lane % CPR) ^ (SW q).
template <int D, int SW>
__device__ __forceinline__ uint32_t dma_lane_offset(int lane, uint32_t tokstride, uint32_t headoff) {
  constexpr int CPR = FaCfg<D>::CPR;
  const int q = lane / CPR, pc = lane % CPR;
  return (uint32_t)q * tokstride + headoff + 16u * (uint32_t)(pc ^ (SW * q));
}

// Group ii of the wave's GPW groups of one tensor's tile (keys n0 ..):
// group I = wave GPW + ii holds rows RPG I .. RPG I + RPG - 1 at dst + I GP.
// Rows past N lie outside the slab and load zeros.  Completion is tracked
// by vmcnt.
template <int D, int GP>
__device__ __forceinline__ void dma_group(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t lane_off,
                                          int n0, uint32_t tokstride, int wave, int ii) {
  using Cf = FaCfg<D>;
  const int I = wave * Cf::GPW + ii;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + I * GP), 16,
                                           lane_off + (uint32_t)(n0 + Cf::RPG * I) * tokstride, 0, 0, 0);
}

// All of the wave's groups of one tensor's tile.
template <int D, int GP>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t lane_off,
                                         int n0, uint32_t tokstride, int wave) {
#pragma unroll
  for (int ii = 0; ii < FaCfg<D>::GPW; ++ii) dma_group<D, GP>(r, dst, lane_off, n0, tokstride, wave, ii);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void flash_kernel(KArgs a, const uint16_t* qr, const uint16_t* kr) {
  using Cf = FaCfg<D>;
  constexpr int KS = Cf::KS, ND = Cf::ND;
  // two K and two V buffers as distinct objects: the compiler then sees that
  // a tile's reads never touch a buffer that a load is filling, and does not
  // wait for those loads before reading
  __shared__ __attribute__((aligned(16))) unsigned char kbuf0[Cf::K_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kbuf1[Cf::K_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf0[Cf::V_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf1[Cf::V_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5, col = lane & 31;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const size_t boff = (size_t)b * a.N * a.H * D;
  const uint32_t tokstride = (uint32_t)a.H * D * 2;
  const uint32_t headoff = (uint32_t)h * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qr + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kr + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + boff, a.slab_bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + boff, a.slab_bytes);

  // the wave's queries as the B operand: query q0 + col, dims 16 s + 8 G
  const int qn = blockIdx.x * Cf::QB + 32 * wave + col;
  const uint32_t qoff = qn < a.N ? (uint32_t)qn * tokstride + headoff + 16u * G : kOob;
  // they stay in accumulation registers (the MFMA reads its B operand from
  // there), which leaves the vector registers to the fragments in flight
  bf16x8 Qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const u32x4 v = load16(rq, qoff + 32u * s);
    uint32_t w0, w1, w2, w3;
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(w0) : "v"(v[0]));
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(w1) : "v"(v[1]));
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(w2) : "v"(v[2]));
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(w3) : "v"(v[3]));
    Qf[s] = __builtin_bit_cast(bf16x8, (u32x4){w0, w1, w2, w3});
  }

  // K and V tiles go straight to LDS (no staging registers)
  const uint32_t klane = dma_lane_offset<D, Cf::KSW>(lane, tokstride, headoff);
  const uint32_t vlane = dma_lane_offset<D, Cf::VSW>(lane, tokstride, headoff);
  auto load_k = [&](int j, unsigned char* dst) {
    dma_tile<D, Cf::KG>(rk, dst, klane, j * Cf::KT, tokstride, wave);
  };
  auto load_v = [&](int j, unsigned char* dst) {
    dma_tile<D, Cf::VG>(rv, dst, vlane, j * Cf::KT, tokstride, wave);
  };

  // LDS read bases.  K: row col (+ 32 t), chunk 2 s + G; base m serves the
  // chunks whose swizzled bits (c / KSW) % RPG equal m.
  constexpr int RPG = Cf::RPG;
  int kb[RPG];
  {
    const int q = col % RPG;
#pragma unroll
    for (int m = 0; m < RPG; ++m)
      kb[m] = (col / RPG) * Cf::KG + q * 2 * D + 16 * (G + Cf::KSW * (m ^ q));
  }
  // V, read transposed: this lane's 4 dims 32 i + 16 (g & 1) + 4 (l & 3) of
  // rows 16 s2 + 4 (g >> 1) + (l & 15) / 4 (and 8 rows on), g = l / 16;
  // base m serves the 32-dim tiles i with i % RPG == m.
  int vb[RPG];
  {
    const int g = lane >> 4, sl = lane & 15;
    const int r0 = 4 * (g >> 1) + (sl >> 2), q = r0 % RPG;
    const int clo = 2 * (g & 1) + ((sl >> 1) & 1);
#pragma unroll
    for (int m = 0; m < RPG; ++m)
      vb[m] = (r0 / RPG) * Cf::VG + q * 2 * D + 8 * (sl & 1) + 16 * (clo + Cf::VSW * (m ^ q));
  }

  auto read_v = [&](const unsigned char* vt, int i, int s2) {
    const unsigned char* p0 =
        vt + vb[i % RPG] + (16 * s2 / RPG) * Cf::VG + 16 * Cf::VSW * RPG * (i / RPG);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + (8 / RPG) * Cf::VG));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // scores of keys 32 t + (8 (r/4) + 4 G + r % 4), t = 0, 1, of the tile at
  // kt (key j * KT first), plus c0; keys past N score -inf.  io(s) runs at
  // k-step s (it issues loads).
  auto scores = [&](int j, const unsigned char* kt, const f32x16& c0, f32x16 (&s_acc)[2], auto&& io) {
    // the K fragments of k-step s + KPF are read while step s multiplies
    constexpr int KPF = Cf::KPF;
    bf16x8 kf[KPF + 1][2];
    auto read_k = [&](int s, bf16x8 (&dst)[2]) {
      const int c = 2 * s;  // the lane adds G
      const int off = 16 * (c % Cf::KSW + Cf::KSW * RPG * (c / (Cf::KSW * RPG)));
      const int base = kb[(c / Cf::KSW) % RPG];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        dst[t] = *reinterpret_cast<const bf16x8*>(kt + base + t * (32 / RPG) * Cf::KG + off);
    };
    static_for<KPF>([&](auto S) { read_k(decltype(S)::value, kf[decltype(S)::value]); });
    static_for<KS>([&](auto S) {
      constexpr int s = decltype(S)::value;
      if constexpr (s + KPF < KS) read_k(s + KPF, kf[(s + KPF) % (KPF + 1)]);
      io(S);
      asm volatile("" : "+a"(Qf[s]));  // read in place from the accumulation registers
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        s_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % (KPF + 1)][t], Qf[s], s == 0 ? c0 : s_acc[t],
                                                           0, 0, 0);
    });
    const int kbase = j * Cf::KT;
    if (kbase + Cf::KT > a.N) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + 32 * t + 8 * (r >> 2) + 4 * G + (r & 3) >= a.N) s_acc[t][r] = -INFINITY;
    }
  };

  // the query's maximum over the tile (both lanes of the query)
  auto tile_max = [&](const f32x16 (&s_acc)[2]) {
    float mt = s_acc[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s_acc[t][r]);
    return fmaxf(mt, __shfl_xor(mt, 32));
  };

  // weights exp2(s - m) as the B operands of the value MFMAs; returns their
  // sum over the lane's 32 keys
  auto weights = [&](const f32x16 (&s_acc)[2], float m, bf16x8 (&Pb)[4]) {
    float psum = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int t = s2 >> 1, r0 = 8 * (s2 & 1);
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p0 = __builtin_amdgcn_exp2f(s_acc[t][r0 + 2 * k] - m);
        const float p1 = __builtin_amdgcn_exp2f(s_acc[t][r0 + 2 * k + 1] - m);
        psum += p0 + p1;
        w[k] = pack_bf16(p0, p1);
      }
      Pb[s2] = __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
    }
    return psum;
  };

  f32x16 acc_o[ND];
  // O^T += V^T P^T over the tile's values at vt
  auto values = [&](const unsigned char* vt, const bf16x8 (&Pb)[4]) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
      for (int i = 0; i < ND; ++i)
        acc_o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v(vt, i, s2), Pb[s2], acc_o[i], 0, 0, 0);
  };

  const int ntiles = (a.N + Cf::KT - 1) / Cf::KT;
  f32x16 zero16;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero16[r] = 0.f;
  float l_run;

  // Main pass.  Every tile's weights are taken against one reference, tile
  // 0's maximum of the query, which enters the score MFMAs as their initial
  // accumulator, so the accumulators are never rescaled.  A tile whose
  // weights pass 2^64 on some lane (only possible when its maximum passes the
  // reference by more than 64 log2 units) flags the block, which then runs
  // the online-rescale pass.
  //   Tile j's value MFMAs run in tile j + 1, beside that tile's
  // exponentials.  Tile j loads K(j + 1) and V(j), one 1 KB group per score
  // k-step: K(j + 1) into the buffer K(j - 1) left in tile j - 1, V(j) into
  // the one V(j - 2) left there; its closing barrier waits for both.
  static_assert(KS == 2 * Cf::GPW, "one load group per score k-step");
  auto no_io = [](auto) {};
  load_k(0, kbuf0);
  dma_tile<D, Cf::VG>(rv, vbuf1, kOob, 0, tokstride, wave);  // V(-1): zeros
  __syncthreads();
  f32x16 cref;
  {
    f32x16 s_acc[2];
    scores(0, kbuf0, zero16, s_acc, no_io);
    const float m_ref = tile_max(s_acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) cref[r] = -m_ref;
  }
#pragma unroll
  for (int i = 0; i < ND; ++i) acc_o[i] = zero16;
  l_run = 0.f;
  bool over = false;
  bf16x8 Pp[4];  // the previous tile's weights (none before tile 0)
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) Pp[s2] = __builtin_bit_cast(bf16x8, (u32x4){0u, 0u, 0u, 0u});
  auto fixed_tile = [&](int j, const unsigned char* kcur, unsigned char* knext, unsigned char* vcur,
                        const unsigned char* vprev) {
    // past the last tile the loads read zeros, never used
    auto io = [&](auto S) {
      constexpr int st = decltype(S)::value;
      if constexpr (st < Cf::GPW)
        dma_group<D, Cf::KG>(rk, knext, klane, (j + 1) * Cf::KT, tokstride, wave, st);
      else
        dma_group<D, Cf::VG>(rv, vcur, vlane, j * Cf::KT, tokstride, wave, st - Cf::GPW);
    };
    f32x16 s_acc[2];
    scores(j, kcur, cref, s_acc, io);
    values(vprev, Pp);
    const float ps = weights(s_acc, 0.f, Pp);
    over |= !(ps <= 0x1p64f);
    l_run += ps;
    // the weights are due before the barrier, beside the value MFMAs (else
    // the compiler sinks them to their use in the next tile)
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) asm volatile("" ::"v"(Pp[s2]));
    // K(j + 1) and V(j) are in LDS, and every wave is done with K(j) and
    // V(j - 1) (the compiler sees this wait, so it does not wait again
    // before reading)
    __syncthreads();
  };
  // two tiles per trip, so each names its buffers statically; an odd count
  // runs one more tile whose keys all lie past N (masked: no weight)
  for (int j = 0; j < ntiles; j += 2) {
    fixed_tile(j, kbuf0, kbuf1, vbuf0, vbuf1);
    fixed_tile(j + 1, kbuf1, kbuf0, vbuf1, vbuf0);
  }
  values(vbuf1, Pp);  // the last tile's values (odd index: V buffer 1)
  __syncthreads();    // no load in flight

  if (__syncthreads_or(over)) {
    // Online-rescale pass: the running maximum moves (and the accumulators
    // are rescaled) only when some query's tile maximum passes it by more
    // than kLazyMax.
#pragma unroll
    for (int i = 0; i < ND; ++i) acc_o[i] = zero16;
    float m_run = -INFINITY;
    l_run = 0.f;
    auto lazy_tile = [&](int j, const unsigned char* kt, const unsigned char* vt, unsigned char* knext,
                         unsigned char* vnext) {
      load_k(j + 1, knext);
      load_v(j + 1, vnext);
      f32x16 s_acc[2];
      scores(j, kt, zero16, s_acc, no_io);
      const float mt = tile_max(s_acc);
      if (__any(mt > m_run + Cf::kLazyMax)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < ND; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[i][r] *= alpha;
      }
      bf16x8 Pb[4];
      l_run += weights(s_acc, m_run, Pb);
      values(vt, Pb);
      __syncthreads();
    };
    load_k(0, kbuf0);
    load_v(0, vbuf0);
    __syncthreads();
    for (int j = 0; j < ntiles; j += 2) {
      lazy_tile(j, kbuf0, vbuf0, kbuf1, vbuf1);
      lazy_tile(j + 1, kbuf1, vbuf1, kbuf0, vbuf0);
    }
  }

  // o = sigmoid(g) * O / l: lane holds query qn at dims 32 i + 8 (r/4) + 4 G + r % 4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  const uint32_t obase = qn < a.N ? (uint32_t)qn * tokstride + headoff : kOob;
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const uint32_t off = obase + 2u * (32 * i + 8 * r4 + 4 * G);
      const u32x2v gv = __builtin_amdgcn_raw_buffer_load_b64(rg, off, 0, 0);
      float o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float gk = (k & 1) ? bf_hi(gv[k >> 1]) : bf_lo(gv[k >> 1]);
        const float e = __expf(-gk);
        o[k] = acc_o[i][4 * r4 + k] * inv * __builtin_amdgcn_rcpf(1.f + e);
      }
      const u32x2v w = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
      __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, kCpolNt);
    }
}


template <int D>
hipError_t launch_softmax_d(const Plan& p, KArgs a, uint16_t* qr, uint16_t* kr,
                            hipStream_t stream) {
  const long long chunks = (long long)p.B * p.N * p.H * (D / 8);
  const float qscale = 1.4426950408889634f / __builtin_sqrtf((float)D);
  const dim3 gp((unsigned)((chunks + 255) / 256));
  if (a.cs)
    hipLaunchKernelGGL((softmax_prep_kernel<D, true>), gp, dim3(256), 0, stream, a, qr, kr, qscale,
                       chunks);
  else
    hipLaunchKernelGGL((softmax_prep_kernel<D, false>), gp, dim3(256), 0, stream, a, qr, kr,
                       qscale, chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  using Cf = FaCfg<D>;
  const dim3 gf((p.N + Cf::QB - 1) / Cf::QB, p.BH);
  hipLaunchKernelGGL((flash_kernel<D>), gf, dim3(256), 0, stream, a, qr, kr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax(const Plan& p, KArgs a, uint16_t* qr, uint16_t* kr, hipStream_t stream) {
  switch (p.D) {
    case 128: return launch_softmax_d<128>(p, a, qr, kr, stream);
    case 256: return launch_softmax_d<256>(p, a, qr, kr, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gla
