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
// K rows are padded to 4 (mod 64) dwords (16 rows of one 16-byte column hit
// distinct banks); V rows to 16 or 48 (mod 64) dwords, as the transposing
// reads want.
template <int D>
struct FaCfg {
  static constexpr int QB = 128;   // queries per block
  static constexpr int KT = 64;    // keys per tile
  static constexpr int KS = D / 16;  // k-steps of the scores
  static constexpr int ND = D / 32;  // 32-dim tiles of O^T
  static constexpr int KP = 2 * D + 16;
  static constexpr int VP = tile_pitch(2 * D);
  static constexpr int K_BYTES = KT * KP;
  static constexpr int STAGE = K_BYTES + KT * VP;
  static_assert((KP / 4) % 64 == 4 || (KP / 4) % 64 == 36, "K pitch");
  static_assert(K_BYTES % 1024 == 0 && (KT * VP) % 1024 == 0, "whole 64-slot DMA groups");
  // a running maximum that trails a tile's maximum by at most this much (in
  // log2 units) is kept: the weights stay below 2^8, and the accumulators
  // are rescaled only when the maximum really moves
  static constexpr float kLazyMax = 8.f;
};

// Transposing read of the V operand: rows 16 s + 4 G + j (first read) and
// 16 s + 8 + 4 G + j (second), G = l / 32, j < 4; columns 32 i + l % 32.
__device__ __forceinline__ bf16x8 frag_tr_keys(const unsigned char* tile, int pitch, int i, int s2,
                                               int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int f = 32 * i + 16 * (g & 1) + 4 * (s & 3);
  const int row = 16 * s2 + 4 * (g >> 1) + (s >> 2);
  const unsigned char* p0 = tile + row * pitch + 2 * f;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * pitch));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

typedef __attribute__((address_space(3))) void lds_void;

// One KT x D tile of a [B, N, H, D] tensor into LDS rows of PITCH bytes by
// buffer loads that write LDS directly: load I of the tile fills the 64
// 16-byte slots 64 I .. 64 I + 63 (lane i writes slot 64 I + i, at the
// uniform base the instruction takes); a slot past a row's D / 8 chunks is
// row padding and rows past N load zeros.  Completion is tracked by vmcnt.
template <int D, int PITCH>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int n0, int N,
                                         uint32_t tokstride, uint32_t headoff, int wave,
                                         int lane) {
  constexpr int SPR = PITCH / 16;                 // slots per row
  constexpr int LOADS = FaCfg<D>::KT * SPR / 64;  // 64-slot groups per tile
#pragma unroll
  for (int I = wave; I < LOADS; I += 4) {
    const int slot = 64 * I + lane;
    const int row = slot / SPR, ch = slot - (slot / SPR) * SPR;
    const int n = n0 + row;
    const uint32_t off = (ch < D / 8 && n < N) ? (uint32_t)n * tokstride + headoff + 16u * ch : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 1024 * I), 16, off, 0, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void flash_kernel(KArgs a, const uint16_t* qr, const uint16_t* kr) {
  using Cf = FaCfg<D>;
  constexpr int KS = Cf::KS, ND = Cf::ND;
  // two stage buffers as distinct objects: the compiler then sees that a
  // tile's reads never touch the buffer the next tile is loading into, and
  // does not wait for those loads before reading
  __shared__ __attribute__((aligned(16))) unsigned char stage0[Cf::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char stage1[Cf::STAGE];
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
  bf16x8 Qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) Qf[s] = __builtin_bit_cast(bf16x8, load16(rq, qoff + 32u * s));

  // K and V tiles go straight to LDS (no staging registers): the next tile's
  // loads are issued at the start of a tile and waited for at its end
  auto load_tile = [&](int j, unsigned char* st) {
    dma_tile<D, Cf::KP>(rk, st, j * Cf::KT, a.N, tokstride, headoff, wave, lane);
    dma_tile<D, Cf::VP>(rv, st + Cf::K_BYTES, j * Cf::KT, a.N, tokstride, headoff, wave, lane);
  };

  f32x16 acc_o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  auto tile = [&](int j, const unsigned char* kt, unsigned char* next) {
    const unsigned char* vt = kt + Cf::K_BYTES;
    load_tile(j + 1, next);   // past the last tile: zeros, never read

    // scores of keys 32 t + (8 (r/4) + 4 G + r % 4), t = 0, 1; the K
    // fragments of k-step s + 1 are read while step s multiplies
    f32x16 s_acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_acc[t][r] = 0.f;
    bf16x8 kf[2][2];
    auto read_k = [&](int s, bf16x8 (&dst)[2]) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        dst[t] = *reinterpret_cast<const bf16x8*>(kt + (32 * t + col) * Cf::KP + 32 * s + 16 * G);
    };
    read_k(0, kf[0]);
    static_for<KS>([&](auto S) {
      constexpr int s = decltype(S)::value;
      if constexpr (s + 1 < KS) read_k(s + 1, kf[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        s_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s & 1][t], Qf[s], s_acc[t], 0, 0, 0);
    });
    // keys past N take no weight
    const int kbase = j * Cf::KT;
    if (kbase + Cf::KT > a.N) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + 32 * t + 8 * (r >> 2) + 4 * G + (r & 3) >= a.N) s_acc[t][r] = -INFINITY;
    }
    float mt = s_acc[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s_acc[t][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // the running maximum moves (and the accumulators are rescaled) only
    // when some query's tile maximum passes it by more than kLazyMax
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
    float psum = 0.f;
    bf16x8 Pb[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int t = s2 >> 1, r0 = 8 * (s2 & 1);
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p0 = __builtin_amdgcn_exp2f(s_acc[t][r0 + 2 * k] - m_run);
        const float p1 = __builtin_amdgcn_exp2f(s_acc[t][r0 + 2 * k + 1] - m_run);
        psum += p0 + p1;
        w[k] = pack_bf16(p0, p1);
      }
      Pb[s2] = __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
    }
    l_run += psum;

#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        const bf16x8 vf = frag_tr_keys(vt, Cf::VP, i, s2, lane);
        acc_o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, Pb[s2], acc_o[i], 0, 0, 0);
      }
    // the next tile is in LDS and every wave is done with this one (the
    // compiler sees this wait, so it does not wait again before reading)
    __syncthreads();
  };

  const int ntiles = (a.N + Cf::KT - 1) / Cf::KT;
  load_tile(0, stage0);
  __syncthreads();
  // two tiles per trip, so each names its buffers statically; an odd count
  // runs one more tile whose keys all lie past N (masked: no weight)
  for (int j = 0; j < ntiles; j += 2) {
    tile(j, stage0, stage1);
    tile(j + 1, stage1, stage0);
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
