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
//                  and stores S as bf16 in the output kernel's operand layout;
//   output kernel  streams q and g, contracts R phi(q) with the LDS-resident S
//                  on bf16 MFMA (16x16x32), applies normaliser and gate, and
//                  writes bf16 out.
// All tensors are bf16 [B, N, H, D]; a head's D-vector of a token is 2D
// contiguous bytes, consecutive tokens are H*D*2 bytes apart.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_internal.h"

namespace gla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kEps = 1e-6f;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest-even) and pack them, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  __bf16 x = (__bf16)a;
  __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// (cos, sin) of rotation pair p for a token whose per-axis row offsets into
// the factorised table are ot, oy, ox (each already minus its axis's first pair).
__device__ __forceinline__ float2 rope_cs(const RopeArgs& r, int p, int ot, int oy, int ox) {
  int idx = (p < r.Pt) ? ot + p : ((p < r.Pt + r.Py) ? oy + p : ox + p);
  return r.cs[idx];
}

__device__ __forceinline__ void rope_rows(const RopeArgs& r, unsigned n, int& ot, int& oy, int& ox) {
  unsigned HW = (unsigned)(r.Hh * r.W);
  unsigned t = n / HW;
  unsigned rem = n - t * HW;
  unsigned y = rem / (unsigned)r.W;
  unsigned x = rem - y * (unsigned)r.W;
  ot = (int)t * r.Pt;
  oy = r.T * r.Pt + (int)y * r.Py - r.Pt;
  ox = r.T * r.Pt + r.Hh * r.Py + (int)x * r.Px - r.Pt - r.Py;
}

// ---------------------------------------------------------------------------
// State kernel.
//
// Block = 256 threads, one (chunk, head).  A tile holds TT = 8192/D tokens,
// so every thread loads 4 tokens x 16 bytes of k and of v per tile (thread t
// takes 16-byte chunk t % (D/8) of tokens 4*(t / (D/8)) + 0..3).  ReLU and
// RoPE are applied in fp32 registers, z accumulates the unrotated ReLU
// features, and R phi(k) (rounded to bf16) and v are written to LDS
// transposed -- one row per feature, tokens contiguous -- because both MFMA
// operands of S = sum_n rk_n v_n^T contract over tokens.  Rows are padded by
// 16 bytes and the 16-byte token units XOR-swizzled by (256/D)*(row/16) mod 8,
// which keeps both the transposed 8-byte writes and the 16-byte MFMA operand
// reads free of LDS bank conflicts.  The next tile's global loads are issued
// before the MFMA phase of the current one.
template <int D>
struct StateCfg {
  static constexpr int NC = D / 8;                 // 16-byte chunks per token vector
  static constexpr int TT = 8192 / D;              // tokens per tile
  static constexpr int ROWB = TT * 2 + 16;         // LDS row pitch, bytes
  static constexpr int UW = 256 / D;               // swizzle step
  static constexpr int RT = D / 32;                // 32x32 output tiles per dimension
  static constexpr int KSPLIT = (RT * RT >= 4) ? 1 : 4 / (RT * RT);
  static constexpr int WR = (RT >= 2) ? 2 : 1;     // wave grid over output tiles
  static constexpr int WC = (RT >= 2) ? 2 : 1;
  static constexpr int TR = RT / WR;               // output tiles per wave (rows, cols)
  static constexpr int TC = RT / WC;
  static constexpr int KSTEPS = TT / 16;
  static constexpr int NG = 256 / NC;              // token groups of 4 per tile
  static_assert(WR * WC * KSPLIT == 4, "four waves per block");
  static_assert(TT / 8 >= 8, "swizzle needs >= 8 token units per row");
};

template <int D>
__device__ __forceinline__ int lds_off(int row, int tok) {
  using Cf = StateCfg<D>;
  int f = (Cf::UW * (row >> 4)) & 7;
  return row * Cf::ROWB + ((((tok >> 3) ^ f)) << 4) + ((tok & 7) << 1);
}

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void state_kernel(const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v, int N, int H,
                                                    int L, int C, RopeArgs rope,
                                                    float* __restrict__ part) {
  using Cf = StateCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[D * Cf::ROWB];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v[D * Cf::ROWB];
  __shared__ float zred[Cf::NG * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int n_begin = c * L;
  const int n_end = min(N, n_begin + L);

  const size_t tok_stride = (size_t)H * D;
  const size_t head_base = ((size_t)b * N * H + h) * D;
  const uint16_t* kb = k + head_base;
  const uint16_t* vb = v + head_base;

  const int c8 = tid % Cf::NC;     // 16-byte chunk of the token vector
  const int grp = tid / Cf::NC;    // token group (4 tokens)

  // MFMA work split
  const int wk = wave % Cf::KSPLIT;
  const int wt = wave / Cf::KSPLIT;
  const int wr = wt / Cf::WC, wc = wt % Cf::WC;

  f32x16 acc[Cf::TR][Cf::TC];
#pragma unroll
  for (int a = 0; a < Cf::TR; ++a)
#pragma unroll
    for (int bb = 0; bb < Cf::TC; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][bb][r] = 0.f;

  float zacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zacc[j] = 0.f;

  uint4 kr[4], vr[4];
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int n = n0 + 4 * grp + i;
      if (n < n_end) {
        kr[i] = *reinterpret_cast<const uint4*>(kb + (size_t)n * tok_stride + 8 * c8);
        vr[i] = *reinterpret_cast<const uint4*>(vb + (size_t)n * tok_stride + 8 * c8);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  if (n_begin < n_end) load_tile(n_begin);

  for (int n0 = n_begin; n0 < n_end; n0 += Cf::TT) {
    // features of this thread's 4 tokens: rk[i][j] (bf16 bits), 8 features each
    uint16_t rkb[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
      float f[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        f[2 * u] = fmaxf(bf_lo(w[u]), 0.f);
        f[2 * u + 1] = fmaxf(bf_hi(w[u]), 0.f);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) zacc[j] += f[j];
      if (ROPE) {
        int n = n0 + 4 * grp + i;
        unsigned np = (unsigned)((n < n_end) ? n : n_begin);
        int ot, oy, ox;
        rope_rows(rope, np, ot, oy, ox);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float2 cs = rope_cs(rope, 4 * c8 + u, ot, oy, ox);
          float a0 = f[2 * u], a1 = f[2 * u + 1];
          f[2 * u] = a0 * cs.x - a1 * cs.y;
          f[2 * u + 1] = a0 * cs.y + a1 * cs.x;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t p = pack_bf16(f[2 * u], f[2 * u + 1]);
        rkb[i][2 * u] = (uint16_t)(p & 0xffffu);
        rkb[i][2 * u + 1] = (uint16_t)(p >> 16);
      }
    }

    __syncthreads();  // previous tile's MFMA reads are done
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 8 * c8 + j;
      const int off = lds_off<D>(row, 4 * grp);
      uint2 wk2, wv2;
      wk2.x = (uint32_t)rkb[0][j] | ((uint32_t)rkb[1][j] << 16);
      wk2.y = (uint32_t)rkb[2][j] | ((uint32_t)rkb[3][j] << 16);
      uint32_t vw[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vw[i][0] = vr[i].x; vw[i][1] = vr[i].y; vw[i][2] = vr[i].z; vw[i][3] = vr[i].w;
      }
      uint16_t v0 = (uint16_t)((j & 1) ? (vw[0][j >> 1] >> 16) : (vw[0][j >> 1] & 0xffffu));
      uint16_t v1 = (uint16_t)((j & 1) ? (vw[1][j >> 1] >> 16) : (vw[1][j >> 1] & 0xffffu));
      uint16_t v2 = (uint16_t)((j & 1) ? (vw[2][j >> 1] >> 16) : (vw[2][j >> 1] & 0xffffu));
      uint16_t v3 = (uint16_t)((j & 1) ? (vw[3][j >> 1] >> 16) : (vw[3][j >> 1] & 0xffffu));
      wv2.x = (uint32_t)v0 | ((uint32_t)v1 << 16);
      wv2.y = (uint32_t)v2 | ((uint32_t)v3 << 16);
      *reinterpret_cast<uint2*>(lds_k + off) = wk2;
      *reinterpret_cast<uint2*>(lds_v + off) = wv2;
    }

    if (n0 + Cf::TT < n_end) load_tile(n0 + Cf::TT);
    __syncthreads();

#pragma unroll
    for (int ks = wk; ks < Cf::KSTEPS; ks += Cf::KSPLIT) {
      const int tok = 16 * ks + 8 * (lane >> 5);
      bf16x8 A[Cf::TR], Bv[Cf::TC];
#pragma unroll
      for (int a = 0; a < Cf::TR; ++a) {
        int row = 32 * (wr * Cf::TR + a) + (lane & 31);
        A[a] = *reinterpret_cast<const bf16x8*>(lds_k + lds_off<D>(row, tok));
      }
#pragma unroll
      for (int bb = 0; bb < Cf::TC; ++bb) {
        int row = 32 * (wc * Cf::TC + bb) + (lane & 31);
        Bv[bb] = *reinterpret_cast<const bf16x8*>(lds_v + lds_off<D>(row, tok));
      }
#pragma unroll
      for (int a = 0; a < Cf::TR; ++a)
#pragma unroll
        for (int bb = 0; bb < Cf::TC; ++bb)
          acc[a][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a], Bv[bb], acc[a][bb], 0, 0, 0);
    }
  }

  // z partial: sum the token groups in a fixed order
#pragma unroll
  for (int j = 0; j < 8; ++j) zred[grp * D + 8 * c8 + j] = zacc[j];

  float* dst = part + ((size_t)bh * C + c) * (size_t)(D * D + D);
  if (Cf::KSPLIT == 1) {
#pragma unroll
    for (int a = 0; a < Cf::TR; ++a)
#pragma unroll
      for (int bb = 0; bb < Cf::TC; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int d = 32 * (wr * Cf::TR + a) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          int e = 32 * (wc * Cf::TC + bb) + (lane & 31);
          dst[d * D + e] = acc[a][bb][r];
        }
    __syncthreads();
  } else {
    // the waves split the token steps of one 32x32 tile; add their results in wave order
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds_k);  // 4 waves x 16 x 64 floats = 16 KB
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[0][0][r];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = red[r * 64 + lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) s += red[(w * 16 + r) * 64 + lane];
        int d = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        int e = lane & 31;
        dst[d * D + e] = s;
      }
    }
  }
  if (tid < D) {
    float s = 0.f;
    for (int gi = 0; gi < Cf::NG; ++gi) s += zred[gi * D + tid];
    dst[D * D + tid] = s;
  }
}

// ---------------------------------------------------------------------------
// Reduce kernel: per head, S = sum_c S_c and z = sum_c z_c over the C chunk
// partials in a fixed pairwise tree (a binary counter merges equal-sized
// partial sums, older operand on the left), so the result does not depend on
// which block finished first.  S is stored as bf16 rows in the output
// kernel's operand order (row R(e) holds S[0..D)[e]); optional fp32 copies of
// S and z go to the caller.

constexpr int kTreeLevels = 9;  // handles C <= 256 = kMaxChunks

struct TreeSum {
  float st[kTreeLevels];
  int cnt;
  __device__ __forceinline__ TreeSum() : cnt(0) {
#pragma unroll
    for (int l = 0; l < kTreeLevels; ++l) st[l] = 0.f;
  }
  __device__ __forceinline__ void push(float x) {
#pragma unroll
    for (int l = 0; l < kTreeLevels; ++l) {
      if ((cnt >> l) & 1) {
        x = st[l] + x;
      } else {
        st[l] = x;
        break;
      }
    }
    ++cnt;
  }
  __device__ __forceinline__ float total() const {
    float s = 0.f;
    bool any = false;
#pragma unroll
    for (int l = 0; l < kTreeLevels; ++l) {
      if ((cnt >> l) & 1) {
        s = any ? st[l] + s : st[l];
        any = true;
      }
    }
    return s;
  }
};

// Output-kernel operand row of value column e (see output_kernel).
template <int D>
__device__ __forceinline__ int out_row_of(int e) {
  int j = 2 * (e >> 5) + ((e & 7) >> 2);
  int r = 4 * ((e & 31) >> 3) + (e & 3);
  return 16 * j + r;
}

template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, int C,
                                                     uint16_t* __restrict__ sl,
                                                     float* __restrict__ zf,
                                                     float* __restrict__ S_out,
                                                     float* __restrict__ z_out) {
  const int bh = blockIdx.y;
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const size_t pstride = (size_t)(D * D + D);
  const float* pb = part + (size_t)bh * C * pstride;
  constexpr int NS = D * D / 8;
  if (gid < NS) {
    const int e = gid % D;
    const int d8 = gid / D;
    TreeSum ts[8];
    for (int cc = 0; cc < C; ++cc) {
      const float* src = pb + cc * pstride + (size_t)(8 * d8) * D + e;
#pragma unroll
      for (int j = 0; j < 8; ++j) ts[j].push(src[j * D]);
    }
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = ts[j].total();
    uint4 w;
    w.x = pack_bf16(s[0], s[1]);
    w.y = pack_bf16(s[2], s[3]);
    w.z = pack_bf16(s[4], s[5]);
    w.w = pack_bf16(s[6], s[7]);
    *reinterpret_cast<uint4*>(sl + (size_t)bh * D * D + (size_t)out_row_of<D>(e) * D + 8 * d8) = w;
    if (S_out) {
#pragma unroll
      for (int j = 0; j < 8; ++j) S_out[(size_t)bh * D * D + (size_t)(8 * d8 + j) * D + e] = s[j];
    }
  } else if (gid < NS + D) {
    const int d = gid - NS;
    TreeSum ts;
    for (int cc = 0; cc < C; ++cc) ts.push(pb[cc * pstride + D * D + d]);
    float s = ts.total();
    zf[(size_t)bh * D + d] = s;
    if (z_out) z_out[(size_t)bh * D + d] = s;
  }
}

// ---------------------------------------------------------------------------
// Output kernel.
//
// Block = 256 threads (4 waves), one (token chunk, head).  The head's S (bf16,
// D x D) is staged in LDS once per block with rows padded by 16 bytes.  Each
// wave handles 16 tokens per step as the B operand of v_mfma_f32_16x16x32_bf16
// computing num^T = S^T (R phi(q))^T: lane l holds token l % 16 and, for
// k-step s, the 16-byte chunk 4s + l/16 of that token's q -- a direct 16-byte
// global load, no LDS round trip.  The accumulator then holds, for the same
// token, value columns E(j, m, i) = 32*(j/2) + 8m + 4*(j%2) + i (m = l/16),
// which for each pair of m-blocks is again the 16-byte chunk 4t + m: g is read
// and out written with the same 16-byte per-lane pattern as q.  The
// denominator phi(q).z (unrotated features) is a per-lane partial dot product
// summed over the four lanes of a token with two xor shuffles.
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void output_kernel(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ g,
                                                     const uint16_t* __restrict__ sl,
                                                     const float* __restrict__ zf, int N, int H,
                                                     int L2, RopeArgs rope,
                                                     uint16_t* __restrict__ out) {
  constexpr int KS = D / 32;       // k-steps of 32 features
  constexpr int MB = D / 16;       // 16-row blocks of S^T
  constexpr int PITCH = D * 2 + 16;
  __shared__ __attribute__((aligned(16))) unsigned char lds_s[D * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane >> 4;
  const int col = lane & 15;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int n_begin = blockIdx.x * L2;
  const int n_end = min(N, n_begin + L2);

  // stage S^T rows
  const uint4* src = reinterpret_cast<const uint4*>(sl + (size_t)bh * D * D);
  for (int i = tid; i < D * D / 8; i += 256) {
    int row = i / (D / 8), u = i % (D / 8);
    *reinterpret_cast<uint4*>(lds_s + row * PITCH + 16 * u) = src[i];
  }
  float zr[KS][8];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const float4* zp = reinterpret_cast<const float4*>(zf + (size_t)bh * D + 8 * (4 * s + m));
    float4 z0 = zp[0], z1 = zp[1];
    zr[s][0] = z0.x; zr[s][1] = z0.y; zr[s][2] = z0.z; zr[s][3] = z0.w;
    zr[s][4] = z1.x; zr[s][5] = z1.y; zr[s][6] = z1.z; zr[s][7] = z1.w;
  }
  __syncthreads();

  const size_t tok_stride = (size_t)H * D;
  const size_t head_base = ((size_t)b * N * H + h) * D;

  for (int base = n_begin + 16 * wave; base < n_end; base += 64) {
    const int n = base + col;
    const bool valid = n < n_end;
    uint4 qv[KS], gv[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      size_t off = head_base + (size_t)n * tok_stride + 8 * (4 * s + m);
      if (valid) {
        qv[s] = *reinterpret_cast<const uint4*>(q + off);
        gv[s] = *reinterpret_cast<const uint4*>(g + off);
      } else {
        qv[s] = make_uint4(0, 0, 0, 0);
        gv[s] = make_uint4(0, 0, 0, 0);
      }
    }
    int ot = 0, oy = 0, ox = 0;
    if (ROPE) rope_rows(rope, (unsigned)(valid ? n : n_begin), ot, oy, ox);

    float den = 0.f;
    bf16x8 Bq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint32_t w[4] = {qv[s].x, qv[s].y, qv[s].z, qv[s].w};
      uint32_t pk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float a0 = fmaxf(bf_lo(w[u]), 0.f);
        float a1 = fmaxf(bf_hi(w[u]), 0.f);
        den += a0 * zr[s][2 * u] + a1 * zr[s][2 * u + 1];
        if (ROPE) {
          float2 cs = rope_cs(rope, 4 * (4 * s + m) + u, ot, oy, ox);
          float r0 = a0 * cs.x - a1 * cs.y;
          float r1 = a0 * cs.y + a1 * cs.x;
          a0 = r0;
          a1 = r1;
        }
        pk[u] = pack_bf16(a0, a1);
      }
      uint4 pv = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      Bq[s] = __builtin_bit_cast(bf16x8, pv);
    }

    f32x4 acc[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bf16x8 A = *reinterpret_cast<const bf16x8*>(lds_s + (16 * j + col) * PITCH +
                                                    16 * (4 * s + m));
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bq[s], acc[j], 0, 0, 0);
      }
    }

    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);
    const float inv = __builtin_amdgcn_rcpf(den + kEps);

#pragma unroll
    for (int t = 0; t < KS; ++t) {
      uint32_t gw[4] = {gv[t].x, gv[t].y, gv[t].z, gv[t].w};
      uint32_t ow[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float o2[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int jj = 2 * u + hlf;            // element of the 16-byte chunk
          const int j = 2 * t + (jj >> 2);       // accumulator block
          const int r = jj & 3;
          float gval = hlf ? bf_hi(gw[u]) : bf_lo(gw[u]);
          float sig = __builtin_amdgcn_rcpf(1.f + __expf(-gval));
          o2[hlf] = acc[j][r] * inv * sig;
        }
        ow[u] = pack_bf16(o2[0], o2[1]);
      }
      if (valid) {
        size_t off = head_base + (size_t)n * tok_stride + 8 * (4 * t + m);
        *reinterpret_cast<uint4*>(out + off) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      }
    }
  }
}

template <int D>
hipError_t launch_state_d(const Plan& p, const uint16_t* k, const uint16_t* v,
                          const RopeArgs& rope, void* ws, float* S_out, float* z_out,
                          hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  uint16_t* sl = reinterpret_cast<uint16_t*>(w + p.off_sl);
  float* zf = reinterpret_cast<float*>(w + p.off_z);
  dim3 g1(p.C, p.BH);
  if (rope.cs)
    hipLaunchKernelGGL((state_kernel<D, true>), g1, dim3(256), 0, stream, k, v, p.N, p.H, p.L,
                       p.C, rope, part);
  else
    hipLaunchKernelGGL((state_kernel<D, false>), g1, dim3(256), 0, stream, k, v, p.N, p.H, p.L,
                       p.C, rope, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((D * D / 8 + D + 255) / 256, p.BH);
  hipLaunchKernelGGL((reduce_kernel<D>), g2, dim3(256), 0, stream, part, p.C, sl, zf, S_out,
                     z_out);
  return hipGetLastError();
}

template <int D>
hipError_t launch_output_d(const Plan& p, const uint16_t* q, const uint16_t* g,
                           const RopeArgs& rope, const void* ws, uint16_t* out,
                           hipStream_t stream) {
  const char* w = static_cast<const char*>(ws);
  const uint16_t* sl = reinterpret_cast<const uint16_t*>(w + p.off_sl);
  const float* zf = reinterpret_cast<const float*>(w + p.off_z);
  dim3 g3(p.C2, p.BH);
  if (rope.cs)
    hipLaunchKernelGGL((output_kernel<D, true>), g3, dim3(256), 0, stream, q, g, sl, zf, p.N,
                       p.H, p.L2, rope, out);
  else
    hipLaunchKernelGGL((output_kernel<D, false>), g3, dim3(256), 0, stream, q, g, sl, zf, p.N,
                       p.H, p.L2, rope, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state(const Plan& p, const uint16_t* k, const uint16_t* v, const RopeArgs& rope,
                        void* ws, float* S_out, float* z_out, hipStream_t stream) {
  switch (p.D) {
    case 32: return launch_state_d<32>(p, k, v, rope, ws, S_out, z_out, stream);
    case 64: return launch_state_d<64>(p, k, v, rope, ws, S_out, z_out, stream);
    case 128: return launch_state_d<128>(p, k, v, rope, ws, S_out, z_out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_output(const Plan& p, const uint16_t* q, const uint16_t* g,
                         const RopeArgs& rope, const void* ws, uint16_t* out,
                         hipStream_t stream) {
  switch (p.D) {
    case 32: return launch_output_d<32>(p, q, g, rope, ws, out, stream);
    case 64: return launch_output_d<64>(p, q, g, rope, ws, out, stream);
    case 128: return launch_output_d<128>(p, q, g, rope, ws, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gla
