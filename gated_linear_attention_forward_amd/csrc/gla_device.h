// gla_device.h -- device helpers shared by the HIP kernel files (buffer
// addressing, bf16 packing, exact division, RoPE table lookups, transposing
// LDS reads).  Included inside each file's own anonymous namespace.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "gla_internal.h"

namespace gla {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr float kEps = 1e-6f;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr uint32_t kOob = 0x80000000u;  // offset past every slab (slabs are < 2 GiB)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Stores of the output stream carry the non-temporal hint (cache policy bit
// nt): nothing reads them back, and without the hint their write-back lands
// in the next pass's state kernel instead of this one.
constexpr int kCpolNt = 2;

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// The state kernels' k and v loads and the output kernel's g loads carry the
// hint too: each of those bytes is read once.  Measured A/B per forward pass:
// the k, v hint took 1-3% off the layer shapes; the g hint another 9% at 5B
// 720p and 14B 480p (0.5% at the 60 s shape, 2% slower on the small 5B 480p
// one).  On q as well as g, or on q alone, it measured worse or mixed.
__device__ __forceinline__ u32x4 load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNt);
}

__device__ __forceinline__ void store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolNt);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ReLU of two bf16 in one dword: as int16 a bf16 is negative exactly when its
// sign bit is set, so a packed signed max with 0 zeroes the negative halves
// (and -0) and keeps the rest bit for bit.
__device__ __forceinline__ uint32_t relu2(uint32_t w) {
  s16x2 x = __builtin_bit_cast(s16x2, w);
  x = __builtin_elementwise_max(x, (s16x2){0, 0});
  return __builtin_bit_cast(uint32_t, x);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest-even) and pack them, a in the low half
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 y = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, y);
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, DivMagic d) {
  uint32_t t = __umulhi(n, d.m);
  return (t + ((n - t) >> d.s1)) >> d.s2;
}

// Compile-time loop: calls f(std::integral_constant<int, i>) for i in [0, N).
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}

// Pairs per RoPE axis for head dimension D: y and x get floor(D/6) pairs each,
// t the rest (the split the host-side table builder uses).
template <int D>
struct Axes {
  static constexpr int Py = D / 6;
  static constexpr int Px = D / 6;
  static constexpr int Pt = D / 2 - 2 * (D / 6);
};

// Where a block reads its RoPE factors: the factorised table, either staged
// in LDS (t-rows of the block's own token range plus the y and x tables) or
// straight from global memory.
struct TabView {
  const float2* tab;
  int tbase;   // first t-row present
  int ntr;     // t-rows present
  int t_last;  // last t of the block's tokens (positions past the range clamp to it)
  const uint32_t* tab16;  // the same pairs as packed fp16 (cos, sin), when so staged
};

// Copies the n (cos, sin) pairs of a RoPE table from global memory to LDS
// with a block of NT threads, as fp32 pairs (F16 = false) or as packed fp16
// pairs (F16 = true, rounded to nearest even).  Whole pairs of pairs go as
// 16-byte loads, R of them per thread issued before any LDS write, so a
// table of up to 2 R NT pairs takes one memory round trip; loads past them
// read zero (buffer bounds) and are not written.  An odd last pair is read
// on its own.  Caller synchronises.
template <bool F16>
__device__ __forceinline__ void put_table_pair(void* dst, int i, float c, float sn) {
  if constexpr (F16) {
    const _Float16 hc = (_Float16)c, hs = (_Float16)sn;
    static_cast<uint32_t*>(dst)[i] = (uint32_t)__builtin_bit_cast(uint16_t, hc) |
                                     ((uint32_t)__builtin_bit_cast(uint16_t, hs) << 16);
  } else {
    static_cast<float2*>(dst)[i] = make_float2(c, sn);
  }
}
// One round of a table copy: R chunks per thread from chunk c0 on.
template <int NT, int R>
struct TableRound {
  u32x4 v[R];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int c0) {
#pragma unroll
    for (int k = 0; k < R; ++k)
      v[k] = __builtin_amdgcn_raw_buffer_load_b128(
          rs, (uint32_t)(c0 + k * NT + (int)threadIdx.x) * 16u, 0, 0);
  }
  template <bool F16>
  __device__ __forceinline__ void store(void* dst, int c0, int nc) const {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int ci = c0 + k * NT + (int)threadIdx.x;
      if (ci < nc) {
        put_table_pair<F16>(dst, 2 * ci, __uint_as_float(v[k][0]), __uint_as_float(v[k][1]));
        put_table_pair<F16>(dst, 2 * ci + 1, __uint_as_float(v[k][2]), __uint_as_float(v[k][3]));
      }
    }
  }
};
// A table of n pairs: its whole 16-byte chunks (n / 2 of them; loads past
// them read zero) and, for odd n, its last pair on its own.
struct TableSrc {
  __amdgpu_buffer_rsrc_t rs;
  int n, nc;
  __device__ __forceinline__ TableSrc(const float2* src, int n_) : n(n_), nc(n_ / 2) {
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float2*>(src), (short)0,
                                           (int)((uint32_t)n_ * 8u), kRsrcWord3);
  }
  // the odd last pair (every thread loads it; thread 0 writes it)
  __device__ __forceinline__ u32x2 load_tail() const {
    return n & 1 ? __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                 rs, (uint32_t)(n - 1) * 8u, 0, 0))
                 : u32x2{0u, 0u};
  }
  template <bool F16>
  __device__ __forceinline__ void store_tail(void* dst, u32x2 t) const {
    if ((n & 1) && threadIdx.x == 0)
      put_table_pair<F16>(dst, n - 1, __uint_as_float(t[0]), __uint_as_float(t[1]));
  }
};
// The first round's loads (and the odd pair's) are issued together, so a
// table of up to 2 R NT pairs costs one memory round trip; longer tables
// take further rounds.
template <int NT, int R, bool F16>
__device__ __forceinline__ void copy_table_to_lds(void* dst, const float2* src, int n) {
  const TableSrc ts(src, n);
  TableRound<NT, R> r;
  r.load(ts.rs, 0);
  const u32x2 tail = ts.load_tail();
  r.template store<F16>(dst, 0, ts.nc);
  ts.template store_tail<F16>(dst, tail);
  for (int c0 = R * NT; c0 < ts.nc; c0 += R * NT) {
    r.load(ts.rs, c0);
    r.template store<F16>(dst, c0, ts.nc);
  }
}
// Two tables (fp32 pairs) whose first rounds share one memory round trip.
template <int NT, int R0, int R1>
__device__ __forceinline__ void copy_two_tables_to_lds(float2* dst0, const float2* src0, int n0,
                                                       float2* dst1, const float2* src1, int n1) {
  const TableSrc t0(src0, n0), t1(src1, n1);
  TableRound<NT, R0> r0;
  TableRound<NT, R1> r1;
  r0.load(t0.rs, 0);
  r1.load(t1.rs, 0);
  const u32x2 e0 = t0.load_tail(), e1 = t1.load_tail();
  r0.template store<false>(dst0, 0, t0.nc);
  r1.template store<false>(dst1, 0, t1.nc);
  t0.template store_tail<false>(dst0, e0);
  t1.template store_tail<false>(dst1, e1);
  for (int c0 = R0 * NT; c0 < t0.nc; c0 += R0 * NT) {
    r0.load(t0.rs, c0);
    r0.template store<false>(dst0, c0, t0.nc);
  }
  for (int c0 = R1 * NT; c0 < t1.nc; c0 += R1 * NT) {
    r1.load(t1.rs, c0);
    r1.template store<false>(dst1, c0, t1.nc);
  }
}

// Copies the table rows a block of NT threads needs into LDS.  Caller
// synchronises.
template <int D, int NT = 256>
__device__ __forceinline__ TabView stage_table(const KArgs& a, float2* ltab, bool in_lds,
                                               int n_begin, int n_end) {
  using X = Axes<D>;
  TabView tv;
  tv.tab16 = nullptr;
  const int t_first = (int)fast_div((uint32_t)n_begin, a.div_hw);
  tv.t_last = (int)fast_div((uint32_t)(n_end - 1), a.div_hw);
  if (in_lds) {
    const int nt_blk = tv.t_last - t_first + 1;
    // the block's t-rows and the y and x tables in one memory round trip
    // (while they fit in one or two 16-byte loads per thread)
    copy_two_tables_to_lds<NT, 1, 2>(ltab, a.cs + (size_t)t_first * X::Pt, nt_blk * X::Pt,
                                     ltab + a.nt * X::Pt, a.cs + (size_t)a.T * X::Pt,
                                     a.Hh * X::Py + a.W * X::Px);
    tv.tab = ltab;
    tv.tbase = t_first;
    tv.ntr = a.nt;
  } else {
    tv.tab = a.cs;
    tv.tbase = 0;
    tv.ntr = a.T;
  }
  return tv;
}

// Per-axis row offsets (in pairs, each minus its axis's first pair index) of
// grid position (t, y, x) in a TabView.
struct RowOff {
  int ot, oy, ox;
};

template <int D>
__device__ __forceinline__ RowOff row_offsets(const KArgs& a, const TabView& tv, int t, int y,
                                              int x) {
  using X = Axes<D>;
  RowOff r;
  t = min(t, tv.t_last);
  r.ot = (t - tv.tbase) * X::Pt;
  r.oy = tv.ntr * X::Pt + y * X::Py - X::Pt;
  r.ox = tv.ntr * X::Pt + a.Hh * X::Py + x * X::Px - X::Pt - X::Py;
  return r;
}

// Token range [n_begin, n_end) of range index c of a kernel: piece c % CB of
// attention block c / CB.  A piece that starts past the last token (the last
// block can be shorter than the others) is the empty range [N, N), which
// stages no table rows and has no tiles.
__device__ __forceinline__ void range_of(const KArgs& a, int c, int& n_begin, int& n_end) {
  const int blk = c / a.CB;
  const int blk_begin = blk * a.BT;
  n_begin = min(blk_begin + (c - blk * a.CB) * a.L, a.N);
  n_end = max(min(min(n_begin + a.L, blk_begin + a.BT), a.N), n_begin);
}

// Grid position of token n (row-major t, y, x).
__device__ __forceinline__ void grid_pos(const KArgs& a, uint32_t n, int& t, int& y, int& x) {
  t = (int)fast_div(n, a.div_hw);
  const uint32_t rem = n - (uint32_t)t * (uint32_t)(a.Hh * a.W);
  y = (int)fast_div(rem, a.div_w);
  x = (int)(rem - (uint32_t)y * (uint32_t)a.W);
}

// Grid position of a token that advances by a fixed number of tokens per
// step: the advance is split once into (dt, dy, dx) with dx < W and dy < Hh,
// so each step needs one carry per axis instead of two divisions.  Positions
// past the last frame keep counting (table lookups clamp t).
struct GridWalk {
  int t, y, x;
  int dt, dy, dx;
  __device__ __forceinline__ void init(const KArgs& a, uint32_t n, uint32_t adv) {
    grid_pos(a, n, t, y, x);
    dt = (int)fast_div(adv, a.div_hw);
    const uint32_t r = adv - (uint32_t)dt * (uint32_t)(a.Hh * a.W);
    dy = (int)fast_div(r, a.div_w);
    dx = (int)(r - (uint32_t)dy * (uint32_t)a.W);
  }
  __device__ __forceinline__ void advance(const KArgs& a) {
    x += dx;
    const int cx = x >= a.W ? 1 : 0;
    x -= cx * a.W;
    y += dy + cx;
    const int cy = y >= a.Hh ? 1 : 0;
    y -= cy * a.Hh;
    t += dt + cy;
  }
};

// (cos, sin) of pair p, where p is known to lie in [PMIN, PMAX]: when that
// range sits inside one axis block the table row is chosen at compile time,
// otherwise by masks (no branches).
template <int D, int PMIN, int PMAX, bool H16 = false>
__device__ __forceinline__ float2 rope_factor(const TabView& tv, const RowOff& r, int p) {
  using X = Axes<D>;
  int base;
  if constexpr (PMAX < X::Pt) {
    base = r.ot;
  } else if constexpr (PMIN >= X::Pt && PMAX < X::Pt + X::Py) {
    base = r.oy;
  } else if constexpr (PMIN >= X::Pt + X::Py) {
    base = r.ox;
  } else {
    const int my = -(int)(p >= X::Pt && p < X::Pt + X::Py);
    const int mx = -(int)(p >= X::Pt + X::Py);
    base = r.ot + ((r.oy - r.ot) & my) + ((r.ox - r.ot) & mx);
  }
  if constexpr (H16) {
    const uint32_t w = tv.tab16[base + p];
    return float2{(float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)),
                  (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16))};
  } else {
    return tv.tab[base + p];
  }
}

// RoPE factors of the 4 pairs of one 16-byte chunk: chunk index c = 4 S + m
// with S compile-time and m in [0, 3].
template <int D, int S, bool H16 = false>
__device__ __forceinline__ void rope_factors(const TabView& tv, const RowOff& ro, int m,
                                             float2 (&cs)[4]) {
  static_for<4>([&](auto U) {
    constexpr int u = decltype(U)::value;
    cs[u] = rope_factor<D, 16 * S + u, 16 * S + 12 + u, H16>(tv, ro, 4 * (4 * S + m) + u);
  });
}

// Rotates the 4 pairs of one 16-byte chunk (8 features, ReLU already
// applied, as packed bf16) and returns them as packed bf16.
__device__ __forceinline__ u32x4 rotate_chunk(const u32x4 fq, const float2 (&cs)[4]) {
  u32x4 pk;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float a0 = bf_lo(fq[u]);
    const float a1 = bf_hi(fq[u]);
    pk[u] = pack_bf16(a0 * cs[u].x - a1 * cs[u].y, a0 * cs[u].y + a1 * cs[u].x);
  }
  return pk;
}

template <int D, int S, bool H16 = false>
__device__ __forceinline__ u32x4 rope_chunk(const u32x4 fq, const TabView& tv, const RowOff& ro,
                                            int m) {
  float2 cs[4];
  rope_factors<D, S, H16>(tv, ro, m, cs);
  return rotate_chunk(fq, cs);
}


// Loads and non-temporal stores of OB bytes (16, 8 or 4) per lane: one
// token's owned output columns in the accumulator layout of the 16x16x32
// MFMA (MB = D / 16 bf16 values).
template <int OB>
struct Chunk;
template <>
struct Chunk<16> {
  typedef u32x4 T;
};
template <>
struct Chunk<8> {
  typedef uint32_t T __attribute__((ext_vector_type(2)));
};
template <>
struct Chunk<4> {
  typedef uint32_t T __attribute__((ext_vector_type(1)));
};

template <int OB>
__device__ __forceinline__ typename Chunk<OB>::T load_chunk(__amdgpu_buffer_rsrc_t r,
                                                            uint32_t off) {
  using T = typename Chunk<OB>::T;
  if constexpr (OB == 16)
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  else if constexpr (OB == 8)
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  else
    return T{__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0)};
}

template <int OB>
__device__ __forceinline__ typename Chunk<OB>::T load_chunk_nt(__amdgpu_buffer_rsrc_t r,
                                                               uint32_t off) {
  using T = typename Chunk<OB>::T;
  if constexpr (OB == 16)
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNt);
  else if constexpr (OB == 8)
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolNt);
  else
    return T{__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCpolNt)};
}

template <int OB>
__device__ __forceinline__ void store_chunk_nt(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                               typename Chunk<OB>::T v) {
  if constexpr (OB == 16)
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolNt);
  else if constexpr (OB == 8)
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpolNt);
  else
    __builtin_amdgcn_raw_buffer_store_b32(v[0], r, off, 0, kCpolNt);
}

// Row tiles of D bf16 (D / 8 chunks of 16 bytes) that 16x16x32 MFMA B
// fragments read (lane l: row 16 j + l % 16, chunk 4 s + l / 16) are stored
// unpadded, chunk c of row r at position c ^ row_swizzle<D>(r).  A 128-bit
// LDS read serves the 16-lane sets {0..7, 24..31}, {8..15, 16..23},
// {32..39, 56..63} and {40..47, 48..55} together (measured with the bank
// conflict counter: this is the one grouping that fits fourteen probe
// patterns); rows of 256 bytes put every row at the same banks, and the
// swizzle gives each set's 16 accesses 16 distinct 16-byte bank groups.
// Shorter rows fold several rows into a 256-byte bank window, so the
// swizzle takes the row bits above those.
template <int D>
__device__ __forceinline__ int row_swizzle(int row) {
  constexpr int CPR = D / 8;
  return (row / (16 / CPR)) & (CPR - 1);
}
template <int D>
__device__ __forceinline__ int row_tile_offset(int row, int byte) {
  return row * 2 * D + 16 * ((byte >> 4) ^ row_swizzle<D>(row)) + (byte & 15);
}

// Stages ROWS dense rows of D bf16, rows ROW0 .. ROW0 + ROWS - 1 of src,
// into the same rows of an LDS row tile (row_tile_offset) with a block of NT
// threads.  load() issues all of a thread's global loads before store()
// writes any of them to LDS, so a block's staging waits for memory once
// rather than once per row chunk.  Caller synchronises.
template <int D, int ROWS, int NT, int ROW0 = 0>
struct RowStage {
  static constexpr int TOTAL = ROWS * D / 8;  // 16-byte chunks
  static constexpr int IT = (TOTAL + NT - 1) / NT;
  u32x4 v[IT];
  __device__ __forceinline__ void load(const uint16_t* src) {
    const u32x4* s = reinterpret_cast<const u32x4*>(src) + ROW0 * D / 8;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int i = threadIdx.x + k * NT;
      if (TOTAL % NT == 0 || i < TOTAL) v[k] = s[i];
    }
  }
  __device__ __forceinline__ void store(unsigned char* dst) const {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int i = threadIdx.x + k * NT;
      if (TOTAL % NT == 0 || i < TOTAL)
        *reinterpret_cast<u32x4*>(dst + row_tile_offset<D>(ROW0 + i / (D / 8), 16 * (i % (D / 8)))) =
            v[k];
    }
  }
};

// Waits until every vector memory access of the wave is done (s_waitcnt
// with vmcnt 0 and the expcnt and lgkmcnt fields at their no-wait maxima).
// Placed after a loop's prologue loads, it leaves nothing in flight on the
// entry path, so the compiler sizes the loop-head waits from the loop body
// alone instead of merging the prologue's different issue order into a wait
// for everything.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

constexpr int tile_pitch(int row_bytes) {
  int dw = row_bytes / 4;
  while (dw % 64 != 16 && dw % 64 != 48) ++dw;
  return 4 * dw;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA operand of features [32 i, 32 i + 32) over the 16 tokens of a
// token-major LDS tile (see the state kernel's description).
__device__ __forceinline__ bf16x8 frag_tr(const unsigned char* tile, int pitch, int i, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int f = 32 * i + 16 * (g & 1) + 4 * (s & 3);
  const int tok = 8 * (g >> 1) + (s >> 2);
  const unsigned char* p0 = tile + tok * pitch + 2 * f;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * pitch));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// ---- host-side launch helpers ----

// Bytes of the RoPE table slice a block stages in LDS.
inline int table_lds_bytes(const KArgs& a) {
  return 8 * (a.nt * a.Pt + a.Hh * a.Py + a.W * a.Px);
}

// A kernel that takes more than 64 KB of dynamic LDS raises its limit on the
// current device to the largest size asked for there so far (one record per
// kernel and device).  Raising happens under a per-kernel lock, so the
// attribute only ever grows: a caller asking for less can never lower it
// below a size another thread has already recorded and launched with.
constexpr int kMaxLdsDevices = 64;
template <auto K>
hipError_t allow_lds(size_t bytes) {
  static std::atomic<size_t> granted[kMaxLdsDevices];
  static std::mutex mu;
  if (bytes <= 65536) return hipSuccess;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxLdsDevices) return hipErrorInvalidDevice;
  if (bytes <= granted[dev].load(std::memory_order_acquire)) return hipSuccess;
  std::lock_guard<std::mutex> lock(mu);
  if (bytes <= granted[dev].load(std::memory_order_relaxed)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(K),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  granted[dev].store(bytes, std::memory_order_release);
  return hipSuccess;
}

}  // namespace
}  // namespace gla
