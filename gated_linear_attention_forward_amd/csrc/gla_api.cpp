// gla_api.cpp -- host side of the C ABI declared in include/gla.h:
// argument validation (before any HIP call), the factorised 3D RoPE table
// builder, the work plan, the per-(device, stream) workspace cache and the
// kernel launches.
#include "gla.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "gla_internal.h"

namespace gla {

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

DivMagic make_div_magic(uint32_t d) {
  DivMagic r{};
  int l = 0;
  while (l < 32 && (1ull << l) < d) ++l;  // l = ceil(log2 d)
  r.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  r.s1 = l < 1 ? l : 1;
  r.s2 = l > 1 ? l - 1 : 0;
  return r;
}

// The state kernel wants one block per compute unit (256 CUs), while every
// chunk adds one fp32 (D*D + D) partial per head.  The output kernel reads
// only a bf16 copy of the state per block, so it takes more, smaller blocks.
// Chunks and output ranges never straddle an attention block.
Plan make_plan(int B, int N, int H, int D, int block_tokens, int output_blocks) {
  Plan p{};
  p.B = B; p.N = N; p.H = H; p.D = D;
  p.BH = B * H;
  if (p.BH == 0 || N == 0) return p;
  p.BT = (block_tokens <= 0 || block_tokens >= N) ? N : block_tokens;
  p.NB = ceil_div(N, p.BT);
  const long long heads_blocks = (long long)p.BH * p.NB;

  // state chunks: whole 16-token tiles, about kStateBlocks blocks in total
  const int tiles = ceil_div(p.BT, 16);
  long long cb = kStateBlocks / heads_blocks;
  const int cmax = ceil_div(tiles, 4 * kStateMinTilesPerWave);
  if (cb > cmax) cb = cmax;
  if (cb > kMaxChunks) cb = kMaxChunks;
  if (cb < 1) cb = 1;
  p.L = ceil_div(tiles, (int)cb) * 16;
  p.CB = ceil_div(p.BT, p.L);
  p.C = p.NB * p.CB;

  const int its = ceil_div(p.BT, kOutputTileTokens);
  // at most output_blocks blocks: a target of whole rounds of resident
  // blocks is then never overshot into a nearly empty extra round
  long long sub = output_blocks / heads_blocks;
  if (sub > its) sub = its;
  if (sub < 1) sub = 1;
  p.L2 = ceil_div(its, (int)sub) * kOutputTileTokens;
  p.SUB = ceil_div(p.BT, p.L2);
  p.C2 = p.NB * p.SUB;

  size_t off = 0;
  p.off_part = off;
  off = align_up(off + (size_t)p.BH * p.C * (size_t)(D * D + D) * sizeof(float), 256);
  p.off_sl = off;
  off = align_up(off + (size_t)p.BH * p.NB * (D + 2) * D * sizeof(uint16_t), 256);
  p.ws_bytes = off;
  return p;
}

}  // namespace gla

using gla::Plan;

namespace {

bool dim_ok(int D) { return D == 32 || D == 64 || D == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + abytes) and [b, b + bbytes) share a byte
bool overlap2(const void* a, size_t abytes, const void* b, size_t bbytes) {
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bbytes && y < x + abytes;
}

bool overlap(const void* a, const void* b, size_t bytes) { return overlap2(a, bytes, b, bytes); }

// Shape checks shared by every entry point.  Returns GLA_OK and the tensor
// size in bytes, or an error.
int check_shape(int B, int N, int H, int D, size_t* bytes) {
  if (B < 0 || N < 0 || H < 0) return GLA_ERR_DIM;
  if (!dim_ok(D)) return GLA_ERR_DIM;
  const long long bh = (long long)B * H;
  if (bh > 65535) return GLA_ERR_DIM;  // heads go to grid.y
  const long long elems = (long long)B * N * H * D;
  // each batch element's [N, H, D] slab is addressed with 31-bit byte offsets
  if ((long long)N * H * D * 2 >= (1LL << 31)) return GLA_ERR_DIM;
  *bytes = (size_t)elems * 2;
  return GLA_OK;
}

int check_rope(const gla_rope_tables* rope, int N, int D) {
  if (!rope) return GLA_OK;
  if (!rope->cs) return GLA_ERR_NULL;
  if (!aligned16(rope->cs)) return GLA_ERR_ALIGN;  // the kernels copy it in 16-byte loads
  if (rope->D != D) return GLA_ERR_ROPE;
  if ((long long)rope->T * rope->Hh * rope->W != (long long)N) return GLA_ERR_ROPE;
  // the kernels fix the axis split for each D (as gla_rope_create builds it)
  if (rope->Py != D / 6 || rope->Px != D / 6 || rope->Pt != D / 2 - 2 * (D / 6)) return GLA_ERR_ROPE;
  if (rope->cs_floats != gla_rope_table_floats(rope->T, rope->Hh, rope->W, D)) return GLA_ERR_ROPE;
  return GLA_OK;
}

int check_tensors(std::initializer_list<const void*> ins, const void* out, size_t bytes) {
  for (const void* p : ins)
    if (!p) return GLA_ERR_NULL;
  if (out == nullptr) return GLA_ERR_NULL;
  for (const void* p : ins)
    if (!aligned16(p)) return GLA_ERR_ALIGN;
  if (!aligned16(out)) return GLA_ERR_ALIGN;
  for (const void* p : ins)
    if (bytes && overlap(p, out, bytes)) return GLA_ERR_ALIAS;
  return GLA_OK;
}

// Kernel arguments of one call.  L and CB are the token range and ranges per
// attention block of the kernel the arguments are for (L also sets how many
// t-rows of the table a block stages).
gla::KArgs kernel_args(const Plan& p, const gla_rope_tables* r, int L, int CB, void* ws) {
  gla::KArgs a{};
  a.N = p.N;
  a.H = p.H;
  a.slab_bytes = (uint32_t)((size_t)p.N * p.H * p.D * 2);
  a.L = L;
  a.CB = CB;
  a.BT = p.BT;
  a.NB = p.NB;
  a.C = p.C;
  if (r) {
    a.cs = reinterpret_cast<const float2*>(r->cs);
    a.T = r->T; a.Hh = r->Hh; a.W = r->W;
    a.Pt = r->Pt; a.Py = r->Py; a.Px = r->Px;
    const uint32_t hw = (uint32_t)r->Hh * (uint32_t)r->W;
    a.div_hw = gla::make_div_magic(hw);
    a.div_w = gla::make_div_magic((uint32_t)r->W);
    // a range of L consecutive tokens touches at most this many t-rows
    long long nt = ((long long)L + hw - 2) / hw + 1;
    a.nt = (int)(nt < r->T ? nt : r->T);
  }
  char* w = static_cast<char*>(ws);
  a.part = reinterpret_cast<float*>(w + p.off_part);
  a.sl = reinterpret_cast<uint16_t*>(w + p.off_sl);
  return a;
}

int rope_device_ok(const gla_rope_tables* rope) {
  if (!rope) return GLA_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GLA_ERR_HIP;
  return dev == rope->device ? GLA_OK : GLA_ERR_ROPE;
}

void axis_split(int D, int* Pt, int* Py, int* Px) {
  *Py = D / 6;
  *Px = D / 6;
  *Pt = D / 2 - 2 * (D / 6);
}

// ---- library-owned workspace, one per (device, stream) -------------------
struct WsKey {
  int device;
  void* stream;
  bool operator<(const WsKey& o) const {
    return device != o.device ? device < o.device : stream < o.stream;
  }
};
struct WsBuf {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<WsKey, WsBuf>* g_ws = nullptr;  // never destroyed: process-lifetime cache

// Returns the (device, stream) workspace of at least `bytes`, with *lk
// holding the cache's lock: the caller keeps it
// until its kernels are enqueued, so no other host thread can replace (and
// free) the buffer in between.  A buffer that grows is freed only after a
// synchronisation of its stream, which covers all earlier work that read it.
int get_workspace(size_t bytes, void* stream, void** out, std::unique_lock<std::mutex>* lk) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GLA_ERR_HIP;
  *lk = std::unique_lock<std::mutex>(g_ws_mu);
  if (!g_ws) g_ws = new (std::nothrow) std::map<WsKey, WsBuf>();
  if (!g_ws) return GLA_ERR_ALLOC;
  WsBuf& b = (*g_ws)[WsKey{dev, stream}];
  if (b.bytes < bytes) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (b.ptr) {
      // earlier work on this stream may still read the old buffer
      if (hipStreamSynchronize(s) != hipSuccess) return GLA_ERR_HIP;
      (void)hipFree(b.ptr);
      b.ptr = nullptr;
      b.bytes = 0;
    }
    size_t want = bytes + bytes / 4;
    if (hipMalloc(&b.ptr, want) != hipSuccess) {
      (void)hipGetLastError();
      b.ptr = nullptr;
      return GLA_ERR_ALLOC;
    }
    b.bytes = want;
  }
  *out = b.ptr;
  return GLA_OK;
}

// Frees the current device's cached workspaces.  The device is synchronised
// first, under the cache's lock: every kernel enqueued with one of these
// buffers was enqueued while the lock was held, so it has finished before the
// buffer goes.  Later calls allocate afresh.
int release_workspaces() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GLA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  if (!g_ws) return GLA_OK;
  bool any = false;
  for (const auto& kv : *g_ws) any = any || (kv.first.device == dev && kv.second.ptr);
  if (!any) return GLA_OK;
  if (hipDeviceSynchronize() != hipSuccess) return GLA_ERR_HIP;
  int rc = GLA_OK;
  for (auto it = g_ws->begin(); it != g_ws->end();) {
    if (it->first.device == dev) {
      if (it->second.ptr && hipFree(it->second.ptr) != hipSuccess) rc = GLA_ERR_HIP;
      it = g_ws->erase(it);
    } else {
      ++it;
    }
  }
  return rc;
}

int check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
  if (!ws) return GLA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return GLA_ERR_WORKSPACE;
  if (ws_bytes < p.ws_bytes) return GLA_ERR_WORKSPACE;
  return GLA_OK;
}

// The used part of a caller workspace overlaps none of the call's tensors
// (each `bytes` long) nor its states.
int check_ws_disjoint(const void* ws, size_t ws_used, std::initializer_list<const void*> tensors,
                      size_t bytes, std::initializer_list<std::pair<const void*, size_t>> extra = {}) {
  for (const void* t : tensors)
    if (t && bytes && overlap2(ws, ws_used, t, bytes)) return GLA_ERR_ALIAS;
  for (const auto& e : extra)
    if (e.first && e.second && overlap2(ws, ws_used, e.first, e.second)) return GLA_ERR_ALIAS;
  return GLA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? GLA_OK : GLA_ERR_LAUNCH; }

// Limits of the block plan: the output grid's second dimension and each
// head's partial-state window (32-bit buffer offsets).
int check_plan_limits(const Plan& p) {
  if (p.C2 > 65535) return GLA_ERR_DIM;
  if ((long long)p.C * (p.D * p.D + p.D) * 4 >= (1LL << 31)) return GLA_ERR_DIM;
  return GLA_OK;
}

// Carried and returned states of the block-causal pass: each may be NULL;
// given ones are 16-byte aligned, overlap none of the bf16 tensors, and the
// returned ones overlap nothing but (exactly) their carried counterpart.
int check_states(const float* S_in, const float* z_in, const float* S_out, const float* z_out,
                 int B, int H, int D, std::initializer_list<const void*> tensors, size_t bytes) {
  const size_t sb = (size_t)B * H * D * D * sizeof(float);
  const size_t zb = (size_t)B * H * D * sizeof(float);
  const void* ptr[4] = {S_in, z_in, S_out, z_out};
  const size_t len[4] = {sb, zb, sb, zb};
  for (int i = 0; i < 4; ++i) {
    if (!ptr[i]) continue;
    if (!aligned16(ptr[i])) return GLA_ERR_ALIGN;
    for (const void* t : tensors)
      if (bytes && overlap2(ptr[i], len[i], t, bytes)) return GLA_ERR_ALIAS;
  }
  // outputs against everything else, except the in-place pairs
  for (int o = 2; o < 4; ++o) {
    if (!ptr[o]) continue;
    for (int i = 0; i < 4; ++i) {
      if (i == o || !ptr[i]) continue;
      if (i == o - 2 && ptr[i] == ptr[o]) continue;  // in-place update
      if (overlap2(ptr[o], len[o], ptr[i], len[i])) return GLA_ERR_ALIAS;
    }
  }
  return GLA_OK;
}

int run_state(const Plan& p, const void* k, const void* v, const gla_rope_tables* rope, void* ws,
              float* S, float* z, const float* S_in, const float* z_in, void* stream) {
  gla::KArgs a = kernel_args(p, rope, p.L, p.CB, ws);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.S_out = S;
  a.z_out = z;
  a.S_in = S_in;
  a.z_in = z_in;
  return status_of(gla::launch_state(p, a, static_cast<hipStream_t>(stream)));
}

int run_output(const Plan& p, const void* q, const void* g, const gla_rope_tables* rope,
               void* out, void* ws, void* stream) {
  gla::KArgs a = kernel_args(p, rope, p.L2, p.SUB, ws);
  a.q = static_cast<const uint16_t*>(q);
  a.g = static_cast<const uint16_t*>(g);
  a.out = static_cast<uint16_t*>(out);
  return status_of(gla::launch_output(p, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* gla_strerror(int status) {
  switch (status) {
    case GLA_OK: return "success";
    case GLA_ERR_NULL: return "a required pointer is NULL";
    case GLA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case GLA_ERR_DIM: return "bad shape: D must be 32, 64 or 128; B, N, H non-negative; B*H <= 65535";
    case GLA_ERR_ROPE: return "RoPE tables do not match the call (grid, head dim or device)";
    case GLA_ERR_ALLOC: return "device memory allocation failed";
    case GLA_ERR_LAUNCH: return "kernel launch failed";
    case GLA_ERR_ALIAS: return "out overlaps an input";
    case GLA_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case GLA_ERR_HIP: return "HIP runtime call failed";
    case GLA_ERR_SCRATCH:
      return "the call needs more workspace than gla_forward_noalloc's fixed 32 MiB scratch";
    default: return "unknown status";
  }
}

size_t gla_rope_table_floats(int T, int Hh, int W, int D) {
  if (T < 1 || Hh < 1 || W < 1 || D < 2 || (D & 1)) return 0;
  int Pt, Py, Px;
  axis_split(D, &Pt, &Py, &Px);
  return 2 * ((size_t)T * Pt + (size_t)Hh * Py + (size_t)W * Px);
}

int gla_rope_fill_host(int T, int Hh, int W, int D, double theta, int t0, int y0, int x0,
                       float* cs, size_t cs_floats) {
  if (!cs) return GLA_ERR_NULL;
  const size_t need = gla_rope_table_floats(T, Hh, W, D);
  if (need == 0) return GLA_ERR_DIM;
  if (cs_floats < need) return GLA_ERR_ROPE;
  if (!(theta > 0.0)) return GLA_ERR_ROPE;
  int P[3];
  axis_split(D, &P[0], &P[1], &P[2]);
  const int len[3] = {T, Hh, W};
  const int off[3] = {t0, y0, x0};
  size_t at = 0;
  for (int a = 0; a < 3; ++a) {
    for (int pos = 0; pos < len[a]; ++pos) {
      for (int j = 0; j < P[a]; ++j) {
        // frequency theta^(-2j / (2 Pa)) of pair j within this axis block
        double omega = std::exp(-std::log(theta) * (2.0 * j) / (2.0 * P[a]));
        double ang = (double)(pos + off[a]) * omega;
        cs[at++] = (float)std::cos(ang);
        cs[at++] = (float)std::sin(ang);
      }
    }
  }
  return GLA_OK;
}

int gla_rope_create(int T, int Hh, int W, int D, double theta, int t0, int y0, int x0,
                    void* stream, gla_rope_tables** out) {
  if (!out) return GLA_ERR_NULL;
  *out = nullptr;
  if (!dim_ok(D) && D != 256) return GLA_ERR_DIM;
  const size_t nf = gla_rope_table_floats(T, Hh, W, D);
  if (nf == 0) return GLA_ERR_DIM;
  if ((long long)T * Hh * W > INT32_MAX) return GLA_ERR_DIM;
  std::vector<float> host;
  try {
    host.resize(nf);
  } catch (...) {
    return GLA_ERR_ALLOC;
  }
  int rc = gla_rope_fill_host(T, Hh, W, D, theta, t0, y0, x0, host.data(), nf);
  if (rc) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GLA_ERR_HIP;
  auto* r = new (std::nothrow) gla_rope_tables();
  if (!r) return GLA_ERR_ALLOC;
  void* d = nullptr;
  if (hipMalloc(&d, nf * sizeof(float)) != hipSuccess) {
    (void)hipGetLastError();
    delete r;
    return GLA_ERR_ALLOC;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(d, host.data(), nf * sizeof(float), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    (void)hipFree(d);
    delete r;
    return GLA_ERR_HIP;
  }
  r->T = T; r->Hh = Hh; r->W = W; r->D = D;
  axis_split(D, &r->Pt, &r->Py, &r->Px);
  r->t0 = t0; r->y0 = y0; r->x0 = x0;
  r->theta = theta;
  r->cs = static_cast<const float*>(d);
  r->cs_floats = nf;
  r->device = dev;
  *out = r;
  return GLA_OK;
}

int gla_rope_destroy(gla_rope_tables* tables) {
  if (!tables) return GLA_OK;
  int rc = GLA_OK;
  if (tables->cs && hipFree(const_cast<float*>(tables->cs)) != hipSuccess) rc = GLA_ERR_HIP;
  delete tables;
  return rc;
}

size_t gla_workspace_bytes(int B, int N, int H, int D) {
  size_t bytes = 0;
  if (check_shape(B, N, H, D, &bytes) != GLA_OK) return 0;
  if (bytes == 0) return 0;
  return gla::make_plan(B, N, H, D).ws_bytes;
}

int gla_workspace_release(void) { return release_workspaces(); }

int gla_forward_check(const void* q, const void* k, const void* v, const void* g,
                      const gla_rope_tables* rope, const void* out, int B, int N, int H, int D) {
  size_t bytes = 0;
  int rc = check_shape(B, N, H, D, &bytes);
  if (rc) return rc;
  if (bytes == 0) return GLA_OK;
  if ((rc = check_rope(rope, N, D))) return rc;
  return check_tensors({q, k, v, g}, out, bytes);
}

int gla_state_ws(const void* k, const void* v, const gla_rope_tables* rope, int B, int N, int H,
                 int D, void* workspace, size_t workspace_bytes, void* stream) {
  size_t bytes = 0;
  int rc = check_shape(B, N, H, D, &bytes);
  if (rc) return rc;
  if (bytes == 0) return GLA_OK;
  if ((rc = check_rope(rope, N, D))) return rc;
  if (!k || !v) return GLA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v)) return GLA_ERR_ALIGN;
  Plan p = gla::make_plan(B, N, H, D);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  if ((rc = check_ws_disjoint(workspace, p.ws_bytes, {k, v}, bytes))) return rc;
  if ((rc = rope_device_ok(rope))) return rc;
  return run_state(p, k, v, rope, workspace, nullptr, nullptr, nullptr, nullptr, stream);
}

int gla_output_ws(const void* q, const void* g, const gla_rope_tables* rope, void* out, int B,
                  int N, int H, int D, void* workspace, size_t workspace_bytes, void* stream) {
  size_t bytes = 0;
  int rc = check_shape(B, N, H, D, &bytes);
  if (rc) return rc;
  if (bytes == 0) return GLA_OK;
  if ((rc = check_rope(rope, N, D))) return rc;
  if ((rc = check_tensors({q, g}, out, bytes))) return rc;
  Plan p = gla::make_plan(B, N, H, D);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  if ((rc = check_ws_disjoint(workspace, p.ws_bytes, {q, g, out}, bytes))) return rc;
  if ((rc = rope_device_ok(rope))) return rc;
  return run_output(p, q, g, rope, out, workspace, stream);
}

int gla_forward_ws(const void* q, const void* k, const void* v, const void* g,
                   const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int rc = gla_forward_check(q, k, v, g, rope, out, B, N, H, D);
  if (rc) return rc;
  if ((long long)B * N * H == 0) return GLA_OK;
  Plan p = gla::make_plan(B, N, H, D);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  if ((rc = check_ws_disjoint(workspace, p.ws_bytes, {q, k, v, g, out},
                              (size_t)B * N * H * D * 2)))
    return rc;
  if ((rc = rope_device_ok(rope))) return rc;
  if (gla::pass_in_block(p)) {
    // short sequence: one launch, one block per head (state, then outputs)
    gla::KArgs a1 = kernel_args(p, rope, p.N, 1, workspace);
    a1.q = static_cast<const uint16_t*>(q);
    a1.k = static_cast<const uint16_t*>(k);
    a1.v = static_cast<const uint16_t*>(v);
    a1.g = static_cast<const uint16_t*>(g);
    a1.out = static_cast<uint16_t*>(out);
    return status_of(gla::launch_pass_in_block(p, a1, static_cast<hipStream_t>(stream)));
  }
  if (gla::output_sums_partials(p)) {
    // small partials: the output kernel sums them (two launches, not three)
    gla::KArgs as = kernel_args(p, rope, p.L, p.CB, workspace);
    as.k = static_cast<const uint16_t*>(k);
    as.v = static_cast<const uint16_t*>(v);
    if ((rc = status_of(gla::launch_state(p, as, static_cast<hipStream_t>(stream), false))))
      return rc;
    gla::KArgs ao = kernel_args(p, rope, p.L2, p.SUB, workspace);
    ao.q = static_cast<const uint16_t*>(q);
    ao.g = static_cast<const uint16_t*>(g);
    ao.out = static_cast<uint16_t*>(out);
    return status_of(gla::launch_output(p, ao, static_cast<hipStream_t>(stream), true));
  }
  rc = run_state(p, k, v, rope, workspace, nullptr, nullptr, nullptr, nullptr, stream);
  if (rc) return rc;
  return run_output(p, q, g, rope, out, workspace, stream);
}

int gla_forward(const void* q, const void* k, const void* v, const void* g,
                const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                void* stream) {
  int rc = gla_forward_check(q, k, v, g, rope, out, B, N, H, D);
  if (rc) return rc;
  if ((long long)B * N * H == 0) return GLA_OK;
  Plan p = gla::make_plan(B, N, H, D);
  void* ws = nullptr;
  std::unique_lock<std::mutex> lk;
  if ((rc = get_workspace(p.ws_bytes, stream, &ws, &lk))) return rc;
  return gla_forward_ws(q, k, v, g, rope, out, B, N, H, D, ws, p.ws_bytes, stream);
}

int gla_forward_noalloc(const void* q, const void* k, const void* v, const void* g,
                        const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                        void* stream) {
  int rc = gla_forward_check(q, k, v, g, rope, out, B, N, H, D);
  if (rc) return rc;
  if ((long long)B * N * H == 0) return GLA_OK;
  Plan p = gla::make_plan(B, N, H, D);
  if (p.ws_bytes > gla::kScratchBytes) return GLA_ERR_SCRATCH;
  void* ws = nullptr;
  if (gla::scratch_pointer(&ws) != hipSuccess) return GLA_ERR_HIP;
  // the same checks and launches as gla_forward_ws, on the fixed scratch
  return gla_forward_ws(q, k, v, g, rope, out, B, N, H, D, ws, gla::kScratchBytes, stream);
}

int gla_state(const void* k, const void* v, const gla_rope_tables* rope, float* S, float* z,
              int B, int N, int H, int D, void* stream) {
  size_t bytes = 0;
  int rc = check_shape(B, N, H, D, &bytes);
  if (rc) return rc;
  if ((rc = check_rope(rope, N, D))) return rc;
  if ((long long)B * H == 0) return GLA_OK;
  if (!S || !z) return GLA_ERR_NULL;
  if (!aligned16(S) || !aligned16(z)) return GLA_ERR_ALIGN;
  if (N > 0) {
    if (!k || !v) return GLA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v)) return GLA_ERR_ALIGN;
  }
  const size_t sbytes = (size_t)B * H * D * D * sizeof(float);
  const size_t zbytes = (size_t)B * H * D * sizeof(float);
  if (bytes && (overlap2(S, sbytes, k, bytes) || overlap2(S, sbytes, v, bytes) ||
                overlap2(z, zbytes, k, bytes) || overlap2(z, zbytes, v, bytes)))
    return GLA_ERR_ALIAS;
  if (overlap2(S, sbytes, z, zbytes)) return GLA_ERR_ALIAS;
  if (N == 0) {
    // empty sequence: S = 0, z = 0, written by the reduce kernel with no
    // partials and no carried state (a kernel, not a memset, so the call
    // can be captured into a graph)
    Plan p{};
    p.B = B; p.N = 0; p.H = H; p.D = D; p.BH = B * H;
    gla::KArgs a{};
    a.H = H;
    a.S_out = S; a.z_out = z;
    return status_of(gla::launch_carry(p, a, static_cast<hipStream_t>(stream)));
  }
  Plan p = gla::make_plan(B, N, H, D);
  void* ws = nullptr;
  std::unique_lock<std::mutex> lk;
  if ((rc = get_workspace(p.ws_bytes, stream, &ws, &lk))) return rc;
  if ((rc = rope_device_ok(rope))) return rc;
  return run_state(p, k, v, rope, ws, S, z, nullptr, nullptr, stream);
}

size_t gla_workspace_bytes_blocks(int B, int N, int H, int D, int block_tokens) {
  size_t bytes = 0;
  if (check_shape(B, N, H, D, &bytes) != GLA_OK || block_tokens < 1) return 0;
  if (bytes == 0) return 0;
  return gla::make_plan(B, N, H, D, block_tokens).ws_bytes;
}

int gla_forward_blocks_check(const void* q, const void* k, const void* v, const void* g,
                             const gla_rope_tables* rope, const void* out, int B, int N, int H,
                             int D, int block_tokens, const float* S_in, const float* z_in,
                             const float* S_out, const float* z_out) {
  size_t bytes = 0;
  int rc = check_shape(B, N, H, D, &bytes);
  if (rc) return rc;
  if (block_tokens < 1) return GLA_ERR_DIM;
  if ((long long)B * H == 0) return GLA_OK;
  if ((rc = check_rope(rope, N, D))) return rc;
  if (bytes) {
    if ((rc = check_tensors({q, k, v, g}, out, bytes))) return rc;
    if ((rc = check_plan_limits(gla::make_plan(B, N, H, D, block_tokens)))) return rc;
  }
  return check_states(S_in, z_in, S_out, z_out, B, H, D, {q, k, v, g, out}, bytes);
}

int gla_forward_blocks_ws(const void* q, const void* k, const void* v, const void* g,
                          const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                          int block_tokens, const float* S_in, const float* z_in, float* S_out,
                          float* z_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = gla_forward_blocks_check(q, k, v, g, rope, out, B, N, H, D, block_tokens, S_in, z_in,
                                    S_out, z_out);
  if (rc) return rc;
  if ((long long)B * H == 0) return GLA_OK;
  if (N == 0) {
    // no tokens: the returned state is the carried one
    if (!S_out && !z_out) return GLA_OK;
    Plan p{};
    p.B = B; p.N = 0; p.H = H; p.D = D; p.BH = B * H;
    gla::KArgs a{};
    a.H = H;
    a.S_in = S_in; a.z_in = z_in; a.S_out = S_out; a.z_out = z_out;
    return status_of(gla::launch_carry(p, a, static_cast<hipStream_t>(stream)));
  }
  Plan p = gla::make_plan(B, N, H, D, block_tokens);
  if ((rc = check_ws(p, workspace, workspace_bytes))) return rc;
  {
    const size_t sb = (size_t)B * H * D * D * sizeof(float), zb = (size_t)B * H * D * sizeof(float);
    if ((rc = check_ws_disjoint(workspace, p.ws_bytes, {q, k, v, g, out},
                                (size_t)B * N * H * D * 2,
                                {{S_in, sb}, {z_in, zb}, {S_out, sb}, {z_out, zb}})))
      return rc;
  }
  if ((rc = rope_device_ok(rope))) return rc;
  rc = run_state(p, k, v, rope, workspace, S_out, z_out, S_in, z_in, stream);
  if (rc) return rc;
  return run_output(p, q, g, rope, out, workspace, stream);
}

int gla_forward_blocks(const void* q, const void* k, const void* v, const void* g,
                       const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                       int block_tokens, const float* S_in, const float* z_in, float* S_out,
                       float* z_out, void* stream) {
  int rc = gla_forward_blocks_check(q, k, v, g, rope, out, B, N, H, D, block_tokens, S_in, z_in,
                                    S_out, z_out);
  if (rc) return rc;
  if ((long long)B * H == 0) return GLA_OK;
  void* ws = nullptr;
  size_t wsb = 0;
  std::unique_lock<std::mutex> lk;
  if (N > 0) {
    Plan p = gla::make_plan(B, N, H, D, block_tokens);
    wsb = p.ws_bytes;
    if ((rc = get_workspace(wsb, stream, &ws, &lk))) return rc;
  }
  return gla_forward_blocks_ws(q, k, v, g, rope, out, B, N, H, D, block_tokens, S_in, z_in, S_out,
                               z_out, ws, wsb, stream);
}

// ---- gated softmax anchor attention -------------------------------------

static int check_softmax_shape(int B, int N, int H, int D, size_t* bytes) {
  if (B < 0 || N < 0 || H < 0) return GLA_ERR_DIM;
  if (D != 128 && D != 256) return GLA_ERR_DIM;
  if ((long long)B * H > 65535) return GLA_ERR_DIM;
  if ((long long)N * H * D * 2 >= (1LL << 31)) return GLA_ERR_DIM;
  *bytes = (size_t)B * N * H * D * 2;
  return GLA_OK;
}

size_t gla_softmax_workspace_bytes(int B, int N, int H, int D) {
  size_t bytes = 0;
  if (check_softmax_shape(B, N, H, D, &bytes) != GLA_OK || bytes == 0) return 0;
  return 2 * gla::align_up(bytes, 256);
}

int gla_softmax_forward_check(const void* q, const void* k, const void* v, const void* g,
                              const gla_rope_tables* rope, const void* out, int B, int N, int H,
                              int D) {
  size_t bytes = 0;
  int rc = check_softmax_shape(B, N, H, D, &bytes);
  if (rc) return rc;
  if (bytes == 0) return GLA_OK;
  if ((rc = check_rope(rope, N, D))) return rc;
  return check_tensors({q, k, v, g}, out, bytes);
}

int gla_softmax_forward_ws(const void* q, const void* k, const void* v, const void* g,
                           const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int rc = gla_softmax_forward_check(q, k, v, g, rope, out, B, N, H, D);
  if (rc) return rc;
  size_t bytes = 0;
  check_softmax_shape(B, N, H, D, &bytes);
  if (bytes == 0) return GLA_OK;
  const size_t need = gla_softmax_workspace_bytes(B, N, H, D);
  if (!workspace) return GLA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
    return GLA_ERR_WORKSPACE;
  if (overlap2(workspace, need, q, bytes) || overlap2(workspace, need, k, bytes) ||
      overlap2(workspace, need, v, bytes) || overlap2(workspace, need, g, bytes) ||
      overlap2(workspace, need, out, bytes))
    return GLA_ERR_ALIAS;
  if ((rc = rope_device_ok(rope))) return rc;
  Plan p{};
  p.B = B; p.N = N; p.H = H; p.D = D; p.BH = B * H;
  gla::KArgs a = kernel_args(p, rope, 0, 1, workspace);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.g = static_cast<const uint16_t*>(g);
  a.out = static_cast<uint16_t*>(out);
  uint16_t* qr = static_cast<uint16_t*>(workspace);
  uint16_t* kr = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + need / 2);
  return status_of(gla::launch_softmax(p, a, qr, kr, static_cast<hipStream_t>(stream)));
}

int gla_softmax_forward(const void* q, const void* k, const void* v, const void* g,
                        const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                        void* stream) {
  int rc = gla_softmax_forward_check(q, k, v, g, rope, out, B, N, H, D);
  if (rc) return rc;
  const size_t need = gla_softmax_workspace_bytes(B, N, H, D);
  if (need == 0) return GLA_OK;
  void* ws = nullptr;
  std::unique_lock<std::mutex> lk;
  if ((rc = get_workspace(need, stream, &ws, &lk))) return rc;
  return gla_softmax_forward_ws(q, k, v, g, rope, out, B, N, H, D, ws, need, stream);
}

// ---- backward pass of the bidirectional mixer ----------------------------

}  // extern "C"

namespace {

// Workspace of the backward pass: the forward plan's partials and S^T
// operand, then the S rows operand, fp32 z, the query kernel's dS and dz
// partials (one D*D + D set per range) and the fp32 dz they reduce to.
struct BwdLayout {
  Plan p;
  size_t off_sl2, off_z, off_dsp, off_dz, bytes;
};

BwdLayout bwd_layout(int B, int N, int H, int D) {
  BwdLayout l{};
  l.p = gla::make_plan(B, N, H, D, 0, gla::kBackwardBlocks);
  size_t off = l.p.ws_bytes;
  l.off_sl2 = off;
  off = gla::align_up(off + (size_t)l.p.BH * D * D * sizeof(uint16_t), 256);
  l.off_z = off;
  off = gla::align_up(off + (size_t)l.p.BH * D * sizeof(float), 256);
  l.off_dsp = off;
  off = gla::align_up(off + (size_t)l.p.BH * l.p.C2 * (D * D + D) * sizeof(float), 256);
  l.off_dz = off;
  off = gla::align_up(off + (size_t)l.p.BH * D * sizeof(float), 256);
  l.bytes = off;
  return l;
}

// The backward pass after argument validation.  S_saved and z_saved: the
// forward's fp32 state, or NULL to recompute it from k and v.
int backward_run(const void* q, const void* k, const void* v, const void* g, const void* dout,
                 const gla_rope_tables* rope, const float* S_saved, const float* z_saved,
                 void* dq, void* dk, void* dv, void* dg, int B, int N, int H, int D,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = GLA_OK;
  size_t bytes = 0;
  check_shape(B, N, H, D, &bytes);
  if (bytes == 0) return GLA_OK;
  const BwdLayout l = bwd_layout(B, N, H, D);
  if (!workspace) return GLA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < l.bytes)
    return GLA_ERR_WORKSPACE;
  for (const void* t : {q, k, v, g, dout, static_cast<const void*>(dq),
                        static_cast<const void*>(dk), static_cast<const void*>(dv),
                        static_cast<const void*>(dg)})
    if (overlap2(workspace, l.bytes, t, bytes)) return GLA_ERR_ALIAS;
  if (S_saved && (overlap2(workspace, l.bytes, S_saved, (size_t)B * H * D * D * sizeof(float)) ||
                  overlap2(workspace, l.bytes, z_saved, (size_t)B * H * D * sizeof(float))))
    return GLA_ERR_ALIAS;
  if ((rc = rope_device_ok(rope))) return rc;
  const Plan& p = l.p;
  char* w = static_cast<char*>(workspace);
  uint16_t* sl2 = reinterpret_cast<uint16_t*>(w + l.off_sl2);
  float* zbuf = reinterpret_cast<float*>(w + l.off_z);
  float* dsp = reinterpret_cast<float*>(w + l.off_dsp);
  float* dzbuf = reinterpret_cast<float*>(w + l.off_dz);
  hipStream_t s = static_cast<hipStream_t>(stream);
  gla::BArgs bw{};
  bw.dout = static_cast<const uint16_t*>(dout);
  bw.dq = static_cast<uint16_t*>(dq);
  bw.dk = static_cast<uint16_t*>(dk);
  bw.dv = static_cast<uint16_t*>(dv);
  bw.dg = static_cast<uint16_t*>(dg);
  bw.z = zbuf;
  bw.dsp = dsp;
  bw.dz = dzbuf;
  bw.C2 = p.C2;

  // 1. S (both operand layouts) and fp32 z: from k and v, or from the saved
  //    state by the reduce kernel alone (no chunk partials: its window is
  //    empty and reads zero, so it writes the saved fp32 values' operands)
  gla::KArgs a1 = kernel_args(p, rope, p.L, p.CB, workspace);
  a1.sl2 = sl2;
  a1.z_out = zbuf;
  if (S_saved) {
    a1.C = 0;
    a1.CB = 0;
    a1.S_in = S_saved;
    a1.z_in = z_saved;
    if ((rc = status_of(gla::launch_reduce_state(p, a1, s)))) return rc;
  } else {
    a1.k = static_cast<const uint16_t*>(k);
    a1.v = static_cast<const uint16_t*>(v);
    if ((rc = status_of(gla::launch_state(p, a1, s)))) return rc;
  }
  // 2. query side: dq, dg and the dS and dz partials of each range
  gla::KArgs a2 = kernel_args(p, rope, p.L2, p.SUB, workspace);
  a2.q = static_cast<const uint16_t*>(q);
  a2.g = static_cast<const uint16_t*>(g);
  a2.sl2 = sl2;
  if ((rc = status_of(gla::launch_bwd_query(p, a2, bw, s)))) return rc;
  // 3. dS (both operand layouts) and fp32 dz: the reduce kernel over the C2
  //    range partials of each head
  Plan p3 = p;
  p3.CB = p.C2;
  p3.C = p.C2;
  p3.NB = 1;
  gla::KArgs a3 = kernel_args(p3, rope, p.L2, p.C2, workspace);
  a3.part = dsp;
  a3.sl2 = sl2;
  a3.z_out = dzbuf;
  if ((rc = status_of(gla::launch_reduce_state(p3, a3, s)))) return rc;
  // 4. key side: dk, dv
  gla::KArgs a4 = kernel_args(p, rope, p.L2, p.SUB, workspace);
  a4.k = static_cast<const uint16_t*>(k);
  a4.v = static_cast<const uint16_t*>(v);
  a4.sl2 = sl2;
  return status_of(gla::launch_bwd_key(p, a4, bw, s));
}

}  // namespace

extern "C" {

size_t gla_backward_workspace_bytes(int B, int N, int H, int D) {
  size_t bytes = 0;
  if (check_shape(B, N, H, D, &bytes) != GLA_OK || bytes == 0) return 0;
  return bwd_layout(B, N, H, D).bytes;
}

int gla_backward_check(const void* q, const void* k, const void* v, const void* g,
                       const void* dout, const gla_rope_tables* rope, const void* dq,
                       const void* dk, const void* dv, const void* dg, int B, int N, int H,
                       int D) {
  size_t bytes = 0;
  int rc = check_shape(B, N, H, D, &bytes);
  if (rc) return rc;
  if (bytes == 0) return GLA_OK;
  if ((rc = check_rope(rope, N, D))) return rc;
  const void* outs[4] = {dq, dk, dv, dg};
  for (const void* o : outs)
    if ((rc = check_tensors({q, k, v, g, dout}, o, bytes))) return rc;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j], bytes)) return GLA_ERR_ALIAS;
  return check_plan_limits(gla::make_plan(B, N, H, D, 0, gla::kBackwardBlocks));
}

int gla_backward_ws(const void* q, const void* k, const void* v, const void* g, const void* dout,
                    const gla_rope_tables* rope, void* dq, void* dk, void* dv, void* dg, int B,
                    int N, int H, int D, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = gla_backward_check(q, k, v, g, dout, rope, dq, dk, dv, dg, B, N, H, D);
  if (rc) return rc;
  return backward_run(q, k, v, g, dout, rope, nullptr, nullptr, dq, dk, dv, dg, B, N, H, D,
                      workspace, workspace_bytes, stream);
}

int gla_backward(const void* q, const void* k, const void* v, const void* g, const void* dout,
                 const gla_rope_tables* rope, void* dq, void* dk, void* dv, void* dg, int B,
                 int N, int H, int D, void* stream) {
  int rc = gla_backward_check(q, k, v, g, dout, rope, dq, dk, dv, dg, B, N, H, D);
  if (rc) return rc;
  const size_t need = gla_backward_workspace_bytes(B, N, H, D);
  if (need == 0) return GLA_OK;
  void* ws = nullptr;
  std::unique_lock<std::mutex> lk;
  if ((rc = get_workspace(need, stream, &ws, &lk))) return rc;
  return gla_backward_ws(q, k, v, g, dout, rope, dq, dk, dv, dg, B, N, H, D, ws, need, stream);
}

int gla_backward_saved_check(const void* q, const void* k, const void* v, const void* g,
                             const void* dout, const gla_rope_tables* rope, const float* S,
                             const float* z, const void* dq, const void* dk, const void* dv,
                             const void* dg, int B, int N, int H, int D) {
  int rc = gla_backward_check(q, k, v, g, dout, rope, dq, dk, dv, dg, B, N, H, D);
  if (rc) return rc;
  size_t bytes = 0;
  check_shape(B, N, H, D, &bytes);
  if (bytes == 0) return GLA_OK;
  if (!S || !z) return GLA_ERR_NULL;
  if (!aligned16(S) || !aligned16(z)) return GLA_ERR_ALIGN;
  const size_t sb = (size_t)B * H * D * D * sizeof(float), zb = (size_t)B * H * D * sizeof(float);
  for (const void* o : {dq, dk, dv, dg})
    if (overlap2(S, sb, o, bytes) || overlap2(z, zb, o, bytes)) return GLA_ERR_ALIAS;
  return GLA_OK;
}

int gla_backward_saved_ws(const void* q, const void* k, const void* v, const void* g,
                          const void* dout, const gla_rope_tables* rope, const float* S,
                          const float* z, void* dq, void* dk, void* dv, void* dg, int B, int N,
                          int H, int D, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = gla_backward_saved_check(q, k, v, g, dout, rope, S, z, dq, dk, dv, dg, B, N, H, D);
  if (rc) return rc;
  return backward_run(q, k, v, g, dout, rope, S, z, dq, dk, dv, dg, B, N, H, D, workspace,
                      workspace_bytes, stream);
}

int gla_backward_saved(const void* q, const void* k, const void* v, const void* g,
                       const void* dout, const gla_rope_tables* rope, const float* S,
                       const float* z, void* dq, void* dk, void* dv, void* dg, int B, int N, int H,
                       int D, void* stream) {
  int rc = gla_backward_saved_check(q, k, v, g, dout, rope, S, z, dq, dk, dv, dg, B, N, H, D);
  if (rc) return rc;
  const size_t need = gla_backward_workspace_bytes(B, N, H, D);
  if (need == 0) return GLA_OK;
  void* ws = nullptr;
  std::unique_lock<std::mutex> lk;
  if ((rc = get_workspace(need, stream, &ws, &lk))) return rc;
  return backward_run(q, k, v, g, dout, rope, S, z, dq, dk, dv, dg, B, N, H, D, ws, need, stream);
}

}  // extern "C"

// ---- projection prologue fused with the mixer ------------------------------

namespace {

// Workspace: the forward plan's partials and state operand, then the
// projected q and g.
struct ProjLayout {
  Plan p;
  size_t off_q, off_g, bytes;
};

ProjLayout proj_layout(int B, int N, int H, int D) {
  ProjLayout l{};
  l.p = gla::make_plan(B, N, H, D);
  const size_t t = (size_t)B * N * H * D * sizeof(uint16_t);
  size_t off = l.p.ws_bytes;
  l.off_q = off;
  off = gla::align_up(off + t, 256);
  l.off_g = off;
  off = gla::align_up(off + t, 256);
  l.bytes = off;
  return l;
}

int check_proj_shape(int B, int N, int C, int H, int D, size_t* out_bytes) {
  int rc = check_shape(B, N, H, D, out_bytes);
  if (rc) return rc;
  if (C < 64 || C % 64 != 0) return GLA_ERR_DIM;
  if ((long long)N * C * 2 >= (1LL << 31)) return GLA_ERR_DIM;           // x slab offsets
  if (4LL * H * D * C * 2 >= (1LL << 31)) return GLA_ERR_DIM;            // weight offsets
  const long long tiles = (N + gla::kProjTileTokens - 1) / gla::kProjTileTokens;
  if (tiles > 65535) return GLA_ERR_DIM;
  // the qg kernel's 1-D grid: B H tiles blocks of up to 512 threads, whose
  // work-item count must fit in 32 bits
  if ((long long)B * H * tiles * 512 > 0xFFFFFFFFLL) return GLA_ERR_DIM;
  return GLA_OK;
}

}  // namespace

extern "C" {

size_t gla_proj_workspace_bytes(int B, int N, int C, int H, int D) {
  size_t bytes = 0;
  if (check_proj_shape(B, N, C, H, D, &bytes) != GLA_OK || bytes == 0) return 0;
  return proj_layout(B, N, H, D).bytes;
}

int gla_forward_proj_check(const void* x, const void* w, const gla_rope_tables* rope,
                           const void* out, int B, int N, int C, int H, int D) {
  size_t bytes = 0;
  int rc = check_proj_shape(B, N, C, H, D, &bytes);
  if (rc) return rc;
  if (bytes == 0) return GLA_OK;
  if ((rc = check_rope(rope, N, D))) return rc;
  if (!x || !w || !out) return GLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return GLA_ERR_ALIGN;
  const size_t xb = (size_t)B * N * C * 2, wb = (size_t)4 * H * D * C * 2;
  if (overlap2(out, bytes, x, xb) || overlap2(out, bytes, w, wb)) return GLA_ERR_ALIAS;
  return check_plan_limits(gla::make_plan(B, N, H, D));
}

int gla_forward_proj_ws(const void* x, const void* w, const gla_rope_tables* rope, void* out,
                        int B, int N, int C, int H, int D, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int rc = gla_forward_proj_check(x, w, rope, out, B, N, C, H, D);
  if (rc) return rc;
  size_t bytes = 0;
  check_proj_shape(B, N, C, H, D, &bytes);
  if (bytes == 0) return GLA_OK;
  const ProjLayout l = proj_layout(B, N, H, D);
  if (!workspace) return GLA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < l.bytes)
    return GLA_ERR_WORKSPACE;
  const size_t xb = (size_t)B * N * C * 2, wb = (size_t)4 * H * D * C * 2;
  if (overlap2(workspace, l.bytes, x, xb) || overlap2(workspace, l.bytes, w, wb) ||
      overlap2(workspace, l.bytes, out, bytes))
    return GLA_ERR_ALIAS;
  if ((rc = rope_device_ok(rope))) return rc;
  const Plan& p = l.p;
  char* wsb = static_cast<char*>(workspace);
  gla::PArgs pa{};
  pa.x = static_cast<const uint16_t*>(x);
  pa.w = static_cast<const uint16_t*>(w);
  pa.Cdim = C;
  pa.qbuf = reinterpret_cast<uint16_t*>(wsb + l.off_q);
  pa.gbuf = reinterpret_cast<uint16_t*>(wsb + l.off_g);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // k, v -> state partials (chunks of the state plan); q, g -> workspace
  const gla::KArgs akv = kernel_args(p, rope, p.L, p.CB, workspace);
  const int tiles = (N + gla::kProjTileTokens - 1) / gla::kProjTileTokens;
  const gla::KArgs aqg = kernel_args(p, nullptr, gla::kProjTileTokens, tiles, workspace);
  if ((rc = status_of(gla::launch_proj(p, akv, aqg, pa, s)))) return rc;
  if ((rc = status_of(gla::launch_reduce_state(p, akv, s)))) return rc;
  return run_output(p, pa.qbuf, pa.gbuf, rope, out, workspace, stream);
}

int gla_forward_proj(const void* x, const void* w, const gla_rope_tables* rope, void* out, int B,
                     int N, int C, int H, int D, void* stream) {
  int rc = gla_forward_proj_check(x, w, rope, out, B, N, C, H, D);
  if (rc) return rc;
  const size_t need = gla_proj_workspace_bytes(B, N, C, H, D);
  if (need == 0) return GLA_OK;
  void* ws = nullptr;
  std::unique_lock<std::mutex> lk;
  if ((rc = get_workspace(need, stream, &ws, &lk))) return rc;
  return gla_forward_proj_ws(x, w, rope, out, B, N, C, H, D, ws, need, stream);
}

}  // extern "C"
