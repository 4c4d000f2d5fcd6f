/*
 * gla.h -- C ABI of the gated bidirectional linear-attention token mixer
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation ("SANA-Video 2.0", NVlabs Sana docs, section Architecture:
 * gated bidirectional linear-attention layers with Wan 3D rotary position
 * embeddings, BF16 inference per section Model zoo; "SANA-Video 2.0: Hybrid
 * Linear Attention with Attention Residuals ..." (mlsanity index), Abstract:
 * gated linear attention for the O(N) token mixing), per batch b and head h:
 *
 *     phi(u) = max(u, 0)
 *     S      = sum_n (R_n phi(k_n)) v_n^T        D x D, no causal mask
 *     z      = sum_n phi(k_n)                    D
 *     o_n    = sigmoid(g_n) * ((R_n phi(q_n))^T S) / (phi(q_n) . z + 1e-6)
 *
 * R_n is the 3D RoPE rotation of token n at latent-grid position (t, y, x):
 * the D/2 interleaved pairs (2i, 2i+1) are split into axis blocks t, y, x of
 * Pt = D/2 - 2*floor(D/6), Py = Px = floor(D/6) pairs; pair j of an axis
 * block with Pa pairs turns by (index + offset) * theta^(-2j / (2 Pa)).
 * Tokens are ordered n = (t*Hh + y)*W + x.  RoPE acts on the numerator only.
 *
 * Tensors.  q, k, v, g and out are device pointers to bf16 arrays of shape
 * [B, N, H, D], contiguous (element (b, n, h, d) at ((b*N + n)*H + h)*D + d),
 * each 16-byte aligned.  D must be 32, 64 or 128.  out must not overlap any
 * input.  The caller owns every tensor; the library never frees them.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the null stream) on the
 * current HIP device; every pointer must belong to that device.  Calls only
 * enqueue work and return without a host synchronisation, except where a
 * library-owned buffer has to grow (noted below).  Results are bitwise
 * reproducible for the same inputs, shape and device.
 *
 * Errors.  Every entry point returns an int status (GLA_OK or a negative
 * gla_status).  Arguments are validated before any HIP call, so a rejected
 * call has no side effect.  Faults inside a kernel surface at the caller's
 * next synchronisation, as with any HIP launch.  No C++ exception crosses
 * this interface.
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gla_status {
  GLA_OK = 0,
  GLA_ERR_NULL = -1,      /* a required pointer is NULL */
  GLA_ERR_ALIGN = -2,     /* a tensor pointer is not 16-byte aligned */
  GLA_ERR_DIM = -3,       /* D not in {32, 64, 128}; B, N or H negative; size overflow */
  GLA_ERR_ROPE = -4,      /* RoPE tables do not fit (T*Hh*W != N, other D, other device) */
  GLA_ERR_ALLOC = -5,     /* device memory allocation failed */
  GLA_ERR_LAUNCH = -6,    /* a kernel launch failed */
  GLA_ERR_ALIAS = -7,     /* out overlaps an input */
  GLA_ERR_WORKSPACE = -8, /* caller workspace too small or not 256-byte aligned */
  GLA_ERR_HIP = -9,       /* another HIP runtime call failed */
  GLA_ERR_SCRATCH = -10   /* gla_forward_noalloc: the call needs more than its fixed scratch */
};

/* Human-readable text of a status code (static storage, never NULL). */
const char* gla_strerror(int status);

/* ---------------------------------------------------------------------
 * 3D RoPE tables.
 *
 * The rotation factors are stored factorised per axis: (cos, sin) float
 * pairs of (index + offset) * omega_j for every grid index of each axis,
 * laid out as [T][Pt] | [Hh][Py] | [W][Px] pairs (t block first).  They are
 * computed in double precision on the host and rounded to float.  For the
 * 5B 720p/60s grid (181 x 22 x 40, D = 128) this is 42 KB, against 81.5 MB
 * for a dense per-token table.
 */
typedef struct gla_rope_tables {
  int32_t T, Hh, W;      /* latent grid: frames, rows, columns */
  int32_t D;             /* head dimension the tables were built for */
  int32_t Pt, Py, Px;    /* rotation pairs per axis; Pt + Py + Px = D/2 */
  int32_t t0, y0, x0;    /* index offsets added to every position */
  double theta;          /* RoPE base (10000 in the Wan convention) */
  const float* cs;       /* device pointer, 16-byte aligned: the (cos, sin) pairs above */
  size_t cs_floats;      /* number of floats behind cs */
  int32_t device;        /* HIP device that holds cs */
} gla_rope_tables;

/* Number of floats the (cos, sin) table of a grid takes, 0 for bad sizes. */
size_t gla_rope_table_floats(int T, int Hh, int W, int D);

/* Fills a HOST buffer of `cs_floats` floats with the table described above
 * (no GPU needed).  D must be even and >= 2; T, Hh, W >= 1. */
int gla_rope_fill_host(int T, int Hh, int W, int D, double theta, int t0, int y0, int x0,
                       float* cs, size_t cs_floats);

/* Builds the table on the host, copies it to the current device (enqueued on
 * `stream`, then synchronised so the host copy can be released) and returns
 * a library-owned descriptor in *out.  D must be 32, 64, 128 or 256 (256 for
 * the softmax anchor layers only). */
int gla_rope_create(int T, int Hh, int W, int D, double theta, int t0, int y0, int x0,
                    void* stream, gla_rope_tables** out);

/* Releases a descriptor from gla_rope_create (NULL is a no-op).  The caller
 * must make sure no enqueued gla_forward still reads it. */
int gla_rope_destroy(gla_rope_tables* tables);

/* ---------------------------------------------------------------------
 * Forward pass.
 */

/* Bytes of device workspace gla_forward_ws needs for this shape (per-chunk
 * partial states and the reduced bf16 state).  0 for N*B*H == 0. */
size_t gla_workspace_bytes(int B, int N, int H, int D);

/* Runs the mixer: out = o as defined above, bf16, round-to-nearest-even.
 * rope == NULL switches RoPE off (identical to all angles being zero).
 * Uses a library-owned workspace cached per (device, stream); growing it
 * calls hipMalloc, which may synchronise.  Calls that share one stream are
 * ordered by it; do not run two calls on the same stream from two host
 * threads at once.  B*N*H == 0 is a no-op that returns GLA_OK. */
int gla_forward(const void* q, const void* k, const void* v, const void* g,
                const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                void* stream);

/* Frees the library-owned workspaces of the current device: the ones
 * gla_forward, gla_forward_blocks, gla_softmax_forward, gla_backward,
 * gla_backward_saved and gla_forward_proj cache per (device, stream) and
 * otherwise keep until the process ends.  It first synchronises the device
 * (hipDeviceSynchronize), so every kernel that may still read one of them
 * has finished; the next call that needs a workspace allocates a new one.
 * Caller-owned workspaces, RoPE tables and gla_forward_noalloc's fixed
 * scratch are not touched.  Returns GLA_OK (also when nothing is cached) or
 * GLA_ERR_HIP if the synchronisation or a hipFree fails; a device fault of
 * earlier work surfaces here as GLA_ERR_HIP.  Do not call it while a stream
 * of the device is being captured into a HIP graph: a device synchronisation
 * is not allowed then, and the capture would be invalidated. */
int gla_workspace_release(void);

/* Same as gla_forward with a caller-owned device workspace (>= the size
 * gla_workspace_bytes returns, 256-byte aligned, overlapping none of the
 * tensors: GLA_ERR_ALIAS otherwise).  The workspace must not be used by
 * other work while this call's kernels run.  Never allocates.  Short passes
 * (D <= 64) may run in fewer launches and use less of the workspace (one
 * launch with none of it for N * D <= 32768); the result does not depend on
 * the workspace's contents either way. */
int gla_forward_ws(const void* q, const void* k, const void* v, const void* g,
                   const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                   void* workspace, size_t workspace_bytes, void* stream);

/* gla_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * calls no hipMalloc, hipFree or allocating library routine.  Instead of a
 * workspace it uses a fixed 32 MiB scratch array in device memory that the
 * library holds on each GPU it runs on until the process ends; calls whose
 * gla_workspace_bytes exceed 32 MiB (33554432 bytes) return GLA_ERR_SCRATCH
 * before any HIP call (at D = 128 every shape with B*H <= 256 fits).  All
 * calls on one GPU share that array, so calls that overlap in time on one
 * GPU (other streams, other host threads) race and must be serialised by the
 * caller.  Nothing in the scratch needs to start at zero: each call writes
 * all of it that it reads.  Arguments, results and errors otherwise as for
 * gla_forward; the first call on a device also looks up the array's device
 * address (GLA_ERR_HIP if that fails). */
int gla_forward_noalloc(const void* q, const void* k, const void* v, const void* g,
                        const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                        void* stream);

/* Argument validation of gla_forward alone: returns the status gla_forward
 * would return before touching the GPU (GLA_OK if the arguments are valid).
 * Makes no HIP call, so it runs on hosts without a GPU. */
int gla_forward_check(const void* q, const void* k, const void* v, const void* g,
                      const gla_rope_tables* rope, const void* out, int B, int N, int H, int D);

/* The two halves of gla_forward_ws, for callers that schedule them apart
 * (timing each half, or exchanging the state between them).  gla_state_ws
 * reads k and v and leaves the reduced state of every head in `workspace`;
 * gla_output_ws reads q and g and that state and writes out.  Calling both
 * in order on one stream with one workspace equals gla_forward_ws.  The
 * workspace contents between the two calls are private to the library. */
int gla_state_ws(const void* k, const void* v, const gla_rope_tables* rope,
                 int B, int N, int H, int D, void* workspace, size_t workspace_bytes,
                 void* stream);
int gla_output_ws(const void* q, const void* g, const gla_rope_tables* rope, void* out,
                  int B, int N, int H, int D, void* workspace, size_t workspace_bytes,
                  void* stream);

/* The state half of the pass: S (fp32 [B, H, D, D], S[d][e]) and z (fp32
 * [B, H, D]) into caller device buffers (16-byte aligned, not overlapping
 * k or v), with the same kernels and reduction order gla_forward uses.
 * k, v, rope as for gla_forward (k and v may be NULL when N == 0; S and z
 * are then set to zero).  Uses the library-owned workspace. */
int gla_state(const void* k, const void* v, const gla_rope_tables* rope, float* S, float* z,
              int B, int N, int H, int D, void* stream);

/* ---------------------------------------------------------------------
 * Block-causal pass with a carried state.
 *
 * The constant-memory KV cache of block linear attention ("SANA-Video_2B_720p"
 * model card, innovation (2): blocks are generated one after another, and the
 * cumulative state of linear attention carries the context of everything
 * before at a fixed memory cost).  The N tokens of a head form blocks of
 * block_tokens tokens in order (the last block may be shorter).  Token n in
 * block b = n / block_tokens sees every token up to the end of its own block,
 * plus a carried state (S_in, z_in) from earlier calls:
 *
 *     S_<=b = S_in + sum over tokens m with m / block_tokens <= b of
 *             (R_m phi(k_m)) v_m^T
 *     z_<=b = z_in + sum over the same tokens of phi(k_m)
 *     o_n   = sigmoid(g_n) * ((R_n phi(q_n))^T S_<=b) / (phi(q_n) . z_<=b + 1e-6)
 *
 * The state after the last block goes to S_out, z_out; a next call takes it
 * as its carried state (with the RoPE tables' t0 moved on by the frames of
 * this call).  block_tokens >= N with no carried state equals gla_forward.
 *
 * q, k, v, g, out, rope: as for gla_forward.  block_tokens >= 1.
 * S_in, S_out: device fp32 [B, H, D, D] (element S[d][e] at
 * ((b*H + h)*D + d)*D + e); z_in, z_out: device fp32 [B, H, D].  Each may be
 * NULL (a NULL carried state is zero; a NULL returned state is not
 * written).  Given ones are 16-byte aligned and overlap no bf16 tensor;
 * S_out may be S_in itself (and z_out z_in), which updates the state in
 * place, but may not partly overlap it or any other state.  The caller owns
 * all of them.
 * Limits (GLA_ERR_DIM): at most 65535 blocks per head, and each head's
 * partial states (one D*D + D fp32 set per state chunk) under 2 GiB.  N == 0 with B*H > 0 only copies the carried state to
 * the returned one (zero if none).  Uses a library-owned workspace as
 * gla_forward does.  Results are bitwise reproducible. */
int gla_forward_blocks(const void* q, const void* k, const void* v, const void* g,
                       const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                       int block_tokens, const float* S_in, const float* z_in, float* S_out,
                       float* z_out, void* stream);

/* Workspace bytes gla_forward_blocks_ws needs: per-chunk partial states and
 * one bf16 state per head and block.  0 for B*N*H == 0 or block_tokens < 1. */
size_t gla_workspace_bytes_blocks(int B, int N, int H, int D, int block_tokens);

/* gla_forward_blocks with a caller-owned workspace (>= the size
 * gla_workspace_bytes_blocks returns, 256-byte aligned, overlapping no
 * tensor or state; may be NULL when N == 0).  Never allocates. */
int gla_forward_blocks_ws(const void* q, const void* k, const void* v, const void* g,
                          const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                          int block_tokens, const float* S_in, const float* z_in, float* S_out,
                          float* z_out, void* workspace, size_t workspace_bytes, void* stream);

/* Argument validation of gla_forward_blocks alone (no HIP call). */
int gla_forward_blocks_check(const void* q, const void* k, const void* v, const void* g,
                             const gla_rope_tables* rope, const void* out, int B, int N, int H,
                             int D, int block_tokens, const float* S_in, const float* z_in,
                             const float* S_out, const float* z_out);

/* ---------------------------------------------------------------------
 * Gated softmax anchor attention.
 *
 * The dense softmax layers of the hybrid ("SANA-Video 2.0", NVlabs Sana
 * docs, section Architecture: a quarter of the layers are dense softmax
 * anchors, 10 heads x 256 at 5B and 16 heads x 256 at 14B, with Wan 3D rotary
 * position embeddings; "SANA-Video 2.0: Hybrid Linear Attention with
 * Attention Residuals ..." (mlsanity index), Abstract: periodic gated-softmax
 * anchors).  Per batch b and head h, with no mask:
 *
 *     o_n = sigmoid(g_n) * sum_m softmax_m(R_n q_n . R_m k_m / sqrt(D)) v_m
 *
 * RoPE (the same tables as above, built for this D) turns q and k
 * themselves; rope == NULL switches it off.  q, k, v, g, out: device bf16
 * [B, N, H, D] as for gla_forward, 16-byte aligned, out overlapping no input;
 * D must be 128 or 256.  The scores, the softmax (online, base 2) and the
 * value sums run in fp32 on bf16 MFMA with q scaled by log2(e)/sqrt(D) and q
 * and k rotated into bf16 copies first.  Uses a library-owned workspace
 * (grown with hipMalloc, which may synchronise).  B*N*H == 0 is a no-op.
 * Results are bitwise reproducible. */
int gla_softmax_forward(const void* q, const void* k, const void* v, const void* g,
                        const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                        void* stream);

/* Workspace bytes gla_softmax_forward_ws needs (the rotated q and k), 0 for
 * bad shapes or B*N*H == 0. */
size_t gla_softmax_workspace_bytes(int B, int N, int H, int D);

/* gla_softmax_forward with a caller-owned device workspace (>= the size
 * above, 256-byte aligned, overlapping no tensor).  Never allocates. */
int gla_softmax_forward_ws(const void* q, const void* k, const void* v, const void* g,
                           const gla_rope_tables* rope, void* out, int B, int N, int H, int D,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Argument validation of gla_softmax_forward alone (no HIP call). */
int gla_softmax_forward_check(const void* q, const void* k, const void* v, const void* g,
                              const gla_rope_tables* rope, const void* out, int B, int N, int H,
                              int D);

/* ---------------------------------------------------------------------
 * Backward pass of the bidirectional mixer.
 *
 * The exact derivative of gla_forward, for training the linear layers
 * ("SANA-Video 2.0: Hybrid Linear Attention with Attention Residuals ..."
 * (mlsanity index), Abstract: the hybrid is trained; the pages give no
 * formula, so this is the chain rule through the form at the top of this
 * file).  Given dout = dL/dout, per batch b and head h, with
 * fq = phi(q_n), rq = R_n fq, den = fq . z + 1e-6, s = sigmoid(g_n),
 * num = S^T rq and o_n = s * num / den:
 *
 *     dg_n = dout_n * o_n * (1 - s)
 *     a_n  = dout_n * s / den,         dden_n = -(dout_n . o_n) / den
 *     dq_n = [q_n > 0] * (R_n^T (S a_n) + dden_n z)
 *     dS   = sum_n rq a_n^T,           dz = sum_n dden_n fq
 *     dv_m = dS^T (R_m phi(k_m))
 *     dk_m = [k_m > 0] * (R_m^T (dS v_m) + dz)
 *
 * The derivative of phi at 0 is taken as 0.  q, k, v, g, dout: device bf16
 * [B, N, H, D] inputs; dq, dk, dv, dg: device bf16 [B, N, H, D] outputs
 * (written in full), each 16-byte aligned, overlapping no input and no
 * other output.  D must be 32, 64 or 128; rope as for gla_forward (NULL:
 * RoPE off).  S and z are recomputed from k and v (no saved state is
 * needed; gla_backward_saved below takes the forward's).  The contractions
 * run on bf16 MFMA with fp32 accumulation: S, dS, the rotated features and
 * a_n are rounded to bf16 as MFMA operands.  Uses
 * a library-owned workspace (grown with hipMalloc, which may synchronise).
 * B*N*H == 0 is a no-op.  Results are bitwise reproducible. */
int gla_backward(const void* q, const void* k, const void* v, const void* g, const void* dout,
                 const gla_rope_tables* rope, void* dq, void* dk, void* dv, void* dg, int B,
                 int N, int H, int D, void* stream);

/* Workspace bytes gla_backward_ws needs (the forward's partials and state
 * operands, the S rows operand, z, and one fp32 dS and dz partial of
 * D*D + D floats per head and token range), 0 for bad shapes or
 * B*N*H == 0. */
size_t gla_backward_workspace_bytes(int B, int N, int H, int D);

/* gla_backward with a caller-owned device workspace (>= the size above,
 * 256-byte aligned, overlapping no tensor).  Never allocates. */
int gla_backward_ws(const void* q, const void* k, const void* v, const void* g, const void* dout,
                    const gla_rope_tables* rope, void* dq, void* dk, void* dv, void* dg, int B,
                    int N, int H, int D, void* workspace, size_t workspace_bytes, void* stream);

/* Argument validation of gla_backward alone (no HIP call). */
int gla_backward_check(const void* q, const void* k, const void* v, const void* g,
                       const void* dout, const gla_rope_tables* rope, const void* dq,
                       const void* dk, const void* dv, const void* dg, int B, int N, int H,
                       int D);

/* gla_backward with the forward's state passed in instead of recomputed.
 * S: device fp32 [B*H][D][D], S = sum_n R_n phi(k_n) v_n^T per head; z:
 * device fp32 [B*H][D], z = sum_n phi(k_n): exactly what
 * gla_forward_blocks returns in S_out and z_out with block_tokens >= N
 * (one attention block: the bidirectional mixer, whose output equals
 * gla_forward's) for the same q, k, v, g and rope.  Both are read only,
 * 16-byte aligned, and overlap no output.  With that state the results are
 * bitwise those of gla_backward (which forms the same fp32 sums itself);
 * the pass skips the read of k and v that forms them.  Any other S and z
 * give the gradients at that state.  Workspace as for gla_backward. */
int gla_backward_saved(const void* q, const void* k, const void* v, const void* g,
                       const void* dout, const gla_rope_tables* rope, const float* S,
                       const float* z, void* dq, void* dk, void* dv, void* dg, int B, int N, int H,
                       int D, void* stream);

/* gla_backward_saved with a caller-owned device workspace of
 * gla_backward_workspace_bytes (256-byte aligned, overlapping no tensor, S
 * or z).  Never allocates. */
int gla_backward_saved_ws(const void* q, const void* k, const void* v, const void* g,
                          const void* dout, const gla_rope_tables* rope, const float* S,
                          const float* z, void* dq, void* dk, void* dv, void* dg, int B, int N,
                          int H, int D, void* workspace, size_t workspace_bytes, void* stream);

/* Argument validation of gla_backward_saved alone (no HIP call). */
int gla_backward_saved_check(const void* q, const void* k, const void* v, const void* g,
                             const void* dout, const gla_rope_tables* rope, const float* S,
                             const float* z, const void* dq, const void* dk, const void* dv,
                             const void* dg, int B, int N, int H, int D);

/* ---------------------------------------------------------------------
 * Projection prologue fused with the mixer.
 *
 * The step before the mixer in a linear layer ("SANA-Video 2.0", NVlabs
 * Sana docs, section Architecture: hidden size 2,560 with 20 heads x 128 at
 * 5B, 4,096 with 32 heads x 128 at 14B; section Model zoo: BF16 inference).
 * The pages give no further detail of the projections; read as four
 * bias-free linear maps of the hidden states, each stored in bf16:
 *
 *     q = bf16(x Wq^T),  k = bf16(x Wk^T),  v = bf16(x Wv^T),  g = bf16(x Wg^T)
 *
 * followed by gla_forward on (q, k, v, g).  x: device bf16 [B, N, C]
 * (C = hidden size, a multiple of 64); w: device bf16 [4][H*D][C], the four
 * maps stacked in the order q, k, v, g, row j of a map being output feature
 * j (h*D + d) contiguous over C (the [out, in] layout of a linear layer);
 * out: device bf16 [B, N, H, D], overlapping neither x nor w; all 16-byte
 * aligned.  D must be 32, 64 or 128; rope as for gla_forward.  The GEMMs
 * run on bf16 MFMA with fp32 accumulation; k and v never reach device
 * memory (the state is contracted from them in the GEMM's epilogue), q and
 * g go through the workspace.  Limits (GLA_ERR_DIM): N*C*2 and 4*H*D*C*2
 * below 2 GiB, ceil(N / 256) <= 65535 and B*H*ceil(N / 256) <= 8,388,607.
 * Uses a library-owned workspace (grown with hipMalloc, which may
 * synchronise).  B*N*H == 0 is a no-op.  Results are bitwise reproducible. */
int gla_forward_proj(const void* x, const void* w, const gla_rope_tables* rope, void* out, int B,
                     int N, int C, int H, int D, void* stream);

/* Workspace bytes gla_forward_proj_ws needs (the state partials and operand
 * and the projected q and g), 0 for bad shapes or B*N*H == 0. */
size_t gla_proj_workspace_bytes(int B, int N, int C, int H, int D);

/* gla_forward_proj with a caller-owned device workspace (>= the size above,
 * 256-byte aligned, overlapping no tensor).  Never allocates. */
int gla_forward_proj_ws(const void* x, const void* w, const gla_rope_tables* rope, void* out,
                        int B, int N, int C, int H, int D, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Argument validation of gla_forward_proj alone (no HIP call). */
int gla_forward_proj_check(const void* x, const void* w, const gla_rope_tables* rope,
                           const void* out, int B, int N, int C, int H, int D);

/* ---------------------------------------------------------------------
 * Bandwidth probe (a measurement aid, not part of the mixer).
 *
 * Streams `bytes` (a multiple of 16, below 2 GiB) of each of two device
 * buffers through the load path the mixer's kernels use (16-byte buffer
 * loads with the non-temporal hint, 16 KB contiguous per block):
 *   mode 0: reads src0 and src1 (the state half's two read streams);
 *   mode 1: also writes dst = src0 ^ src1 with non-temporal stores (the
 *           output half's two reads and one write).
 * dst must hold `bytes` (mode 0 may write at most 4 KB of it).  Pointers
 * 16-byte aligned; GLA_ERR_NULL / GLA_ERR_ALIGN / GLA_ERR_DIM before any HIP
 * call.  Enqueued on `stream`; the caller times it. */
int gla_stream_probe(const void* src0, const void* src1, void* dst, size_t bytes, int mode,
                     void* stream);

/* The same probe for any mix of `nsrc` (1..3) read streams and `ndst` (1..2)
 * write streams, `bytes` of each buffer (the backward pass's query kernel
 * reads three tensors and writes two, its key kernel reads two and writes
 * two).  srcs and dsts are host arrays of device pointers; every destination
 * receives the XOR of the sources, written with non-temporal stores.  Same
 * rules and error codes as gla_stream_probe (GLA_ERR_DIM also for nsrc or
 * ndst out of range), all checked before any HIP call. */
int gla_stream_probe_mix(const void* const* srcs, int nsrc, void* const* dsts, int ndst,
                         size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
