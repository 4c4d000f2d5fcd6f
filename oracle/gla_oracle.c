/*
 * gla_oracle.c -- plain fp64 CPU oracle for the gated bidirectional
 * linear-attention token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers.  The product library
 * never links, loads or calls this file, and this file includes nothing
 * from the product (no shared headers, tables or helpers).
 *
 * What is computed (the method, as the pages describe it):
 *   - "SANA-Video 2.0" (NVlabs Sana docs), section Architecture: 75% of the
 *     layers are gated *bidirectional* linear attention, positions use Wan 3D
 *     rotary embeddings, latent patches are (1,1,1).
 *   - "SANA-Video 2.0: Hybrid Linear Attention with Attention Residuals for
 *     Efficient Video Generation" (mlsanity index), Abstract: gated linear
 *     attention does the O(N) mixing.
 * The pages give no formula.  The fixed form followed here, per (b, h):
 *     phi(u) = max(u, 0)                              (feature map)
 *     R_n    = block-diagonal rotation of token n     (3D RoPE)
 *     S      = sum_n (R_n phi(k_n)) v_n^T             (D x D)
 *     z      = sum_n phi(k_n)                         (D)
 *     o_n[e] = sigmoid(g_n[e]) * ((R_n phi(q_n))^T S)[e] / (phi(q_n).z + eps)
 * "Bidirectional" is read as: no causal mask, S and z sum over all N tokens.
 * gla_oracle_forward_blocks adds the block-causal form with a carried state
 * (the constant-memory KV cache for block linear attention of the
 * "SANA-Video_2B_720p" model card, innovation (2)); gla_oracle_softmax_rows
 * the gated softmax anchor attention of the other quarter of the layers;
 * gla_oracle_backward and its row/state helpers the exact derivative of the
 * bidirectional mixer; gla_oracle_project the linear maps that produce q, k,
 * v and g from the hidden states; see their comments.
 *
 * RoPE reading (the pages only name "Wan 3D rotary position embeddings"):
 *   - the D/2 rotation pairs are (2i, 2i+1), interleaved;
 *   - pairs are split into axis blocks in the order (t, y, x) with
 *     Py = Px = floor(D/6) and Pt = D/2 - 2*floor(D/6);
 *   - pair j of an axis block with Pa pairs has frequency
 *     omega_j = theta^(-2j / (2 Pa)), theta = 10000 by default;
 *   - the angle is (grid index + offset) * omega_j;
 *   - the rotation of (a, b) by angle w is (a cos w - b sin w, a sin w + b cos w);
 *   - RoPE is applied after phi, to q and k in the numerator only; the
 *     denominator uses the unrotated features.
 * Token order: n = (t*Hh + y)*W + x, row-major over the latent grid.
 *
 * Arithmetic: every input is a bf16 bit pattern widened exactly to double;
 * all arithmetic is IEEE double in the order written; nothing is blocked,
 * fused or reordered beyond the definition above.  OpenMP runs independent
 * (b, h) heads in parallel; each head's sums run sequentially over n.
 *
 * Pins (what checks this file against something other than itself) live in
 * tests/test_oracle.py: quadratic brute force, hand-derived closed forms,
 * rotation invariants, special cases.  The frequency constants omega_j are
 * a reading of the pages and are "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_ARG = -1,
  ORACLE_ERR_GRID = -2,
  ORACLE_ERR_ALLOC = -3
};

/* Grid description used when RoPE is on.  rope == NULL means RoPE off. */
typedef struct {
  int T, Hh, W;          /* latent grid: frames, rows, columns */
  double theta;          /* RoPE base */
  long t0, y0, x0;       /* offsets added to every grid index */
} oracle_grid;

/* Exact widening of a bf16 bit pattern: bf16 is the top half of an IEEE
 * binary32, so shifting the 16 bits up gives the same value as a float. */
double gla_oracle_bf16_to_f64(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int gla_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Pair counts of the (t, y, x) axis blocks for head dimension D. */
void gla_oracle_axis_split(int D, int* Pt, int* Py, int* Px) {
  int P = D / 2;
  *Py = D / 6;
  *Px = D / 6;
  *Pt = P - 2 * (D / 6);
}

/* Rotation angle of pair p for a token at grid indices (t, y, x), offsets
 * already included. */
double gla_oracle_angle(int D, double theta, int p, long t, long y, long x) {
  int Pt, Py, Px;
  gla_oracle_axis_split(D, &Pt, &Py, &Px);
  long pos;
  int j, Pa;
  if (p < Pt) {
    pos = t; j = p; Pa = Pt;
  } else if (p < Pt + Py) {
    pos = y; j = p - Pt; Pa = Py;
  } else {
    pos = x; j = p - Pt - Py; Pa = Px;
  }
  double omega = pow(theta, -2.0 * (double)j / (2.0 * (double)Pa));
  return (double)pos * omega;
}

/* Grid indices of token n (offsets included). */
static void token_position(const oracle_grid* gr, long n, long* t, long* y, long* x) {
  long HW = (long)gr->Hh * gr->W;
  *t = n / HW + gr->t0;
  *y = (n / gr->W) % gr->Hh + gr->y0;
  *x = n % gr->W + gr->x0;
}

/* out = R_n u for token n; with rope == NULL the rotation is the identity. */
static void rotate(int D, const oracle_grid* gr, long n, const double* u, double* out) {
  if (gr == NULL) {
    for (int d = 0; d < D; ++d) out[d] = u[d];
    return;
  }
  long t, y, x;
  token_position(gr, n, &t, &y, &x);
  for (int p = 0; p < D / 2; ++p) {
    double w = gla_oracle_angle(D, gr->theta, p, t, y, x);
    double c = cos(w), s = sin(w);
    double a = u[2 * p], b = u[2 * p + 1];
    out[2 * p] = a * c - b * s;
    out[2 * p + 1] = a * s + b * c;
  }
}

/* Public wrapper of the rotation, so tests can check it in isolation:
 * u and out hold D doubles for token n of the grid. */
int gla_oracle_rotate(int D, int T, int Hh, int W, double theta, long t0, long y0, long x0,
                      long n, const double* u, double* out) {
  if (D <= 0 || (D & 1) || T <= 0 || Hh <= 0 || W <= 0) return ORACLE_ERR_ARG;
  oracle_grid gr = {T, Hh, W, theta, t0, y0, x0};
  rotate(D, &gr, n, u, out);
  return ORACLE_OK;
}

static double relu(double u) { return u > 0.0 ? u : 0.0; }

static double sigmoid(double u) { return 1.0 / (1.0 + exp(-u)); }

/* Widen the D-vector of token n, head (b, h) from a [B, N, H, D] bf16 array. */
static void load_row(const uint16_t* a, int N, int H, int D, int b, int h, long n, double* out) {
  const uint16_t* p = a + (((long)b * N + n) * H + h) * (long)D;
  for (int d = 0; d < D; ++d) out[d] = gla_oracle_bf16_to_f64(p[d]);
}

static int check_args(int B, int N, int H, int D, const oracle_grid* gr) {
  if (B < 0 || N < 0 || H < 0 || D <= 0 || (D & 1)) return ORACLE_ERR_ARG;
  if (gr != NULL) {
    if (gr->T <= 0 || gr->Hh <= 0 || gr->W <= 0) return ORACLE_ERR_GRID;
    if ((long)gr->T * gr->Hh * gr->W != (long)N) return ORACLE_ERR_GRID;
  }
  return ORACLE_OK;
}

/* Adds the terms of tokens n0 .. n1-1 of head (b, h), in order:
 * S[d*D + e] += (R_n phi(k_n))[d] v_n[e],  z[d] += phi(k_n)[d]. */
static int add_range(const uint16_t* k, const uint16_t* v, int N, int H, int D,
                     const oracle_grid* gr, int b, int h, long n0, long n1, double* S, double* z) {
  double* fk = malloc(sizeof(double) * D);
  double* rk = malloc(sizeof(double) * D);
  double* vr = malloc(sizeof(double) * D);
  if (!fk || !rk || !vr) {
    free(fk); free(rk); free(vr);
    return ORACLE_ERR_ALLOC;
  }
  for (long n = n0; n < n1; ++n) {
    load_row(k, N, H, D, b, h, n, fk);
    load_row(v, N, H, D, b, h, n, vr);
    for (int d = 0; d < D; ++d) fk[d] = relu(fk[d]);
    rotate(D, gr, n, fk, rk);
    for (int d = 0; d < D; ++d) {
      z[d] += fk[d];
      for (int e = 0; e < D; ++e) S[(long)d * D + e] += rk[d] * vr[e];
    }
  }
  free(fk); free(rk); free(vr);
  return ORACLE_OK;
}

/* First pass for head (b, h): S[d*D + e] = sum_n (R_n phi(k_n))[d] v_n[e],
 * z[d] = sum_n phi(k_n)[d].  Sums run over n = 0 .. N-1 in order. */
static int head_state(const uint16_t* k, const uint16_t* v, int N, int H, int D,
                      const oracle_grid* gr, int b, int h, double* S, double* z) {
  memset(S, 0, sizeof(double) * D * D);
  memset(z, 0, sizeof(double) * D);
  return add_range(k, v, N, H, D, gr, b, h, 0, N, S, z);
}

/* Second pass for one token n of head (b, h), given that head's S and z. */
static void head_row(const uint16_t* q, const uint16_t* g, int N, int H, int D,
                     const oracle_grid* gr, int b, int h, const double* S, const double* z,
                     double eps, long n, double* fq, double* rq, double* gr_row, double* out) {
  load_row(q, N, H, D, b, h, n, fq);
  load_row(g, N, H, D, b, h, n, gr_row);
  for (int d = 0; d < D; ++d) fq[d] = relu(fq[d]);
  rotate(D, gr, n, fq, rq);
  double den = 0.0;
  for (int d = 0; d < D; ++d) den += fq[d] * z[d];
  den += eps;
  for (int e = 0; e < D; ++e) {
    double num = 0.0;
    for (int d = 0; d < D; ++d) num += rq[d] * S[(long)d * D + e];
    out[e] = sigmoid(gr_row[e]) * num / den;
  }
}

static int make_grid(int rope, int T, int Hh, int W, double theta, long t0, long y0, long x0,
                     oracle_grid* gr, const oracle_grid** out) {
  if (!rope) {
    *out = NULL;
    return ORACLE_OK;
  }
  gr->T = T; gr->Hh = Hh; gr->W = W; gr->theta = theta;
  gr->t0 = t0; gr->y0 = y0; gr->x0 = x0;
  *out = gr;
  return ORACLE_OK;
}

/* State (S, z) of every head.  S: [B, H, D, D], z: [B, H, D], doubles.
 * rope == 0 switches RoPE off (T, Hh, W, theta and offsets are then ignored). */
int gla_oracle_state(const uint16_t* k, const uint16_t* v, int B, int N, int H, int D,
                     int rope, int T, int Hh, int W, double theta, long t0, long y0, long x0,
                     double* S, double* z) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  int err = ORACLE_OK;
  long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    int b = (int)(bh / H), h = (int)(bh % H);
    int r = head_state(k, v, N, H, D, gr, b, h, S + bh * D * (long)D, z + bh * D);
    if (r) {
#pragma omp critical
      err = r;
    }
  }
  return err;
}

/* Outputs of selected tokens of one head (b, h), given that head's S and z
 * (layout as gla_oracle_state writes for one head).  out: [nrows, D]. */
int gla_oracle_rows(const uint16_t* q, const uint16_t* g, int B, int N, int H, int D,
                    int rope, int T, int Hh, int W, double theta, long t0, long y0, long x0,
                    int b, int h, const double* S, const double* z, double eps,
                    const long* rows, long nrows, double* out) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  if (b < 0 || b >= B || h < 0 || h >= H) return ORACLE_ERR_ARG;
  for (long i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= N) return ORACLE_ERR_ARG;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* fq = malloc(sizeof(double) * D);
    double* rq = malloc(sizeof(double) * D);
    double* gv = malloc(sizeof(double) * D);
    if (!fq || !rq || !gv) {
#pragma omp critical
      err = ORACLE_ERR_ALLOC;
    } else {
#pragma omp for schedule(static)
      for (long i = 0; i < nrows; ++i)
        head_row(q, g, N, H, D, gr, b, h, S, z, eps, rows[i], fq, rq, gv, out + i * D);
    }
    free(fq); free(rq); free(gv);
  }
  return err;
}

/* Whole forward pass: out[B, N, H, D] (doubles) from bf16 q, k, v, g. */
int gla_oracle_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                       int B, int N, int H, int D,
                       int rope, int T, int Hh, int W, double theta, long t0, long y0, long x0,
                       double eps, double* out) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  int err = ORACLE_OK;
  long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    int b = (int)(bh / H), h = (int)(bh % H);
    double* S = malloc(sizeof(double) * D * (long)D);
    double* z = malloc(sizeof(double) * D);
    double* fq = malloc(sizeof(double) * D);
    double* rq = malloc(sizeof(double) * D);
    double* gv = malloc(sizeof(double) * D);
    double* row = malloc(sizeof(double) * D);
    int r = (S && z && fq && rq && gv && row) ? ORACLE_OK : ORACLE_ERR_ALLOC;
    if (!r) r = head_state(k, v, N, H, D, gr, b, h, S, z);
    if (!r) {
      for (long n = 0; n < N; ++n) {
        head_row(q, g, N, H, D, gr, b, h, S, z, eps, n, fq, rq, gv, row);
        double* dst = out + (((long)b * N + n) * H + h) * (long)D;
        for (int e = 0; e < D; ++e) dst[e] = row[e];
      }
    }
    free(S); free(z); free(fq); free(rq); free(gv); free(row);
    if (r) {
#pragma omp critical
      err = r;
    }
  }
  return err;
}

/* Block-causal form with a carried state: the constant-memory KV cache for
 * block linear attention ("SANA-Video_2B_720p" model card, innovation (2):
 * blocks are generated one after another and the cumulative state of linear
 * attention carries the context of everything before).  Tokens are split
 * into blocks of L tokens in order (the last block may be shorter); token n
 * in block n / L sees every token up to the end of its own block, plus a
 * carried state (S_in, z_in) from earlier calls:
 *     S_<=b = S_in + sum over tokens m with m / L <= b of (R_m phi(k_m)) v_m^T
 *     z_<=b = z_in + sum over the same tokens of phi(k_m)
 *     o_n   = sigmoid(g_n) * ((R_n phi(q_n))^T S_<=b) / (phi(q_n).z_<=b + eps)
 * with b = n / L.  S_in, z_in ([B, H, D, D] and [B, H, D]) may be NULL
 * (zero).  S_out, z_out, when not NULL, receive the state after the last
 * block, which a next call takes as its carried state.  L >= N with no
 * carried state is the bidirectional mixer of gla_oracle_forward.
 * The sums run block after block, tokens in order within a block. */
int gla_oracle_forward_blocks(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const uint16_t* g, int B, int N, int H, int D,
                              int rope, int T, int Hh, int W, double theta, long t0, long y0,
                              long x0, double eps, long L, const double* S_in, const double* z_in,
                              double* out, double* S_out, double* z_out) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  if (L <= 0) return ORACLE_ERR_ARG;
  int err = ORACLE_OK;
  long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    int b = (int)(bh / H), h = (int)(bh % H);
    double* S = malloc(sizeof(double) * D * (long)D);
    double* z = malloc(sizeof(double) * D);
    double* fq = malloc(sizeof(double) * D);
    double* rq = malloc(sizeof(double) * D);
    double* gv = malloc(sizeof(double) * D);
    double* row = malloc(sizeof(double) * D);
    int r = (S && z && fq && rq && gv && row) ? ORACLE_OK : ORACLE_ERR_ALLOC;
    if (!r) {
      for (long i = 0; i < (long)D * D; ++i) S[i] = S_in ? S_in[bh * D * (long)D + i] : 0.0;
      for (int d = 0; d < D; ++d) z[d] = z_in ? z_in[bh * D + d] : 0.0;
      for (long n0 = 0; n0 < N && !r; n0 += L) {
        long n1 = n0 + L < N ? n0 + L : N;
        r = add_range(k, v, N, H, D, gr, b, h, n0, n1, S, z);
        for (long n = n0; n < n1 && !r; ++n) {
          head_row(q, g, N, H, D, gr, b, h, S, z, eps, n, fq, rq, gv, row);
          double* dst = out + (((long)b * N + n) * H + h) * (long)D;
          for (int e = 0; e < D; ++e) dst[e] = row[e];
        }
      }
      if (!r && S_out)
        for (long i = 0; i < (long)D * D; ++i) S_out[bh * D * (long)D + i] = S[i];
      if (!r && z_out)
        for (int d = 0; d < D; ++d) z_out[bh * D + d] = z[d];
    }
    free(S); free(z); free(fq); free(rq); free(gv); free(row);
    if (r) {
#pragma omp critical
      err = r;
    }
  }
  return err;
}

/* ---------------------------------------------------------------------------
 * Gated softmax anchor attention: the dense softmax layers of the hybrid
 * ("SANA-Video 2.0" NVlabs Sana docs, section Architecture: a quarter of the
 * layers are dense softmax anchors, 10 heads x 256 at 5B and 16 x 256 at
 * 14B, with the same Wan 3D rotary embeddings; "SANA-Video 2.0: Hybrid
 * Linear Attention with Attention Residuals for Efficient Video Generation"
 * (mlsanity index), Abstract: periodic gated-softmax anchors).  The reading
 * taken, per (b, h), with no mask:
 *     rq_n = R_n q_n,  rk_m = R_m k_m            (RoPE on q and k themselves)
 *     s_nm = rq_n . rk_m / sqrt(D)
 *     o_n  = sigmoid(g_n) * sum_m softmax_m(s_nm) v_m
 * softmax_m(s_nm) = exp(s_nm - max_m s_nm) / sum_m exp(s_nm - max_m s_nm),
 * two passes over m in order. */

/* Outputs of selected query tokens of head (b, h).  out: [nrows, D]. */
int gla_oracle_softmax_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const uint16_t* g, int B, int N, int H, int D,
                            int rope, int T, int Hh, int W, double theta, long t0, long y0,
                            long x0, int b, int h, const long* rows, long nrows, double* out) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  if (b < 0 || b >= B || h < 0 || h >= H || N < 1) return ORACLE_ERR_ARG;
  for (long i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= N) return ORACLE_ERR_ARG;
  /* every key rotated once */
  double* rk = malloc(sizeof(double) * (size_t)N * D);
  if (!rk) return ORACLE_ERR_ALLOC;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    double* u = malloc(sizeof(double) * D);
    if (!u) {
#pragma omp critical
      err = ORACLE_ERR_ALLOC;
    } else {
#pragma omp for schedule(static)
      for (long m = 0; m < N; ++m) {
        load_row(k, N, H, D, b, h, m, u);
        rotate(D, gr, m, u, rk + m * (long)D);
      }
    }
    free(u);
  }
  const double scale = 1.0 / sqrt((double)D);
  if (!err) {
#pragma omp parallel
    {
      double* qr = malloc(sizeof(double) * D);
      double* rq = malloc(sizeof(double) * D);
      double* gv = malloc(sizeof(double) * D);
      double* vr = malloc(sizeof(double) * D);
      double* s = malloc(sizeof(double) * (size_t)N);
      double* acc = malloc(sizeof(double) * D);
      if (!qr || !rq || !gv || !vr || !s || !acc) {
#pragma omp critical
        err = ORACLE_ERR_ALLOC;
      } else {
#pragma omp for schedule(dynamic, 1)
        for (long i = 0; i < nrows; ++i) {
          long n = rows[i];
          load_row(q, N, H, D, b, h, n, qr);
          load_row(g, N, H, D, b, h, n, gv);
          rotate(D, gr, n, qr, rq);
          double mx = -INFINITY;
          for (long m = 0; m < N; ++m) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += rq[d] * rk[m * (long)D + d];
            s[m] = dot * scale;
            if (s[m] > mx) mx = s[m];
          }
          double den = 0.0;
          for (int e = 0; e < D; ++e) acc[e] = 0.0;
          for (long m = 0; m < N; ++m) {
            double p = exp(s[m] - mx);
            den += p;
            load_row(v, N, H, D, b, h, m, vr);
            for (int e = 0; e < D; ++e) acc[e] += p * vr[e];
          }
          for (int e = 0; e < D; ++e) out[i * D + e] = sigmoid(gv[e]) * acc[e] / den;
        }
      }
      free(qr); free(rq); free(gv); free(vr); free(s); free(acc);
    }
  }
  free(rk);
  return err;
}

/* ---------------------------------------------------------------------------
 * Backward pass of the bidirectional mixer: the exact derivative of the
 * forward form above, for training the linear layers from scratch ("SANA-
 * Video 2.0: Hybrid Linear Attention with Attention Residuals for Efficient
 * Video Generation" (mlsanity index), Abstract: the hybrid is trained, not
 * distilled from a softmax model).  Given the gradient dout of a loss with
 * respect to the output, per (b, h), written out by the chain rule through
 * the forward definition with
 *     fq = phi(q_n), rq = R_n fq, den = fq.z + eps, s = sigmoid(g_n),
 *     num = S^T rq,  o_n = s * num / den:
 *     dg_n  = dout_n * o_n * (1 - s)             (sigmoid' = s (1 - s))
 *     a_n   = dout_n * s / den                   (gradient reaching num)
 *     dden  = -(a_n . num) / den                 (gradient reaching den)
 *     dq_n  = [q_n > 0] * (R_n^T (S a_n) + dden z)
 *     dS    = sum_n rq a_n^T,   dz = sum_n dden fq
 *     dv_m  = dS^T (R_m phi(k_m))
 *     dk_m  = [k_m > 0] * (R_m^T (dS v_m) + dz)
 * R_n^T is the rotation by the negated angles (R_n is orthogonal).  The
 * derivative of phi at 0 is taken as 0 (the one-sided choice of common
 * autograd systems; the pages do not discuss it).
 * ------------------------------------------------------------------------ */

/* out = R_n^T u: each pair rotated by the negated angle. */
static void rotate_back(int D, const oracle_grid* gr, long n, const double* u, double* out) {
  if (gr == NULL) {
    for (int d = 0; d < D; ++d) out[d] = u[d];
    return;
  }
  long t, y, x;
  token_position(gr, n, &t, &y, &x);
  for (int p = 0; p < D / 2; ++p) {
    double w = gla_oracle_angle(D, gr->theta, p, t, y, x);
    double c = cos(w), s = sin(w);
    double a = u[2 * p], b = u[2 * p + 1];
    out[2 * p] = a * c + b * s;
    out[2 * p + 1] = -a * s + b * c;
  }
}

typedef struct {
  double *x, *f, *r, *gv, *dv, *num, *a, *t, *t2;
} bwd_scratch;

static int scratch_alloc(bwd_scratch* w, int D) {
  double** p[] = {&w->x, &w->f, &w->r, &w->gv, &w->dv, &w->num, &w->a, &w->t, &w->t2};
  int ok = 1;
  for (unsigned i = 0; i < sizeof p / sizeof p[0]; ++i) {
    *p[i] = malloc(sizeof(double) * D);
    if (!*p[i]) ok = 0;
  }
  return ok ? ORACLE_OK : ORACLE_ERR_ALLOC;
}

static void scratch_free(bwd_scratch* w) {
  free(w->x); free(w->f); free(w->r); free(w->gv); free(w->dv);
  free(w->num); free(w->a); free(w->t); free(w->t2);
}

/* Query side of token n of head (b, h), given S and z: writes dq_row and
 * dg_row (either may be NULL) and, when dS / dz are not NULL, adds the
 * token's terms rq a^T and dden fq to them. */
static void bwd_query_token(const uint16_t* q, const uint16_t* g, const uint16_t* dout, int N,
                            int H, int D, const oracle_grid* gr, int b, int h, const double* S,
                            const double* z, double eps, long n, bwd_scratch* w, double* dq_row,
                            double* dg_row, double* dS, double* dz) {
  load_row(q, N, H, D, b, h, n, w->x);
  load_row(g, N, H, D, b, h, n, w->gv);
  load_row(dout, N, H, D, b, h, n, w->dv);
  for (int d = 0; d < D; ++d) w->f[d] = relu(w->x[d]);
  rotate(D, gr, n, w->f, w->r);
  double den = 0.0;
  for (int d = 0; d < D; ++d) den += w->f[d] * z[d];
  den += eps;
  for (int e = 0; e < D; ++e) {
    double num = 0.0;
    for (int d = 0; d < D; ++d) num += w->r[d] * S[(long)d * D + e];
    w->num[e] = num;
  }
  double dden = 0.0;
  for (int e = 0; e < D; ++e) {
    double s = sigmoid(w->gv[e]);
    double o = s * w->num[e] / den;
    if (dg_row) dg_row[e] = w->dv[e] * o * (1.0 - s);
    w->a[e] = w->dv[e] * s / den;
    dden -= w->a[e] * w->num[e];
  }
  dden /= den;
  if (dq_row) {
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int e = 0; e < D; ++e) acc += S[(long)d * D + e] * w->a[e];
      w->t[d] = acc;
    }
    rotate_back(D, gr, n, w->t, w->t2);
    for (int d = 0; d < D; ++d)
      dq_row[d] = w->x[d] > 0.0 ? w->t2[d] + dden * z[d] : 0.0;
  }
  if (dS)
    for (int d = 0; d < D; ++d)
      for (int e = 0; e < D; ++e) dS[(long)d * D + e] += w->r[d] * w->a[e];
  if (dz)
    for (int d = 0; d < D; ++d) dz[d] += dden * w->f[d];
}

/* Key/value side of token m of head (b, h), given dS and dz. */
static void bwd_key_token(const uint16_t* k, const uint16_t* v, int N, int H, int D,
                          const oracle_grid* gr, int b, int h, const double* dS, const double* dz,
                          long m, bwd_scratch* w, double* dk_row, double* dv_row) {
  load_row(k, N, H, D, b, h, m, w->x);
  load_row(v, N, H, D, b, h, m, w->gv);
  for (int d = 0; d < D; ++d) w->f[d] = relu(w->x[d]);
  rotate(D, gr, m, w->f, w->r);
  if (dv_row)
    for (int e = 0; e < D; ++e) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += dS[(long)d * D + e] * w->r[d];
      dv_row[e] = acc;
    }
  if (dk_row) {
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int e = 0; e < D; ++e) acc += dS[(long)d * D + e] * w->gv[e];
      w->t[d] = acc;
    }
    rotate_back(D, gr, m, w->t, w->t2);
    for (int d = 0; d < D; ++d) dk_row[d] = w->x[d] > 0.0 ? w->t2[d] + dz[d] : 0.0;
  }
}

/* Gradient state of every head: dS[B, H, D, D] = sum_n rq_n a_n^T and
 * dz[B, H, D] = sum_n dden_n phi(q_n), given the forward state S [B, H, D, D]
 * and z [B, H, D] (as gla_oracle_state writes them).  Sums in token order. */
int gla_oracle_backward_state(const uint16_t* q, const uint16_t* g, const uint16_t* dout,
                              int B, int N, int H, int D, int rope, int T, int Hh, int W,
                              double theta, long t0, long y0, long x0, double eps,
                              const double* S, const double* z, double* dS, double* dz) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  int err = ORACLE_OK;
  long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    int b = (int)(bh / H), h = (int)(bh % H);
    bwd_scratch w;
    int r = scratch_alloc(&w, D);
    double* dSh = dS + bh * D * (long)D;
    double* dzh = dz + bh * D;
    memset(dSh, 0, sizeof(double) * D * D);
    memset(dzh, 0, sizeof(double) * D);
    if (!r)
      for (long n = 0; n < N; ++n)
        bwd_query_token(q, g, dout, N, H, D, gr, b, h, S + bh * D * (long)D, z + bh * D, eps,
                        n, &w, NULL, NULL, dSh, dzh);
    scratch_free(&w);
    if (r) {
#pragma omp critical
      err = r;
    }
  }
  return err;
}

/* dq and dg of selected tokens of head (b, h), given that head's S and z.
 * dq_rows, dg_rows: [nrows, D]. */
int gla_oracle_backward_q_rows(const uint16_t* q, const uint16_t* g, const uint16_t* dout,
                               int B, int N, int H, int D, int rope, int T, int Hh, int W,
                               double theta, long t0, long y0, long x0, double eps, int b, int h,
                               const double* S, const double* z, const long* rows, long nrows,
                               double* dq_rows, double* dg_rows) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  if (b < 0 || b >= B || h < 0 || h >= H) return ORACLE_ERR_ARG;
  for (long i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= N) return ORACLE_ERR_ARG;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    bwd_scratch w;
    if (scratch_alloc(&w, D)) {
#pragma omp critical
      err = ORACLE_ERR_ALLOC;
    } else {
#pragma omp for schedule(static)
      for (long i = 0; i < nrows; ++i)
        bwd_query_token(q, g, dout, N, H, D, gr, b, h, S, z, eps, rows[i], &w, dq_rows + i * D,
                        dg_rows + i * D, NULL, NULL);
    }
    scratch_free(&w);
  }
  return err;
}

/* dk and dv of selected tokens of head (b, h), given that head's dS and dz.
 * dk_rows, dv_rows: [nrows, D]. */
int gla_oracle_backward_kv_rows(const uint16_t* k, const uint16_t* v, int B, int N, int H, int D,
                                int rope, int T, int Hh, int W, double theta, long t0, long y0,
                                long x0, int b, int h, const double* dS, const double* dz,
                                const long* rows, long nrows, double* dk_rows, double* dv_rows) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  if (b < 0 || b >= B || h < 0 || h >= H) return ORACLE_ERR_ARG;
  for (long i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= N) return ORACLE_ERR_ARG;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    bwd_scratch w;
    if (scratch_alloc(&w, D)) {
#pragma omp critical
      err = ORACLE_ERR_ALLOC;
    } else {
#pragma omp for schedule(static)
      for (long i = 0; i < nrows; ++i)
        bwd_key_token(k, v, N, H, D, gr, b, h, dS, dz, rows[i], &w, dk_rows + i * D,
                      dv_rows + i * D);
    }
    scratch_free(&w);
  }
  return err;
}

/* Whole backward pass: dq, dk, dv, dg [B, N, H, D] (doubles) from bf16 q, k,
 * v, g and the output gradient dout.  Per head: the forward state, then the
 * query side of every token (dq, dg, and the sums dS, dz), then the key side
 * of every token (dk, dv). */
int gla_oracle_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                        const uint16_t* dout, int B, int N, int H, int D, int rope, int T, int Hh,
                        int W, double theta, long t0, long y0, long x0, double eps, double* dq,
                        double* dk, double* dv, double* dg) {
  oracle_grid g0;
  const oracle_grid* gr;
  make_grid(rope, T, Hh, W, theta, t0, y0, x0, &g0, &gr);
  int rc = check_args(B, N, H, D, gr);
  if (rc) return rc;
  int err = ORACLE_OK;
  long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    int b = (int)(bh / H), h = (int)(bh % H);
    double* S = malloc(sizeof(double) * D * (long)D);
    double* z = malloc(sizeof(double) * D);
    double* dS = calloc((size_t)D * D, sizeof(double));
    double* dz = calloc((size_t)D, sizeof(double));
    bwd_scratch w;
    int r = scratch_alloc(&w, D);
    if (!S || !z || !dS || !dz) r = ORACLE_ERR_ALLOC;
    if (!r) r = head_state(k, v, N, H, D, gr, b, h, S, z);
    if (!r) {
      for (long n = 0; n < N; ++n) {
        long o = (((long)b * N + n) * H + h) * (long)D;
        bwd_query_token(q, g, dout, N, H, D, gr, b, h, S, z, eps, n, &w, dq + o, dg + o, dS, dz);
      }
      for (long m = 0; m < N; ++m) {
        long o = (((long)b * N + m) * H + h) * (long)D;
        bwd_key_token(k, v, N, H, D, gr, b, h, dS, dz, m, &w, dk + o, dv + o);
      }
    }
    scratch_free(&w);
    free(S); free(z); free(dS); free(dz);
    if (r) {
#pragma omp critical
      err = r;
    }
  }
  return err;
}

/* ---------------------------------------------------------------------------
 * Projection prologue: the linear maps that produce q, k, v and g from the
 * hidden states ("SANA-Video 2.0", NVlabs Sana docs, section Architecture:
 * hidden size 2,560 with 20 heads x 128 at 5B, 4,096 with 32 heads x 128 at
 * 14B).  The pages give no further detail; the reading taken is four
 * bias-free linear maps, y = x W^T with W of shape [H*D, C] per map (the
 * weights stacked as [4][H*D][C] in the order q, k, v, g), each result
 * rounded to bf16 as a BF16 model stores it (section Model zoo: BF16
 * inference), and then the mixer above on the four bf16 tensors.
 * ------------------------------------------------------------------------ */

/* Round a double to the nearest bf16 value (ties to even) and return its
 * bit pattern.  bf16 keeps 8 significant bits: with x = f 2^E, 0.5 <= |f| < 1,
 * the spacing is 2^(E-8).  Finite inputs of normal bf16 magnitude only
 * (|x| in [2^-126, 2^127]) or zero. */
uint16_t gla_oracle_round_bf16(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000 : 0;
  int E;
  frexp(x, &E);
  double ulp = ldexp(1.0, E - 8);
  double r = nearbyint(x / ulp) * ulp;   /* default rounding: nearest, ties to even */
  float f = (float)r;                    /* exact: r has 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* out[b][n][i] = sum_c x[b][n][c] * w[feat[i]][c] in fp64, for the nfeat
 * output features listed in feat (rows of the stacked [4*H*D][C] weights).
 * x: bf16 [B, N, C]; w: bf16 [P, C]; out: [B, N, nfeat] doubles. */
int gla_oracle_project(const uint16_t* x, const uint16_t* w, int B, int N, int C, int P,
                       const int* feat, int nfeat, double* out) {
  if (B < 0 || N < 0 || C <= 0 || P <= 0 || nfeat < 0) return ORACLE_ERR_ARG;
  for (int i = 0; i < nfeat; ++i)
    if (feat[i] < 0 || feat[i] >= P) return ORACLE_ERR_ARG;
  long rows = (long)B * N;
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    const uint16_t* xr = x + r * (long)C;
    for (int i = 0; i < nfeat; ++i) {
      const uint16_t* wr = w + (long)feat[i] * C;
      double acc = 0.0;
      for (int c = 0; c < C; ++c)
        acc += gla_oracle_bf16_to_f64(xr[c]) * gla_oracle_bf16_to_f64(wr[c]);
      out[r * nfeat + i] = acc;
    }
  }
  return ORACLE_OK;
}

/* gla_oracle_round_bf16 over an array. */
void gla_oracle_round_bf16_array(const double* in, long n, uint16_t* out) {
  for (long i = 0; i < n; ++i) out[i] = gla_oracle_round_bf16(in[i]);
}
