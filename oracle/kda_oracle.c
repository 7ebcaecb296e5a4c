/*
 * kda_oracle.c -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA) mixer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
 * shares no code, header or constant with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [p1] docs.rs "ferrox_models::kda" module page -- per-channel decay gate, sigmoid
 *        output gate, short causal Conv1d with padding kernel_size-1 and no bias, q/k
 *        L2-normalised (eps 1e-6) then q scaled by head_dim^-1/2.
 *   [p2] "Kimi Delta Attention (KDA) -- analysis & C kernel plan" (sqliteai/waste
 *        docs/KDA.md) -- sections "The KDA layer, precisely" and "Recurrence".
 *   [p3] docs.rs "memra_engine::kda" module page -- header prose (conv fusion: fused
 *        [3*qkv, kernel] weights and ring; chunk form with per-channel Gcum).
 *   [p4] OpenModelAtlas "Kimi K3 - Retention gate" -- formulas and the gate.py
 *        excerpt (naive_kda_lowerbound_gate), and the 16-token tile bound ("Why").
 *
 * Everything is computed in double precision, token by token, with no blocking,
 * fusion or reordering beyond what the definitions state.  io inputs arrive either as
 * fp32 or as bf16 bit patterns (uint16); both convert to double exactly.
 *
 * Readings taken where the pages are silent:
 *   - conv taps: cross-correlation with left zero padding of kernel-1, tap index
 *     kernel-1 multiplies the current token (PyTorch Conv1d semantics, [p1]);
 *   - the conv history ("ring") holds the kernel-1 most recent raw inputs, oldest first;
 *   - L2 norm: x * (sum x^2 + eps)^-1/2;
 *   - gated RMSNorm: normalise, multiply by the weight, then by sigmoid(gate);
 *   - low-rank decay gate (optional): the gate's pre-activation is z = z_low f_b^T with
 *     rank head_dim, f_b laid out [H*d][d] (output channel first, as a linear layer's
 *     weight) in the io dtype ([p2] "The KDA layer, precisely", structural fact 2: hidden
 *     -> head_dim -> H*head_dim; [p4] the model code's f_b_proj(f_a_proj(.)) and the
 *     7,168 -> 128 -> 12,288 pair).
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ io decoding */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* io_dtype: 0 = fp32, 1 = bf16 stored as uint16 bit patterns */
static double load_io(const void* base, int io_dtype, int64_t idx) {
  if (io_dtype == 0) return (double)((const float*)base)[idx];
  return bf16_bits_to_double(((const uint16_t*)base)[idx]);
}

/* ------------------------------------------------------------------ elementwise steps */

/* logistic sigmoid, 1 / (1 + e^-x) */
double kdao_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* SiLU activation applied after the short conv: y * sigmoid(y)  ([p2] layer equations) */
double kdao_silu(double y) { return y * kdao_sigmoid(y); }

/*
 * Lower-bounded per-channel log decay ([p4] gate.py, naive_kda_lowerbound_gate; [p1]
 * fact 1): g = lower_bound * sigmoid(exp(A_log[h]) * (z + dt_bias[c])).
 */
double kdao_gate(double z, double dt_bias, double A_log, double lower_bound) {
  return lower_bound * kdao_sigmoid(exp(A_log) * (z + dt_bias));
}

/* softplus(x) = log(1 + e^x), written to avoid overflow for large x */
double kdao_softplus(double x) { return x > 30.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/*
 * Kimi-Linear's unbounded per-channel log decay ([p2] status note: -e^{A_log} softplus(z),
 * the gate used when a model sets no lower bound; z carries dt_bias as in the bounded
 * gate): g = -exp(A_log[h]) * softplus(z + dt_bias[c]).
 */
double kdao_gate_softplus(double z, double dt_bias, double A_log) {
  return -exp(A_log) * kdao_softplus(z + dt_bias);
}

/* x <- x * (sum_i x_i^2 + eps)^-1/2 * scale, over one head row of length d ([p1]). */
void kdao_l2norm(double* x, int d, double eps, double scale) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  double r = scale / sqrt(ss + eps);
  for (int i = 0; i < d; ++i) x[i] *= r;
}

/*
 * Sigmoid-gated RMSNorm over one head row ([p1] fact 2; [p2] "o = RMSNormGated(o, gate)";
 * [p4] FusedRMSNormGated(head_dim, eps=rms_norm_eps, activation='sigmoid')):
 *   y_j = w_j * o_j / sqrt(mean_i o_i^2 + eps) * sigmoid(gate_j).
 */
void kdao_gated_rmsnorm(const double* o, const double* gate, const float* w, int d, double eps,
                        double* y) {
  double ss = 0.0;
  for (int j = 0; j < d; ++j) ss += o[j] * o[j];
  double r = 1.0 / sqrt(ss / (double)d + eps);
  for (int j = 0; j < d; ++j) y[j] = (double)w[j] * o[j] * r * kdao_sigmoid(gate[j]);
}

/* ------------------------------------------------------------------ the recurrence */

/*
 * One step of the gated delta rule ([p2] "Recurrence"; [p1] naive_recurrent_kda):
 *   S'  = Diag(exp(g)) S            (decay along the key axis, S is [dk][dv])
 *   u   = S'^T k
 *   S   = S' + beta * k (v - u)^T   (delta against the decayed state)
 *   o   = S^T q                     (readout from the updated state)
 * q is already normalised and scaled.  S is updated in place; o has length dv.
 */
void kdao_step(double* S, int dk, int dv, const double* q, const double* k, const double* v,
               const double* g, double beta, double* o, double* work /* dv */) {
  for (int i = 0; i < dk; ++i) {
    double a = exp(g[i]);
    for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= a;
  }
  for (int j = 0; j < dv; ++j) {
    double u = 0.0;
    for (int i = 0; i < dk; ++i) u += S[(int64_t)i * dv + j] * k[i];
    work[j] = beta * (v[j] - u);
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += k[i] * work[j];
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * q[i];
    o[j] = acc;
  }
}

/*
 * The bare recurrence over T tokens of one (sequence, head) on already-prepared inputs:
 * qh, kh [T][dk], v [T][dv], g [T][dk], beta [T].  S (dk*dv) holds the initial state on
 * entry and the final state on exit.  o [T][dv].  If S_trace is non-null it receives
 * the state after every token, [T][dk][dv].
 */
void kdao_core(int T, int dk, int dv, const double* qh, const double* kh, const double* v,
               const double* g, const double* beta, double* S, double* o, double* S_trace) {
  double* work = (double*)malloc(sizeof(double) * (size_t)dv);
  for (int t = 0; t < T; ++t) {
    kdao_step(S, dk, dv, qh + (int64_t)t * dk, kh + (int64_t)t * dk, v + (int64_t)t * dv,
              g + (int64_t)t * dk, beta[t], o + (int64_t)t * dv, work);
    if (S_trace) memcpy(S_trace + (int64_t)t * dk * dv, S, sizeof(double) * (size_t)dk * dv);
  }
  free(work);
}

/* ------------------------------------------------------------------ the chunked twin */

/*
 * The same recurrence reached through the chunk form ([p3] header prose: per-channel
 * cumulative log gate Gcum, keys scaled by exp(-Gcum), queries by exp(+Gcum); [p4]
 * "Why": within a 16-token tile every rescale stays below e^80).  Written from the
 * algebra, in fp64, with no reference to any kernel:
 *
 *   Within a chunk of C tokens, r = 1..C, with Gcum_r = sum_{s<=r} g_s (per key channel):
 *     A[r][j] = beta_r * sum_i k_ri k_ji exp(Gcum_ri - Gcum_ji)   (j < r)
 *     P[r][j] =          sum_i q_ri k_ji exp(Gcum_ri - Gcum_ji)   (j <= r)
 *     (I + A) U = Diag(beta) (V - Ka S0),  Ka_r = k_r * exp(Gcum_r)
 *     O = Qa S0 + P U,                      Qa_r = q_r * exp(Gcum_r)
 *     S_C = Diag(exp(Gcum_C)) S0 + Kl^T U,  Kl_r = k_r * exp(Gcum_C - Gcum_r)
 *
 * Each exp(Gcum_ri - Gcum_ji) is formed from a reference point inside its tile pair:
 * for r and j in the same tau-token tile, the tile start; for j in an earlier tile, the
 * end of j's tile.  Each factor then lies in [e^(-5 tau), e^(5 tau)] (same tile) or in
 * (0, 1] (earlier tile) when g > -5.  The products are exact rewrites of the formula
 * above, so in fp64 this equals the token recurrence up to rounding.
 */
void kdao_core_chunked(int T, int dk, int dv, int C, int tau, const double* qh, const double* kh,
                       const double* v, const double* g, const double* beta, double* S, double* o) {
  double* G = (double*)malloc(sizeof(double) * (size_t)C * dk);  /* Gcum within chunk */
  double* A = (double*)malloc(sizeof(double) * (size_t)C * C);
  double* P = (double*)malloc(sizeof(double) * (size_t)C * C);
  double* U = (double*)malloc(sizeof(double) * (size_t)C * dv);
  double* Snew = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  for (int c0 = 0; c0 < T; c0 += C) {
    int L = (T - c0 < C) ? (T - c0) : C;
    /* cumulative log gate per channel, Gcum_r = g_1 + ... + g_r (r counted from 1) */
    for (int i = 0; i < dk; ++i) {
      double acc = 0.0;
      for (int r = 0; r < L; ++r) {
        acc += g[(int64_t)(c0 + r) * dk + i];
        G[(int64_t)r * dk + i] = acc;
      }
    }
    /* Gram matrices with a per-pair reference point */
    for (int r = 0; r < L; ++r) {
      for (int j = 0; j <= r; ++j) {
        int tr = r / tau, tj = j / tau;
        double sa = 0.0, sp = 0.0;
        for (int i = 0; i < dk; ++i) {
          double ref;
          if (tr == tj) {
            int s = tj * tau; /* tile start: Gcum of the token before the tile (0 at chunk start) */
            ref = (s == 0) ? 0.0 : G[(int64_t)(s - 1) * dk + i];
          } else {
            int e = tj * tau + tau - 1; /* last token of j's tile */
            ref = G[(int64_t)e * dk + i];
          }
          double left = exp(G[(int64_t)r * dk + i] - ref);
          double right = exp(ref - G[(int64_t)j * dk + i]);
          double kj = kh[(int64_t)(c0 + j) * dk + i] * right;
          sa += kh[(int64_t)(c0 + r) * dk + i] * left * kj;
          sp += qh[(int64_t)(c0 + r) * dk + i] * left * kj;
        }
        A[r * C + j] = (j < r) ? beta[c0 + r] * sa : 0.0;
        P[r * C + j] = sp;
      }
    }
    /* right-hand side Diag(beta)(V - Ka S0), then forward substitution through (I + A) */
    for (int r = 0; r < L; ++r) {
      for (int jv = 0; jv < dv; ++jv) {
        double ks = 0.0;
        for (int i = 0; i < dk; ++i)
          ks += kh[(int64_t)(c0 + r) * dk + i] * exp(G[(int64_t)r * dk + i]) * S[(int64_t)i * dv + jv];
        double rhs = beta[c0 + r] * (v[(int64_t)(c0 + r) * dv + jv] - ks);
        for (int j = 0; j < r; ++j) rhs -= A[r * C + j] * U[(int64_t)j * dv + jv];
        U[(int64_t)r * dv + jv] = rhs;
      }
    }
    /* outputs O = Qa S0 + P U */
    for (int r = 0; r < L; ++r) {
      for (int jv = 0; jv < dv; ++jv) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i)
          acc += qh[(int64_t)(c0 + r) * dk + i] * exp(G[(int64_t)r * dk + i]) * S[(int64_t)i * dv + jv];
        for (int j = 0; j <= r; ++j) acc += P[r * C + j] * U[(int64_t)j * dv + jv];
        o[(int64_t)(c0 + r) * dv + jv] = acc;
      }
    }
    /* state carry S_C = Diag(exp(Gcum_L)) S0 + Kl^T U */
    for (int i = 0; i < dk; ++i) {
      double GL = G[(int64_t)(L - 1) * dk + i];
      for (int jv = 0; jv < dv; ++jv) {
        double acc = exp(GL) * S[(int64_t)i * dv + jv];
        for (int r = 0; r < L; ++r)
          acc += kh[(int64_t)(c0 + r) * dk + i] * exp(GL - G[(int64_t)r * dk + i]) * U[(int64_t)r * dv + jv];
        Snew[(int64_t)i * dv + jv] = acc;
      }
    }
    memcpy(S, Snew, sizeof(double) * (size_t)dk * dv);
  }
  free(G); free(A); free(P); free(U); free(Snew);
}

/* ------------------------------------------------------------------ gate projection */

/*
 * The low-rank decay-gate projection: z[t][c] = sum_r z_low[t][r] f_b[c][r] for rows
 * t < rows and channels c < channels, in double precision ([p2] "The KDA layer,
 * precisely", fact 2; [p4] f_b_proj applied to the rank-128 f_a_proj output).  z_low is
 * [rows][rank] and f_b [channels][rank], both io dtype; z is [rows][channels].
 */
void kdao_gate_projection(const void* z_low, const void* f_b, int io_dtype, int64_t rows,
                          int32_t rank, int64_t channels, double* z) {
  for (int64_t t = 0; t < rows; ++t)
    for (int64_t c = 0; c < channels; ++c) {
      double acc = 0.0;
      for (int32_t r = 0; r < rank; ++r)
        acc += load_io(z_low, io_dtype, t * rank + r) * load_io(f_b, io_dtype, c * rank + r);
      z[t * channels + c] = acc;
    }
}

/* ------------------------------------------------------------------ full mixer core */

typedef struct {
  int32_t num_heads, head_dim, conv_kernel;
  int32_t gate_kind; /* 0: lower-bounded sigmoid gate, 1: softplus gate */
  double lower_bound, l2_eps, rms_eps;
  const float* conv_w;  /* [3*H*d][conv_kernel], planes q,k,v ([p3] conv fusion) */
  const float* dt_bias; /* [H*d] */
  const float* A_log;   /* [H] */
  const float* norm_w;  /* [d] */
} kdao_layer;

typedef struct {
  const kdao_layer* L;
  int io_dtype;
  const int64_t* cu_seqlens; /* [N+1] */
  const void *q, *k, *v, *z, *beta, *gate; /* token-major [T_tot][H*d]; beta [T_tot][H] */
  const void* f_b;           /* NULL, or [H*d][d]: then z is z_low [T_tot][d] */
  const double* state_in;    /* [N][H][d][d] or NULL (zero) */
  const float* ring_in;      /* [N][3*H*d][kconv-1] or NULL (zero) */
  /* per-unit outputs, in unit order: out [sum T][d], state [d][d], ring [3][d][kconv-1] */
  const int32_t* units;      /* [n_units][2] = (sequence, head) */
  const int64_t* out_offset; /* [n_units] row offset of each unit inside out */
  double* out;
  double* state_out;         /* [n_units][d][d] or NULL */
  double* ring_out;          /* [n_units][3][d][kconv-1] or NULL */
  /* optional per-token traces for a single unit (used by the tiny pins): */
  double *tr_q, *tr_k, *tr_v, *tr_g, *tr_beta, *tr_o_raw, *tr_S;
  int n_units;
  int next;                  /* work counter */
  pthread_mutex_t mu;
} kdao_job;

/*
 * One (sequence, head) unit: short conv + SiLU on q/k/v with the history taken from the
 * ring ([p1]; [p2] structural fact 1; [p3] conv fusion), L2 norm and q scale ([p1]),
 * the gate and beta ([p4] gate.py; [p2] layer equations), the recurrence ([p2]
 * "Recurrence") and the gated RMSNorm ([p1] fact 2).  Emits the final state and the
 * last kconv-1 raw inputs of each plane as the new ring.
 */
static void run_unit(kdao_job* J, int u) {
  const kdao_layer* L = J->L;
  const int H = L->num_heads, d = L->head_dim, K = L->conv_kernel, R = K - 1;
  const int64_t Hd = (int64_t)H * d;
  const int n = J->units[2 * u], h = J->units[2 * u + 1];
  const int64_t t0 = J->cu_seqlens[n], T = J->cu_seqlens[n + 1] - t0;
  const double scale = 1.0 / sqrt((double)d);

  double* S = (double*)calloc((size_t)d * d, sizeof(double));
  if (J->state_in)
    for (int64_t e = 0; e < (int64_t)d * d; ++e)
      S[e] = J->state_in[((int64_t)n * H + h) * d * d + e];

  /* hist[p][i][0..R-1]: the R most recent raw inputs of channel i of plane p, oldest first */
  double* hist = (double*)calloc((size_t)3 * d * R, sizeof(double));
  if (J->ring_in)
    for (int p = 0; p < 3; ++p)
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < R; ++j)
          hist[((int64_t)p * d + i) * R + j] =
              (double)J->ring_in[((int64_t)n * 3 * Hd + p * Hd + (int64_t)h * d + i) * R + j];

  double *a[3], *gv = (double*)malloc(sizeof(double) * d), *o = (double*)malloc(sizeof(double) * d);
  double *gt = (double*)malloc(sizeof(double) * d), *y = (double*)malloc(sizeof(double) * d);
  double* work = (double*)malloc(sizeof(double) * d);
  for (int p = 0; p < 3; ++p) a[p] = (double*)malloc(sizeof(double) * d);
  const void* planes[3] = {J->q, J->k, J->v};

  for (int64_t t = 0; t < T; ++t) {
    const int64_t row = t0 + t;
    /* short causal conv, then SiLU, per plane and channel */
    for (int p = 0; p < 3; ++p) {
      for (int i = 0; i < d; ++i) {
        const int64_t c = (int64_t)h * d + i;
        const float* w = L->conv_w + ((int64_t)p * Hd + c) * K;
        double* hi = hist + ((int64_t)p * d + i) * R;
        double x = load_io(planes[p], J->io_dtype, row * Hd + c);
        double acc = w[K - 1] * x;
        for (int j = 0; j < R; ++j) acc += (double)w[j] * hi[j];
        a[p][i] = kdao_silu(acc);
        for (int j = 0; j + 1 < R; ++j) hi[j] = hi[j + 1];
        if (R > 0) hi[R - 1] = x;
      }
    }
    kdao_l2norm(a[0], d, L->l2_eps, scale); /* q-hat, scaled by d^-1/2 */
    kdao_l2norm(a[1], d, L->l2_eps, 1.0);   /* k-hat */
    for (int i = 0; i < d; ++i) {
      const int64_t c = (int64_t)h * d + i;
      double zz;
      if (J->f_b) { /* low-rank gate: one row of z_low f_b^T, the reading in the header */
        zz = 0.0;
        for (int r = 0; r < d; ++r)
          zz += load_io(J->z, J->io_dtype, row * d + r) * load_io(J->f_b, J->io_dtype, c * d + r);
      } else {
        zz = load_io(J->z, J->io_dtype, row * Hd + c);
      }
      gv[i] = L->gate_kind == 1
                  ? kdao_gate_softplus(zz, (double)L->dt_bias[c], (double)L->A_log[h])
                  : kdao_gate(zz, (double)L->dt_bias[c], (double)L->A_log[h], L->lower_bound);
      gt[i] = load_io(J->gate, J->io_dtype, row * Hd + c);
    }
    double beta = kdao_sigmoid(load_io(J->beta, J->io_dtype, row * H + h));
    kdao_step(S, d, d, a[0], a[1], a[2], gv, beta, o, work);
    kdao_gated_rmsnorm(o, gt, L->norm_w, d, L->rms_eps, y);
    memcpy(J->out + (J->out_offset[u] + t) * d, y, sizeof(double) * d);
    if (J->tr_q) {
      memcpy(J->tr_q + t * d, a[0], sizeof(double) * d);
      memcpy(J->tr_k + t * d, a[1], sizeof(double) * d);
      memcpy(J->tr_v + t * d, a[2], sizeof(double) * d);
      memcpy(J->tr_g + t * d, gv, sizeof(double) * d);
      J->tr_beta[t] = beta;
      memcpy(J->tr_o_raw + t * d, o, sizeof(double) * d);
      memcpy(J->tr_S + t * d * d, S, sizeof(double) * d * d);
    }
  }
  if (J->state_out) memcpy(J->state_out + (int64_t)u * d * d, S, sizeof(double) * d * d);
  if (J->ring_out) memcpy(J->ring_out + (int64_t)u * 3 * d * R, hist, sizeof(double) * 3 * d * R);
  for (int p = 0; p < 3; ++p) free(a[p]);
  free(S); free(hist); free(gv); free(o); free(gt); free(y); free(work);
}

static void* worker(void* arg) {
  kdao_job* J = (kdao_job*)arg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int u = J->next;
    J->next = u + 1;
    pthread_mutex_unlock(&J->mu);
    if (u >= J->n_units) break;
    run_unit(J, u);
  }
  return NULL;
}

/*
 * Prefill over packed sequences for the listed (sequence, head) units, threaded over
 * units.  The caller lists units longest-first if it wants balanced threads.  Returns 0
 * on success, -1 on a bad argument.  `units` holds n_units (sequence, head) pairs.
 * If trace pointers are non-null, exactly one unit must be listed.  With f_b non-NULL
 * ([H*d][head_dim], io dtype) z is the rank-head_dim input z_low [T_tot][head_dim] and
 * the gate's pre-activation is its projection (kdao_gate_projection).
 */
int kdao_prefill_units(int32_t num_heads, int32_t head_dim, int32_t conv_kernel,
                       int32_t gate_kind, double lower_bound, double l2_eps, double rms_eps,
                       const float* conv_w,
                       const float* dt_bias, const float* A_log, const float* norm_w,
                       int io_dtype, const int64_t* cu_seqlens, const void* q, const void* k,
                       const void* v, const void* z, const void* beta, const void* gate,
                       const void* f_b, const double* state_in, const float* ring_in,
                       int32_t n_units, const int32_t* units, const int64_t* out_offset, double* out,
                       double* state_out, double* ring_out, int nthreads, double* tr_q,
                       double* tr_k, double* tr_v, double* tr_g, double* tr_beta,
                       double* tr_o_raw, double* tr_S) {
  if (head_dim <= 0 || num_heads <= 0 || conv_kernel < 1) return -1;
  if (gate_kind != 0 && gate_kind != 1) return -1;
  if (n_units < 0 || (tr_q && n_units != 1)) return -1;
  kdao_layer L = {num_heads, head_dim, conv_kernel, gate_kind, lower_bound, l2_eps, rms_eps,
                  conv_w, dt_bias, A_log, norm_w};
  kdao_job J;
  memset(&J, 0, sizeof J);
  J.L = &L; J.io_dtype = io_dtype; J.cu_seqlens = cu_seqlens;
  J.q = q; J.k = k; J.v = v; J.z = z; J.beta = beta; J.gate = gate; J.f_b = f_b;
  J.state_in = state_in; J.ring_in = ring_in;
  J.units = units; J.n_units = n_units; J.out_offset = out_offset; J.out = out;
  J.state_out = state_out; J.ring_out = ring_out;
  J.tr_q = tr_q; J.tr_k = tr_k; J.tr_v = tr_v; J.tr_g = tr_g; J.tr_beta = tr_beta;
  J.tr_o_raw = tr_o_raw; J.tr_S = tr_S;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_units) nthreads = n_units > 0 ? n_units : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return 0;
}
