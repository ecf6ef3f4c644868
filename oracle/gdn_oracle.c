/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle of the Gated DeltaNet mixer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py use it.  It shares no code, header, table or helper with the HIP
 * library; the two meet only through the seeded input generator.
 *
 * What it computes, and where each step is defined:
 *
 *  - Causal depthwise conv1d + SiLU over the packed [Q|K|V] rows
 *    (kernel handles `conv1d_k`, `conv1d_prefill_k`, `conv1d_l2norm_k` and the
 *    `causal_conv1d_update_l2norm_f32_strided` doc comment on the
 *    metrale_model_layers/layers/qwen3_ssm/layer_struct.rs source page; the
 *    [Q | K | V | Z] row order is the struct's doc comment on that page).
 *    y[t][c] = SiLU(sum_j w[c][j] * x[t-K+1+j][c]); rows before the start of a
 *    sequence come from its conv state of K-1 raw rows, oldest first; no bias.
 *  - L2 normalisation of every q and k head over d_k:
 *    x_hat = x / sqrt(sum x^2 + eps)  (handle `l2_norm_k`, same page).
 *  - The gated delta rule, token by token (the decode-once-per-token default of
 *    `prefill` on the metrale_model_layers/layer/transformer_layer.rs page;
 *    the recurrence itself is the gated delta rule of Yang, Kautz and
 *    Hatamizadeh, "Gated Delta Networks", ICLR 2025, section 3):
 *        S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t.
 *    It is evaluated in the algebraically identical rank-1 order
 *        kv = S k;  u = b (v - a kv);  S <- a S + u k^T
 *    because a S (I - b k k^T) = a S - (a b)(S k) k^T.  The state is stored as
 *    h = S^T, i.e. h[head][i][j] with i over d_k and j over d_v, which is the
 *    `nv * kd * vd` per-sequence state order of the `h_state_bytes` field.
 *  - Z-gated RMSNorm per (token, value head) over d_v (handles
 *    `gated_rms_norm_k`, `gated_rms_norm_prefill_k`):
 *        out = o / sqrt(mean(o^2) + eps) * w * SiLU(z),
 *    or with the gate sigmoid(z) in place of SiLU(z) for a model of the
 *    `gdn_norm_sigmoid` kind (doc comment of `gated_rms_norm_f32_strided_k`).
 *  - Optional storage of the state in IEEE binary16 (the FP16 h-state variants
 *    and the `ssm_h_f16_to_f32_k` / `ssm_h_f32_to_f16_k` width converters on
 *    the layer_struct.rs page): the state is rounded to the nearest binary16
 *    value (ties to even) whenever it is stored -- after every token for the
 *    one-token and verify forms, once at the end for a prefill, which widens
 *    the stored state, runs at full width and narrows the result.
 *  - Optional record of the rank-1 update vector u_t of every token (what a
 *    write-on-accept verify keeps instead of whole states; `gdn_wy4_woa_k`,
 *    `gdn_wy4_fold_k` on the layer_struct.rs page).
 *
 * Value head h reads key head floor(h * Hk / Hv) (grouped heads).
 * All arithmetic is double precision, in the order the definitions state.
 * OpenMP parallelises over independent (sequence, value head) pairs only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double silu(double x) { return x / (1.0 + exp(-x)); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Nearest IEEE binary16 value of x, ties to even (the default rounding mode of
 * nearbyint): 11 significant bits, so the spacing of values in [2^(e-1), 2^e) is
 * 2^(e-11), never below the subnormal spacing 2^-24; beyond the largest finite
 * value 65504 the result overflows to infinity. */
double orc_round_binary16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  frexp(x, &e);
  int q = e - 11;
  if (q < -24) q = -24;
  const double r = ldexp(nearbyint(ldexp(x, -q)), q);
  return fabs(r) > 65504.0 ? copysign(INFINITY, x) : r;
}

void orc_round_binary16_array(double *x, long long n) {
  for (long long i = 0; i < n; ++i) x[i] = orc_round_binary16(x[i]);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Conv1d + SiLU + L2 over a packed batch of n sequences.
 *   cu    [n+1]             token offsets of each sequence in the packed rows
 *   x     [T][C]            pre-conv rows, C = 2*Hk*dk + Hv*dv
 *   w     [C][K]            per-channel taps, tap K-1 multiplies the current row
 *   ring  [n][K-1][C]       per-sequence conv state, oldest row first; replaced
 *                           by the last K-1 rows of [old ring ; x rows]
 *   y     [T][C]            [q_hat | k_hat | v]
 */
void orc_conv_l2norm(int n, const int32_t *cu, int Hk, int Hv, int dk, int dv, int K,
                     const double *x, const double *w, double *ring, double l2_eps,
                     double *y) {
  const int C = 2 * Hk * dk + Hv * dv;
  const int R = K - 1;
  for (int s = 0; s < n; ++s) {
    const int t0 = cu[s], len = cu[s + 1] - cu[s];
    double *rs = ring + (size_t)s * R * C;
    for (int tau = 0; tau < len; ++tau) {
      double *yt = y + (size_t)(t0 + tau) * C;
      for (int c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int j = 0; j < K; ++j) {
          int src = tau - (K - 1) + j; /* relative row index, negative = history */
          double xv = (src >= 0) ? x[(size_t)(t0 + src) * C + c] : rs[(size_t)(R + src) * C + c];
          acc += w[(size_t)c * K + j] * xv;
        }
        yt[c] = silu(acc);
      }
      /* L2 normalise every q head and every k head. */
      for (int part = 0; part < 2; ++part) {
        for (int g = 0; g < Hk; ++g) {
          double *p = yt + (size_t)part * Hk * dk + (size_t)g * dk;
          double ss = 0.0;
          for (int i = 0; i < dk; ++i) ss += p[i] * p[i];
          double inv = 1.0 / sqrt(ss + l2_eps);
          for (int i = 0; i < dk; ++i) p[i] *= inv;
        }
      }
    }
    /* New conv state: last R rows of the concatenation [old ring ; x rows]. */
    if (len > 0) {
      double *tmp = (double *)malloc(sizeof(double) * (size_t)R * C);
      for (int r = 0; r < R; ++r) {
        int idx = len + r; /* index into concatenation of length R + len */
        const double *src = (idx < R) ? rs + (size_t)idx * C : x + (size_t)(t0 + idx - R) * C;
        memcpy(tmp + (size_t)r * C, src, sizeof(double) * C);
      }
      memcpy(rs, tmp, sizeof(double) * (size_t)R * C);
      free(tmp);
    }
  }
}

/*
 * Gated delta rule over a packed batch, token by token.
 *   q, k  [T][Hk][dk]   (already L2 normalised by the caller, or not: the rule
 *                        is defined for any k)
 *   v     [T][Hv][dv]
 *   a, b  [T][Hv]       decay and write strength of each token and value head
 *   S     [n][Hv][dk][dv]  h = S^T per head, read as the initial state and
 *                        overwritten with the final state
 *   o     [T][Hv][dv]   scale * S_t q_t
 *   heads [nh]          value heads to compute (NULL: all heads, nh ignored)
 *   states_out          NULL, or [T][nh][dk][dv]: h after every token, for the
 *                        listed heads in list order
 *   state_round         0: full width throughout; 1: the state is rounded to
 *                        binary16 after every token (the output of the token
 *                        uses the state before that rounding); 2: only the final
 *                        state of each sequence is rounded
 *   u_out               NULL, or [T][nh][dv]: the update vector u of every token
 * Heads not listed are left untouched in S and o.
 */
void orc_delta_rule(int n, const int32_t *cu, int Hk, int Hv, int dk, int dv,
                    const double *q, const double *k, const double *v, const double *a,
                    const double *b, double scale, double *S, double *o,
                    const int32_t *heads, int nh, double *states_out, int state_round,
                    double *u_out) {
  if (heads == NULL) nh = Hv;
  const long long pairs = (long long)n * nh;
#pragma omp parallel for schedule(dynamic, 1)
  for (long long pr = 0; pr < pairs; ++pr) {
    const int s = (int)(pr / nh), hi = (int)(pr % nh);
    const int h = heads ? heads[hi] : hi;
    const int g = (int)((long long)h * Hk / Hv);
    double *hs = S + ((size_t)s * Hv + h) * (size_t)dk * dv;
    double *kv = (double *)malloc(sizeof(double) * dv);
    double *u = (double *)malloc(sizeof(double) * dv);
    for (int t = cu[s]; t < cu[s + 1]; ++t) {
      const double *qt = q + ((size_t)t * Hk + g) * dk;
      const double *kt = k + ((size_t)t * Hk + g) * dk;
      const double *vt = v + ((size_t)t * Hv + h) * dv;
      const double at = a[(size_t)t * Hv + h], bt = b[(size_t)t * Hv + h];
      /* kv = S k  (column j of h is row j of S) */
      for (int j = 0; j < dv; ++j) kv[j] = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) kv[j] += kt[i] * hs[(size_t)i * dv + j];
      for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - at * kv[j]);
      /* S <- a S + u k^T */
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) hs[(size_t)i * dv + j] = at * hs[(size_t)i * dv + j] + kt[i] * u[j];
      /* o = scale * S q */
      double *ot = o + ((size_t)t * Hv + h) * dv;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += qt[i] * hs[(size_t)i * dv + j];
        ot[j] = scale * acc;
      }
      if (state_round == 1 || (state_round == 2 && t == cu[s + 1] - 1))
        for (size_t e = 0; e < (size_t)dk * dv; ++e) hs[e] = orc_round_binary16(hs[e]);
      if (states_out)
        memcpy(states_out + ((size_t)t * nh + hi) * (size_t)dk * dv, hs, sizeof(double) * (size_t)dk * dv);
      if (u_out) memcpy(u_out + ((size_t)t * nh + hi) * (size_t)dv, u, sizeof(double) * (size_t)dv);
    }
    free(kv);
    free(u);
  }
}

/*
 * Z-gated RMSNorm per (token, value head) over dv.
 *   o, z, out [T][Hv][dv];  w [dv] shared by all heads.
 *   gate_sigmoid: 0 gates with SiLU(z), 1 with sigmoid(z).
 */
void orc_gated_rmsnorm(long long T, int Hv, int dv, const double *o, const double *z,
                       const double *w, double eps, int gate_sigmoid, double *out) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < T * Hv; ++r) {
    const double *orow = o + (size_t)r * dv;
    const double *zrow = z + (size_t)r * dv;
    double *dst = out + (size_t)r * dv;
    double ss = 0.0;
    for (int j = 0; j < dv; ++j) ss += orow[j] * orow[j];
    double inv = 1.0 / sqrt(ss / dv + eps);
    for (int j = 0; j < dv; ++j)
      dst[j] = orow[j] * inv * w[j] * (gate_sigmoid ? sigmoid(zrow[j]) : silu(zrow[j]));
  }
}
