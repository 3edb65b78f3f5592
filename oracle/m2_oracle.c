/* CPU oracle for the Mamba-2 mixer layer, fp64. TEST INFRASTRUCTURE ONLY:
 * loaded by the tests, the smoke check and the bench's CPU-baseline leg, never
 * by the product path. The step list and its sources are in m2_oracle.h.
 *
 * Style: one plain loop per step of the definition, double everywhere, libm
 * exp/log1p/sqrt, OpenMP only across independent output rows and heads.
 * Nothing is blocked, fused or reordered beyond the definition.
 */
#include "m2_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element decoders (IEEE 754 binary16; bfloat16 = top half of binary32) ---- */

double orc_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double orc_fp16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m | 0x400), e - 25);    /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* Code k of row `row` of a low-bit [rows][K] weight matrix.
 * 4-bit: a row is K/2 bytes; byte j holds code 2j in bits 0-3 and code 2j+1 in bits 4-7.
 * 3-bit: a row is 3K/8 bytes; each run of 32 codes fills 12 bytes read as one 96-bit
 * little-endian integer, code i of the run in bits 3i .. 3i+2. */
int32_t orc_lowbit_code(int32_t wtype, const void *w, int64_t row, int64_t K, int64_t k) {
  const uint8_t *p = (const uint8_t *)w;
  if (wtype == ORC_W_INT4G) {
    const uint8_t byte = p[row * (K / 2) + k / 2];
    return (k & 1) ? byte >> 4 : byte & 15;
  }
  const uint8_t *blk = p + row * (K / 32) * 12 + (k / 32) * 12;
  const int64_t bit = 3 * (k % 32);
  uint32_t v = blk[bit / 8];
  if (bit % 8 > 5) v |= (uint32_t)blk[bit / 8 + 1] << 8;   /* the code straddles two bytes */
  return (int32_t)((v >> (bit % 8)) & 7);
}

/* ---- scalar functions ---- */

double orc_softplus(double x) {
  /* log(1 + e^x), written so that e^x never overflows */
  return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

double orc_silu(double x) { return x / (1.0 + exp(-x)); }

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the parallel loops that follow (n >= 1), for timing the oracle on one core. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---- weights ---- */

/* Row `row` of a [rows][K] weight matrix as doubles. */
static void dequant_row(const orc_cfg *c, const void *w, const uint16_t *s, int64_t row, int64_t K,
                        double gamma, double *dst) {
  if (c->wtype == ORC_W_F32) {
    const float *p = (const float *)w + row * K;
    for (int64_t k = 0; k < K; ++k) dst[k] = (double)p[k];
  } else if (c->wtype == ORC_W_BF16) {
    const uint16_t *p = (const uint16_t *)w + row * K;
    for (int64_t k = 0; k < K; ++k) dst[k] = orc_bf16_to_double(p[k]);
  } else if (c->wtype == ORC_W_INT8G) {
    const int8_t *p = (const int8_t *)w + row * K;
    const int64_t ng = K / c->q_group;
    for (int64_t j = 0; j < ng; ++j) {            /* one scale per q_group columns */
      const double sj = orc_fp16_to_double(s[row * ng + j]);
      for (int64_t k = j * c->q_group; k < (j + 1) * c->q_group; ++k) dst[k] = (double)p[k] * sj * gamma;
    }
  } else {
    /* low-bit affine groups: code q (unsigned, 4 or 3 bits), per q_group columns a
       (scale, bias) pair of fp16, w = gamma (scale q + bias) */
    const int64_t ng = K / c->q_group;
    for (int64_t k = 0; k < K; ++k) {
      const int32_t q = orc_lowbit_code(c->wtype, w, row, K, k);
      const int64_t j = k / c->q_group;
      const double sj = orc_fp16_to_double(s[(row * ng + j) * 2]);
      const double mj = orc_fp16_to_double(s[(row * ng + j) * 2 + 1]);
      dst[k] = (sj * (double)q + mj) * gamma;
    }
  }
}

/* out[b][r] = sum_k W[r][k] u[b][k] for b < B, r < rows. */
static void gemv(const orc_cfg *c, const void *w, const uint16_t *s, int64_t rows, int64_t K,
                 double gamma, const double *u, double *out, int64_t B) {
#pragma omp parallel
  {
    double *wr = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      dequant_row(c, w, s, r, K, gamma, wr);
      for (int64_t b = 0; b < B; ++b) {
        const double *ub = u + b * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += wr[k] * ub[k];
        out[b * rows + r] = acc;
      }
    }
    free(wr);
  }
}

int orc_head_argmax(int32_t wtype, int32_t q_group, double gamma, int64_t vocab, int64_t K, const void *w,
                    const uint16_t *s, const double *h, int32_t B, double *logits, int32_t *token) {
  if (wtype < ORC_W_F32 || wtype > ORC_W_INT3G || vocab < 1 || K < 1 || B < 1 || !w || !h || !logits || !token)
    return -1;
  if (wtype >= ORC_W_INT8G && (!s || q_group < 1 || K % q_group)) return -1;
  orc_cfg c;
  memset(&c, 0, sizeof c);
  c.wtype = wtype;
  c.q_group = q_group;
  gemv(&c, w, s, vocab, K, gamma, h, logits, B);
  for (int32_t b = 0; b < B; ++b) {
    int64_t best = -1;
    for (int64_t v = 0; v < vocab; ++v) {
      const double l = logits[b * vocab + v];
      if (isnan(l)) continue;
      if (best < 0 || l > logits[b * vocab + best]) best = v;   /* equal: the earlier index stays */
    }
    token[b] = (int32_t)best;
  }
  return 0;
}

/* ---- attention decode (orc_attn_step) ---- */

uint16_t orc_double_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  const uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                       /* a = f 2^e, f in [0.5, 1): leading bit at 2^(e-1) */
  int lsb = e - 8;                    /* 8 significant bits */
  if (lsb < -133) lsb = -133;         /* subnormal spacing 2^-133 */
  double r = nearbyint(ldexp(a, -lsb));   /* default rounding: to nearest, ties to even */
  r = ldexp(r, lsb);
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80;     /* overflow -> infinity */
  float f = (float)r;                 /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

int orc_attn_step(const orc_attn_cfg *c, const void *w_qkv, const uint16_t *s_qkv, const void *w_o,
                  const uint16_t *s_o, uint16_t *kc, uint16_t *vc, int32_t *pos, int32_t n_slots,
                  const double *x, double *y, int32_t B, const int32_t *slot_ids, int32_t residual,
                  double *qkv_out, double *o_out) {
  if (!c || !w_qkv || !w_o || !kc || !vc || !pos || !x || !y || B < 1 || n_slots < 1) return -1;
  if (c->n_q < 1 || c->n_kv < 1 || c->n_q % c->n_kv || c->head_dim < 1 || c->max_len < 1 || c->d_model < 1)
    return -1;
  if (c->wtype < ORC_W_F32 || c->wtype > ORC_W_INT3G) return -1;
  const int64_t D = c->head_dim, Hq = c->n_q, Hk = c->n_kv, L = c->max_len;
  const int64_t rows = (Hq + 2 * Hk) * D, K = c->d_model, Ko = Hq * D;
  if (c->wtype >= ORC_W_INT8G && (!s_qkv || !s_o || c->q_group < 1 || K % c->q_group || Ko % c->q_group))
    return -1;
  orc_cfg wc;
  memset(&wc, 0, sizeof wc);
  wc.wtype = c->wtype;
  wc.q_group = c->q_group;
  double *qkv = (double *)malloc(sizeof(double) * (size_t)(B * rows));
  double *o = (double *)malloc(sizeof(double) * (size_t)(B * Ko));
  double *out = (double *)malloc(sizeof(double) * (size_t)(B * K));
  double *sc = (double *)malloc(sizeof(double) * (size_t)L);
  /* step 1 */
  gemv(&wc, w_qkv, s_qkv, rows, K, c->q_gamma_qkv, x, qkv, B);
  if (qkv_out) memcpy(qkv_out, qkv, sizeof(double) * (size_t)(B * rows));
  int *live = (int *)malloc(sizeof(int) * (size_t)B);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t slot = slot_ids ? slot_ids[b] : b;
    live[b] = slot >= 0 && slot < n_slots && pos[slot] >= 0 && pos[slot] < L;
    double *ob = o + b * Ko;
    if (!live[b]) {
      for (int64_t i = 0; i < Ko; ++i) ob[i] = NAN;
      continue;
    }
    const int64_t t = pos[slot];
    const double *q = qkv + b * rows, *kn = q + Hq * D, *vn = kn + Hk * D;
    uint16_t *ks = kc + (size_t)slot * Hk * L * D, *vs = vc + (size_t)slot * Hk * L * D;
    /* step 2 */
    for (int64_t g = 0; g < Hk; ++g)
      for (int64_t d = 0; d < D; ++d) {
        ks[(g * L + t) * D + d] = orc_double_to_bf16(kn[g * D + d]);
        vs[(g * L + t) * D + d] = orc_double_to_bf16(vn[g * D + d]);
      }
    /* steps 3 and 4 */
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t g = h / (Hq / Hk);
      double m = -INFINITY;
      for (int64_t j = 0; j <= t; ++j) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += q[h * D + d] * orc_bf16_to_double(ks[(g * L + j) * D + d]);
        sc[j] = acc / sqrt((double)D);
        if (sc[j] > m) m = sc[j];
      }
      double den = 0.0;
      for (int64_t j = 0; j <= t; ++j) {
        sc[j] = exp(sc[j] - m);       /* softmax, shifted by the maximum (the same ratio) */
        den += sc[j];
      }
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j <= t; ++j) acc += sc[j] * orc_bf16_to_double(vs[(g * L + j) * D + d]);
        ob[h * D + d] = acc / den;
      }
    }
    pos[slot] = (int32_t)(t + 1);
  }
  if (o_out) memcpy(o_out, o, sizeof(double) * (size_t)(B * Ko));
  /* step 5 */
  gemv(&wc, w_o, s_o, K, Ko, c->q_gamma_o, o, out, B);
  for (int32_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < K; ++i)
      y[b * K + i] = live[b] ? (residual ? x[b * K + i] : 0.0) + out[b * K + i] : NAN;
  free(live);
  free(sc);
  free(out);
  free(o);
  free(qkv);
  return 0;
}

/* ---- SSD token update (steps 6 and 7 for one head) ---- */

static void ssd_token(int32_t P, int32_t N, double dt, double A, double D, const double *x,
                      const double *Bg, const double *Cg, double *S, double *y) {
  const double dA = exp(dt * A);
  for (int32_t p = 0; p < P; ++p)
    for (int32_t n = 0; n < N; ++n)
      S[(int64_t)p * N + n] = dA * S[(int64_t)p * N + n] + dt * x[p] * Bg[n];
  for (int32_t p = 0; p < P; ++p) {
    double acc = 0.0;
    for (int32_t n = 0; n < N; ++n) acc += S[(int64_t)p * N + n] * Cg[n];
    y[p] = acc + D * x[p];
  }
}

void orc_ssd_recurrent(int32_t T, int32_t H, int32_t P, int32_t N, int32_t G, const double *x,
                       const double *Bm, const double *Cm, const double *dt, const double *A,
                       const double *D, double *S, double *y) {
  const int32_t hpg = H / G;
  for (int32_t t = 0; t < T; ++t) {
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < H; ++h) {
      const int32_t g = h / hpg;
      ssd_token(P, N, dt[(int64_t)t * H + h], A[h], D[h], x + ((int64_t)t * H + h) * P,
                Bm + ((int64_t)t * G + g) * N, Cm + ((int64_t)t * G + g) * N,
                S + (int64_t)h * P * N, y + ((int64_t)t * H + h) * P);
    }
  }
}

void orc_ssd_quadratic(int32_t T, int32_t H, int32_t P, int32_t N, int32_t G, const double *x,
                       const double *Bm, const double *Cm, const double *dt, const double *A,
                       const double *D, const double *S0, double *y, double *S_final) {
  const int32_t hpg = H / G;
#pragma omp parallel for schedule(static)
  for (int32_t h = 0; h < H; ++h) {
    const int32_t g = h / hpg;
    double *cs = (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
    double run = 0.0;
    for (int32_t t = 0; t < T; ++t) {
      run += dt[(int64_t)t * H + h] * A[h];
      cs[t] = run;
    }
    const double *S0h = S0 + (int64_t)h * P * N;
    for (int32_t t = 0; t < T; ++t) {
      const double *Ct = Cm + ((int64_t)t * G + g) * N;
      for (int32_t p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int32_t s = 0; s <= t; ++s) {
          const double *Bs = Bm + ((int64_t)s * G + g) * N;
          double cb = 0.0;
          for (int32_t n = 0; n < N; ++n) cb += Ct[n] * Bs[n];
          acc += cb * exp(cs[t] - cs[s]) * dt[(int64_t)s * H + h] * x[((int64_t)s * H + h) * P + p];
        }
        double c_s0 = 0.0;
        for (int32_t n = 0; n < N; ++n) c_s0 += Ct[n] * S0h[(int64_t)p * N + n];
        acc += exp(cs[t]) * c_s0;
        y[((int64_t)t * H + h) * P + p] = acc + D[h] * x[((int64_t)t * H + h) * P + p];
      }
    }
    if (S_final) {
      double *Sf = S_final + (int64_t)h * P * N;
      const double cT = T > 0 ? cs[T - 1] : 0.0;
      for (int32_t p = 0; p < P; ++p)
        for (int32_t n = 0; n < N; ++n) {
          double acc = exp(cT) * S0h[(int64_t)p * N + n];
          for (int32_t s = 0; s < T; ++s)
            acc += exp(cT - cs[s]) * dt[(int64_t)s * H + h] * x[((int64_t)s * H + h) * P + p] *
                   Bm[((int64_t)s * G + g) * N + n];
          Sf[(int64_t)p * N + n] = acc;
        }
    }
    free(cs);
  }
}

/* ---- one decode step ---- */

static int check_cfg(const orc_cfg *c) {
  if (!c) return -1;
  if (c->d_model <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->d_state <= 0 ||
      c->n_groups <= 0 || c->d_conv < 2 || c->norm_group <= 0)
    return -1;
  if (c->n_heads % c->n_groups) return -1;
  if ((c->n_heads * c->head_dim) % c->norm_group) return -1;
  if (c->wtype == ORC_W_INT8G || c->wtype == ORC_W_INT4G || c->wtype == ORC_W_INT3G) {
    if (c->q_group <= 0 || c->d_model % c->q_group || (c->n_heads * c->head_dim) % c->q_group)
      return -1;
    if (c->wtype != ORC_W_INT8G && c->q_group % 32) return -1;   /* whole 32-code runs per group */
  } else if (c->wtype != ORC_W_F32 && c->wtype != ORC_W_BF16) {
    return -1;
  }
  return 0;
}

int orc_step(const orc_cfg *c, const orc_weights *w, double *ssm, double *conv, int32_t n_slots,
             const double *x, double *y, int32_t batch, const int32_t *slot_ids, int32_t residual,
             orc_trace *tr) {
  if (check_cfg(c) || !w || !ssm || !conv || !x || !y || batch <= 0) return -1;
  if (!slot_ids && batch > n_slots) return -1;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t sl = slot_ids ? slot_ids[b] : b;
    if (sl < 0 || sl >= n_slots) return -1;
    for (int32_t b2 = 0; b2 < b; ++b2)          /* sessions must own distinct slots */
      if (slot_ids && slot_ids[b2] == sl) return -1;
  }
  const int64_t Dm = c->d_model, H = c->n_heads, P = c->head_dim, N = c->d_state, G = c->n_groups;
  const int64_t Kc = c->d_conv;
  const int64_t d_inner = H * P, conv_dim = d_inner + 2 * G * N, d_in_proj = 2 * d_inner + 2 * G * N + H;
  const int64_t hpg = H / G;
  const int64_t B = batch;

  double *zx = (double *)malloc((size_t)(B * d_in_proj) * sizeof(double));
  double *xc = (double *)malloc((size_t)(B * conv_dim) * sizeof(double));
  double *dtv = (double *)malloc((size_t)(B * H) * sizeof(double));
  double *yv = (double *)malloc((size_t)(B * d_inner) * sizeof(double));
  double *v = (double *)malloc((size_t)(B * d_inner) * sizeof(double));
  double *yn = (double *)malloc((size_t)(B * d_inner) * sizeof(double));
  double *out = (double *)malloc((size_t)(B * Dm) * sizeof(double));

  /* 1. in_proj */
  gemv(c, w->w_in, w->s_in, d_in_proj, Dm, c->q_gamma_in, x, zx, B);

  for (int64_t b = 0; b < B; ++b) {
    const int64_t sl = slot_ids ? slot_ids[b] : b;
    const double *zb = zx + b * d_in_proj;
    /* 2-3. conv over xBC = zb[d_inner : d_inner + conv_dim] */
    double *cache = conv + sl * (Kc - 1) * conv_dim;
    for (int64_t ch = 0; ch < conv_dim; ++ch) {
      const double raw = zb[d_inner + ch];
      double a = (double)w->conv_b[ch];
      for (int64_t k = 0; k < Kc - 1; ++k) a += (double)w->conv_w[ch * Kc + k] * cache[k * conv_dim + ch];
      a += (double)w->conv_w[ch * Kc + Kc - 1] * raw;
      xc[b * conv_dim + ch] = orc_silu(a);
      for (int64_t k = 0; k + 1 < Kc - 1; ++k) cache[k * conv_dim + ch] = cache[(k + 1) * conv_dim + ch];
      cache[(Kc - 2) * conv_dim + ch] = raw;
    }
    /* 5. dt */
    for (int64_t h = 0; h < H; ++h)
      dtv[b * H + h] = orc_softplus(zb[d_inner + conv_dim + h] + (double)w->dt_bias[h]);
  }

  /* 4, 6, 7. state update and readout per (session, head) */
#pragma omp parallel for schedule(static) collapse(2)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h) {
      const int64_t sl = slot_ids ? slot_ids[b] : b;
      const int64_t g = h / hpg;
      const double *xb = xc + b * conv_dim;
      const double A = -exp((double)w->A_log[h]);
      ssd_token((int32_t)P, (int32_t)N, dtv[b * H + h], A, (double)w->D[h], xb + h * P,
                xb + d_inner + g * N, xb + d_inner + G * N + g * N, ssm + (sl * H + h) * P * N,
                yv + b * d_inner + h * P);
    }

  for (int64_t b = 0; b < B; ++b) {
    const double *zb = zx + b * d_in_proj;
    /* 8. gate */
    for (int64_t ch = 0; ch < d_inner; ++ch) v[b * d_inner + ch] = yv[b * d_inner + ch] * orc_silu(zb[ch]);
    /* 9. grouped RMSNorm */
    for (int64_t j = 0; j < d_inner / c->norm_group; ++j) {
      const int64_t c0 = j * c->norm_group;
      double ss = 0.0;
      for (int64_t ch = c0; ch < c0 + c->norm_group; ++ch) ss += v[b * d_inner + ch] * v[b * d_inner + ch];
      const double r = 1.0 / sqrt(ss / (double)c->norm_group + c->norm_eps);
      for (int64_t ch = c0; ch < c0 + c->norm_group; ++ch)
        yn[b * d_inner + ch] = v[b * d_inner + ch] * r * (double)w->norm_w[ch];
    }
  }

  /* 10. out_proj (+ residual) */
  gemv(c, w->w_out, w->s_out, Dm, d_inner, c->q_gamma_out, yn, out, B);
  for (int64_t i = 0; i < B * Dm; ++i) y[i] = residual ? x[i] + out[i] : out[i];

  if (tr) {
    if (tr->zxbcdt) memcpy(tr->zxbcdt, zx, (size_t)(B * d_in_proj) * sizeof(double));
    if (tr->xconv) memcpy(tr->xconv, xc, (size_t)(B * conv_dim) * sizeof(double));
    if (tr->dt) memcpy(tr->dt, dtv, (size_t)(B * H) * sizeof(double));
    if (tr->y) memcpy(tr->y, yv, (size_t)(B * d_inner) * sizeof(double));
    if (tr->v) memcpy(tr->v, v, (size_t)(B * d_inner) * sizeof(double));
    if (tr->yn) memcpy(tr->yn, yn, (size_t)(B * d_inner) * sizeof(double));
    if (tr->out) memcpy(tr->out, out, (size_t)(B * Dm) * sizeof(double));
  }
  free(zx); free(xc); free(dtv); free(yv); free(v); free(yn); free(out);
  return 0;
}

int orc_prefill(const orc_cfg *c, const orc_weights *w, double *ssm, double *conv, int32_t n_slots,
                const double *x, double *y, int32_t batch, int32_t seqlen, const int32_t *slot_ids,
                int32_t residual) {
  if (check_cfg(c) || batch <= 0 || seqlen < 0) return -1;
  const int64_t Dm = c->d_model, B = batch, T = seqlen;
  double *xt = (double *)malloc((size_t)(B * Dm) * sizeof(double));
  double *yt = (double *)malloc((size_t)(B * Dm) * sizeof(double));
  int rc = 0;
  for (int64_t t = 0; t < T && rc == 0; ++t) {
    for (int64_t b = 0; b < B; ++b) memcpy(xt + b * Dm, x + (b * T + t) * Dm, (size_t)Dm * sizeof(double));
    rc = orc_step(c, w, ssm, conv, n_slots, xt, yt, batch, slot_ids, residual, NULL);
    for (int64_t b = 0; b < B; ++b) memcpy(y + (b * T + t) * Dm, yt + b * Dm, (size_t)Dm * sizeof(double));
  }
  free(xt);
  free(yt);
  return rc;
}
