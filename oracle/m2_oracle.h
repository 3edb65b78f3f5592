/* CPU oracle for the Mamba-2 mixer layer (and, further below, the attention layer and
 * the output heads of the same backbone): plain fp64 loops.
 *
 * TEST INFRASTRUCTURE ONLY. This code is the slow, obviously correct definition
 * that the HIP path is checked against. Only the tests, the smoke check and the
 * bench's CPU-baseline leg may load it; the product path never does. It shares
 * no code, header, table or helper with the HIP library.
 *
 * What it computes: the per-frame decode step of one Mamba-2 mixer layer of the
 * hybrid Mamba-2/attention backbone (page "NemotronLabs VoiceChat 11B: GPTQ
 * 3-bit LLM, MLX", introduction: Nemotron-Nano-9B-v2, Mamba-2 and attention;
 * page "NemotronLabs VoiceChat" (SGLang-Omni cookbook), introduction: one
 * token per 80 ms frame), and the prompt prefill (GPTQ page, "Recipe":
 * system-prompt prefill before streaming) as that many recurrent steps.
 * The pages print no equation of the mixer; the steps are:
 *   1. zxbcdt = W_in u                         (in_proj, no bias)
 *   2. split [z | xBC | dt_raw]
 *   3. causal depthwise conv (width d_conv) over xBC with bias, then SiLU;
 *      the cache holds the last d_conv-1 raw inputs, oldest first
 *   4. split the conv output into x (head-major), B and C (group-major)
 *   5. dt = softplus(dt_raw + dt_bias), A = -exp(A_log), dA = exp(dt A)
 *   6. S[h][p][n] = dA S[h][p][n] + dt x[h][p] B[g][n],  g = h / (H/G)
 *   7. y[h][p] = sum_n S[h][p][n] C[g][n] + D[h] x[h][p]    (updated S)
 *   8. v = y * SiLU(z)
 *   9. per group of norm_group channels: yn = v / sqrt(mean(v^2) + eps) * norm_w
 *  10. out = W_out yn  (optionally y = u + out: residual stack)
 * A second, independent definition of steps 5-7 over a sequence, the
 * materialised quadratic (attention-like) form, is orc_ssd_quadratic.
 *
 * Parity pins live in tests/test_oracle_pins.py.
 */
#ifndef M2_ORACLE_H
#define M2_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_W_F32 = 0, ORC_W_BF16 = 1, ORC_W_INT8G = 2, ORC_W_INT4G = 3, ORC_W_INT3G = 4 };

typedef struct {
  int32_t d_model, n_heads, head_dim, d_state, n_groups, d_conv;
  int32_t norm_group;          /* channels per RMS group (> 0) */
  double norm_eps;
  int32_t wtype;               /* ORC_W_* */
  int32_t q_group;             /* K-group of the int8 scales / low-bit (scale, bias) pairs */
  double q_gamma_in, q_gamma_out;
} orc_cfg;

/* Low-bit weights (the GPTQ page, introduction and "Details": the LLM quantized to
 * 3 bits with groups of 64, and a 4-bit build): unsigned codes q with, per row and per
 * q_group columns, an fp16 (scale, bias) pair; w = gamma (scale q + bias). Packing:
 * see orc_lowbit_code. */
typedef struct {
  const void *w_in;            /* [d_in_proj][d_model]: float, bf16 bits (uint16), int8, or packed codes */
  const uint16_t *s_in;        /* fp16 bits: int8 scales [d_in_proj][d_model/q_group], low-bit
                                  (scale, bias) pairs [d_in_proj][d_model/q_group][2] */
  const void *w_out;           /* [d_model][d_inner] */
  const uint16_t *s_out;       /* as s_in, [d_model][d_inner/q_group]([2]) */
  const float *conv_w;         /* [conv_dim][d_conv], tap d_conv-1 = newest */
  const float *conv_b;         /* [conv_dim] */
  const float *dt_bias, *A_log, *D;   /* [n_heads] */
  const float *norm_w;         /* [d_inner] */
} orc_weights;

/* Optional intermediates of the last token processed, all [batch][...] doubles. */
typedef struct {
  double *zxbcdt;              /* [B][d_in_proj] */
  double *xconv;               /* [B][conv_dim] conv + SiLU output */
  double *dt;                  /* [B][n_heads] softplus output */
  double *y;                   /* [B][d_inner] SSM readout incl. D x */
  double *v;                   /* [B][d_inner] gated */
  double *yn;                  /* [B][d_inner] normalised */
  double *out;                 /* [B][d_model] out_proj result (before residual) */
} orc_trace;

/* One token for `batch` sessions. ssm [n_slots][H][P][N], conv [n_slots][d_conv-1][conv_dim]
 * are updated in place for the slots named by slot_ids (NULL: session b uses slot b).
 * x, y: [batch][d_model]. residual != 0 gives y = x + out. Returns 0, or -1 on bad arguments. */
int orc_step(const orc_cfg *cfg, const orc_weights *w, double *ssm, double *conv, int32_t n_slots,
             const double *x, double *y, int32_t batch, const int32_t *slot_ids, int32_t residual,
             orc_trace *trace);

/* Code k (unsigned) of row `row` of a packed low-bit [rows][K] matrix (wtype ORC_W_INT4G or
 * ORC_W_INT3G). */
int32_t orc_lowbit_code(int32_t wtype, const void *w, int64_t row, int64_t K, int64_t k);

/* Prompt prefill as `seqlen` recurrent steps: x, y [batch][seqlen][d_model]. */
int orc_prefill(const orc_cfg *cfg, const orc_weights *w, double *ssm, double *conv, int32_t n_slots,
                const double *x, double *y, int32_t batch, int32_t seqlen, const int32_t *slot_ids,
                int32_t residual);

/* Steps 5-7 alone, token by token over T tokens (the same code orc_step uses).
 * x [T][H][P], Bm and Cm [T][G][N], dt [T][H] (already softplus'd), A [H] (negative),
 * D [H]; S [H][P][N] is updated in place; y [T][H][P]. */
void orc_ssd_recurrent(int32_t T, int32_t H, int32_t P, int32_t N, int32_t G, const double *x,
                       const double *Bm, const double *Cm, const double *dt, const double *A,
                       const double *D, double *S, double *y);

/* The same map as a materialised quadratic form:
 *   cs_t = sum_{r<=t} dt_r A
 *   y_t  = sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) dt_s x_s + exp(cs_t) C_t S0 + D x_t
 *   S_T  = exp(cs_{T-1}) S0 + sum_s exp(cs_{T-1} - cs_s) dt_s x_s (x) B_s
 * S0 [H][P][N] is read; S_final [H][P][N] written (may be NULL). */
void orc_ssd_quadratic(int32_t T, int32_t H, int32_t P, int32_t N, int32_t G, const double *x,
                       const double *Bm, const double *Cm, const double *dt, const double *A,
                       const double *D, const double *S0, double *y, double *S_final);

/* Output head (page "NemotronLabs VoiceChat" of the SGLang-Omni cookbook, introduction and
 * "Request parameters": every frame yields a token from each of two heads, text and
 * function, chosen greedily). For each session b < B: logits[b][v] = W[v] . h[b] for a
 * [vocab][K] matrix in the layer's weight formats (quantized types times gamma), and
 * token[b] = the lowest v whose logit is the largest; a NaN logit is never chosen, -1 if all are NaN.
 * Returns 0, or -1 on bad arguments. */
int orc_head_argmax(int32_t wtype, int32_t q_group, double gamma, int64_t vocab, int64_t K, const void *w,
                    const uint16_t *s, const double *h, int32_t B, double *logits, int32_t *token);

/* Attention layer of the hybrid backbone, one decode token per session (blog page
 * "NemotronLabs VoiceChat 11B" overview, "Key design decisions" item 2: Mamba layers
 * alternate with attention layers; its "Known limitations": a 2-minute audio context; the
 * SGLang-Omni cookbook page, "Known limitations": the backbone and its KV cache run in
 * bfloat16). The pages print no attention equation; the steps are standard scaled
 * dot-product attention with grouped key/value heads and no positional term:
 *   1. qkv = W_qkv u, rows [q: n_q heads x D | k: n_kv x D | v: n_kv x D], no bias
 *   2. k and v rounded to bfloat16 (nearest, ties to even) and stored at position pos of
 *      the session's cache [n_kv][max_len][D]
 *   3. query head h reads key/value head g = h / (n_q / n_kv):
 *      s_j = q_h . K_g[j] / sqrt(D) for j = 0 .. pos (the new entry included)
 *   4. p = softmax(s); o_h = sum_j p_j V_g[j]
 *   5. out = W_o o (o head-major, n_q x D), y = out or u + out; pos += 1
 * A session whose pos is already max_len (or whose slot is out of range) gets NaN outputs
 * and its cache and pos are not touched. */
typedef struct {
  int32_t d_model, n_q, n_kv, head_dim, max_len;
  int32_t wtype, q_group;          /* weight format of W_qkv and W_o, as for the mixer */
  double q_gamma_qkv, q_gamma_o;
} orc_attn_cfg;

/* kc, vc: bf16 bits [n_slots][n_kv][max_len][D]; pos: [n_slots]; x, y: [B][d_model];
 * qkv_out ([B][(n_q + 2 n_kv) D]) and o_out ([B][n_q D]) receive intermediates if non-NULL.
 * Returns 0, or -1 on bad arguments. */
int orc_attn_step(const orc_attn_cfg *c, const void *w_qkv, const uint16_t *s_qkv, const void *w_o,
                  const uint16_t *s_o, uint16_t *kc, uint16_t *vc, int32_t *pos, int32_t n_slots,
                  const double *x, double *y, int32_t B, const int32_t *slot_ids, int32_t residual,
                  double *qkv_out, double *o_out);

/* bfloat16 bits of the value nearest to v (ties to even; beyond the largest finite
 * bfloat16 by half a step or more: infinity). */
uint16_t orc_double_to_bf16(double v);

/* Helpers exposed so tests can pin them: element decoders and scalar functions. */
double orc_bf16_to_double(uint16_t h);
double orc_fp16_to_double(uint16_t h);
double orc_softplus(double x);
double orc_silu(double x);

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
