/* m2.h: C ABI of libm2.so, the MI355X (gfx950) Mamba-2 mixer layer.
 *
 * The operation is one Mamba-2 mixer layer of the hybrid Mamba-2/attention LLM
 * backbone of a full-duplex speech model (page "NemotronLabs VoiceChat 11B:
 * GPTQ 3-bit LLM, MLX", introduction: Nemotron-Nano-9B-v2, a hybrid of Mamba-2
 * and attention with 56 layers; page "NVIDIA NemotronLabs VoiceChat 11B: The
 * First Open Full-Duplex Voice Model with Tool Calling", "Key design
 * decisions" 2: Mamba keeps inference linear in the length of the streamed
 * 80 ms frames). Two entry points:
 *   m2_step     one token per session per 80 ms frame (page "NemotronLabs
 *               VoiceChat", SGLang-Omni cookbook, introduction: the thinker
 *               emits one token per frame; "Request parameters": one token per
 *               80 ms of input);
 *   m2_prefill  a whole prompt, before streaming starts (GPTQ page, "Recipe":
 *               system-prompt prefill, then the user's speech; cookbook "Known
 *               limitations": the system-prompt region is walked before frame 0).
 * The pages print no equation of the mixer. The layer computes, per token:
 *   zxbcdt = W_in u, split [z | x | B | C | dt_raw] (x head-major, B and C
 *   group-major); causal depthwise conv (width d_conv, bias, SiLU) over x|B|C
 *   with a cache of the last d_conv-1 raw inputs; dt = softplus(dt_raw+dt_bias);
 *   A = -exp(A_log); S = exp(dt A) S + dt x B^T; y = C.S + D x; v = y*SiLU(z);
 *   grouped RMSNorm with weight; out = W_out yn; optionally y = u + out.
 *
 * Memory: every pointer passed to these calls is a DEVICE pointer owned by
 * the caller, except the m2_config / m2_weights structs themselves and the
 * size outputs, which are host memory. Handles borrow pointers; no call frees
 * caller memory. Float activations, states and small parameters are fp32.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = default stream).
 * m2_step, m2_prefill and m2_state_zero only enqueue kernels: they never
 * allocate, never synchronise and never enqueue a memset, so they can be
 * captured into a HIP graph.
 *
 * Errors: every argument check runs on the host before anything is enqueued.
 * On failure a call returns a negative m2_status, enqueues nothing, and
 * m2_last_error() (thread-local) describes the failure. A failed launch
 * returns M2_ERR_HIP. Device-side faults surface at the caller's next
 * synchronisation. Slot ids live in device memory and cannot be checked on the
 * host: a session whose slot id is outside [0, n_slots) gets NaN outputs and
 * touches no state; slot ids within one call must be distinct (not checked).
 */
#ifndef M2_H
#define M2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define M2_ABI_VERSION 2

typedef enum {
  M2_OK = 0,
  M2_ERR_NULL = -1,         /* a required pointer or handle is NULL */
  M2_ERR_SHAPE = -2,        /* dimensions inconsistent or unsupported */
  M2_ERR_DTYPE = -3,        /* unknown weight type */
  M2_ERR_ALIGN = -4,        /* a device pointer is not 16-byte aligned */
  M2_ERR_WORKSPACE = -5,    /* ws_bytes smaller than the *_workspace size, or ws NULL */
  M2_ERR_SLOT = -6,         /* batch larger than the state's slot count */
  M2_ERR_UNSUPPORTED = -7,  /* valid but not implemented combination */
  M2_ERR_HIP = -8           /* HIP runtime error (message carries the HIP error string) */
} m2_status;

/* Storage of the two projection matrices. */
typedef enum {
  M2_W_F32 = 0,             /* float32 */
  M2_W_BF16 = 1,            /* bfloat16 */
  M2_W_INT8G = 2,           /* int8, symmetric, one fp16 scale per (row, q_group columns) */
  /* Low-bit weights (page "NemotronLabs VoiceChat 11B: GPTQ 3-bit LLM, MLX", introduction
     and "Details": the LLM quantized to 3 bits with groups of 64, and a 4-bit build):
     unsigned codes q, and per (row, q_group columns) an fp16 (scale, bias) pair;
     w = scale * q + bias (times q_gamma). A row of K codes is packed as */
  M2_W_INT4G = 3,           /* K/2 bytes: byte j holds code 2j in bits 0-3, code 2j+1 in bits 4-7 */
  M2_W_INT3G = 4            /* 3K/8 bytes: every 32 codes fill 12 bytes read as one little-endian
                               96-bit integer, code i of the run in bits 3i .. 3i+2 */
} m2_wtype;

/* flags */
enum {
  M2_RESIDUAL = 1,          /* y = x + mixer(x); y may alias x */
  M2_PERSISTENT = 2         /* m2_step: run plan 2 where it applies (see m2_step_plan) */
};

typedef struct {
  int32_t d_model;          /* model width (K of in_proj); multiple of 16 */
  int32_t n_heads;          /* H */
  int32_t head_dim;         /* P (multiple of 4); d_inner = H * P */
  int32_t d_state;          /* N */
  int32_t n_groups;         /* G: B/C groups; H % G == 0; head h uses group h / (H/G) */
  int32_t d_conv;           /* causal conv width, 2..8 */
  int32_t norm_group;       /* channels per RMS group (multiple of 4); 0 means d_inner / n_groups */
  float norm_eps;           /* RMSNorm epsilon */
  int32_t wtype;            /* m2_wtype */
  int32_t q_group;          /* columns per scale: M2_W_INT8G power of two >= 16; low-bit types
                               power of two >= 32 */
  float q_gamma_in;         /* per-tensor multiplier applied to quantized in_proj results (1 = none) */
  float q_gamma_out;        /* per-tensor multiplier applied to quantized out_proj results */
} m2_config;

/* Layer parameters, all device pointers, each 16-byte aligned, row-major. */
typedef struct {
  const void *w_in;         /* [d_in_proj][d_model], d_in_proj = 2 d_inner + 2 G N + H;
                               rows [z: d_inner | x: d_inner | B: G N | C: G N | dt: H] */
  const void *s_in;         /* int8: fp16 scales [d_in_proj][d_model / q_group]; low-bit: fp16
                               (scale, bias) pairs [d_in_proj][d_model / q_group][2]; else NULL */
  const void *w_out;        /* [d_model][d_inner] */
  const void *s_out;        /* as s_in, [d_model][d_inner / q_group]([2]) */
  const float *conv_w;      /* [conv_dim][d_conv], conv_dim = d_inner + 2 G N; tap d_conv-1 = newest */
  const float *conv_b;      /* [conv_dim] */
  const float *dt_bias;     /* [H] */
  const float *A_log;       /* [H]: A = -exp(A_log) */
  const float *D;           /* [H] */
  const float *norm_w;      /* [d_inner] */
  /* Optional (NULL: not used): w_in / w_out of a bf16 or int8 layer repacked into 16-row
     panels by m2_pack_panels. The batched decode step (3 to 32 sessions) and the bf16
     prefill GEMMs then read these instead of w_in / w_out (same results, bit for bit);
     every other path reads w_in / w_out. */
  const void *w_in_panels;  /* m2_panels_bytes(wtype, d_in_proj, d_model) bytes */
  const void *w_out_panels; /* m2_panels_bytes(wtype, d_model, d_inner) bytes */
} m2_weights;

typedef struct m2_layer_s *m2_layer;  /* borrows the m2_weights pointers; immutable */
typedef struct m2_state_s *m2_state;  /* borrows the ssm and conv buffers */

/* Version of this ABI (M2_ABI_VERSION). */
int m2_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *m2_last_error(void);

/* Validate cfg and w and create a layer handle (host memory only; no HIP call). */
int m2_layer_create(const m2_config *cfg, const m2_weights *w, m2_layer *out);
void m2_layer_destroy(m2_layer layer);

/* Panel layout of the projections W_in and W_out (the zxbcdt = W_in u and out = W_out yn
 * products above) for the batched decode step, whose matrix-core GEMVs take 16 rows x 32
 * columns per instruction, and for the bf16 prefill GEMMs: the matrix is cut into panels of 16 rows (the last one padded
 * with zero rows), each stored as ceil(K/32) steps of 32 columns (the last padded with
 * zeros); step s of panel p is 64 fragments of 8 consecutive elements in fragment order,
 * fragment l holding row 16p + l%16, columns 32s + 8(l/16) .. +7, so that one load
 * instruction of a wave reads whole cache lines.
 * m2_panels_bytes: the size of the panel copy of a [rows][K] matrix of wtype (M2_W_BF16 or
 * M2_W_INT8G); 0 for other types or rows, K <= 0.
 * m2_pack_panels: enqueue on `stream` the kernel that writes the panel copy of the device
 * row-major matrix w ([rows][K], wtype; any alignment) into out (device, m2_panels_bytes
 * bytes, 16-byte aligned, not overlapping w). Int8 scales are not repacked. Returns
 * M2_ERR_DTYPE for other types, M2_ERR_SHAPE for rows or K <= 0 or above 2^24,
 * M2_ERR_NULL / M2_ERR_ALIGN for the pointers, M2_ERR_HIP if the launch fails. */
size_t m2_panels_bytes(int32_t wtype, int32_t rows, int32_t K);
int m2_pack_panels(int32_t wtype, const void *w, int32_t rows, int32_t K, void *out, void *stream);

/* Bytes of the per-layer state buffers for n_slots sessions:
 *   ssm  fp32 [n_slots][H][P][N]           (N contiguous)
 *   conv fp32 [n_slots][d_conv-1][conv_dim] (oldest raw input first) */
int m2_state_sizes(const m2_config *cfg, int32_t n_slots, size_t *ssm_bytes, size_t *conv_bytes);

/* Wrap caller-owned ssm / conv buffers (sizes from m2_state_sizes) as a state handle. */
int m2_state_create(m2_layer layer, int32_t n_slots, float *ssm, float *conv, m2_state *out);
void m2_state_destroy(m2_state st);

/* Zero the state and conv cache of the n slots listed in slot_ids (device int32[n]);
 * slot_ids == NULL zeroes every slot (n ignored). Session rollover. */
int m2_state_zero(m2_state st, const int32_t *slot_ids, int32_t n, void *stream);

/* Workspace bytes m2_step needs for `batch` sessions. */
size_t m2_step_workspace(m2_layer layer, int32_t batch);

/* One decode step for `batch` sessions: x, y fp32 [batch][d_model]; session b
 * uses state slot slot_ids[b] (device int32[batch]) or slot b if slot_ids is
 * NULL. Updates those slots' ssm and conv state in place. flags: M2_RESIDUAL.
 * ws: device workspace of at least m2_step_workspace(layer, batch) bytes. */
int m2_step(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch,
            const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes, void *stream);

/* m2_step that also records hipEvent_t events[0..3] on `stream`: events[0] before the
 * step and events[i] after its i-th phase (see m2_step_plan); a phase is one kernel,
 * or two or three for plan 1. For per-phase timing; the events must have been
 * created by the caller. NULL events are skipped. */
int m2_step_timed(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch,
                  const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes, void *stream,
                  void *const *events);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): m2_step with no workspace argument. Its
 * workspace is a static device array of M2_NOALLOC_SCRATCH_BYTES per GPU, held by the
 * library until the process ends and shared by every call on that GPU; the first call on a
 * device looks up the array's device address (no allocation). It makes no allocating call.
 * Steps whose m2_step_workspace exceeds the array fail with M2_ERR_WORKSPACE (at the 9B
 * shape: up to 32 sessions fit). Calls that overlap on one GPU (other streams, other
 * threads) race on the array: serialise them. Arguments, results and errors otherwise as
 * m2_step. */
#define M2_NOALLOC_SCRATCH_BYTES (16u << 20)
size_t m2_noalloc_scratch_bytes(void);
int m2_step_noalloc(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch,
                    const int32_t *slot_ids, int32_t flags, void *stream);

/* How m2_step runs `batch` sessions. Every plan has three phases: in_proj | conv + SSD
 * update + readout + gate | RMSNorm + out_proj.
 *   0  VALU GEMVs: one kernel per phase
 *   1  MFMA GEMVs (batch 3..32 with bf16 weights, or int8 weights whose q_group is
 *      a multiple of 32 up to 256): in_proj GEMV + reduction | SSD | RMS factors +
 *      out_proj GEMV + reduction
 *   2  only when asked for with M2_PERSISTENT (slower than plan 0 on MI355X), for one
 *      session with bf16 weights on a device where two workgroups of the persistent kernel
 *      fit on every CU (shapes up to d_model 2 x CUs x 9 = 4608 on 256 CUs, d_inner 12288,
 *      and n_heads x head_dim / prange no larger than 2 x CUs, prange being the layer's SSD
 *      row range: the largest multiple of 4 up to 32 dividing gcd(head_dim, norm_group)): the
 *      in_proj GEMV of plan 0,
 *      then the SSD update and out_proj in one persistent kernel whose workgroups meet at
 *      one grid-wide barrier, out_proj's weights in flight across it.
 * m2_step_timed's events delimit the phases of plans 0 and 1; with plan 2, events[2] and
 * events[3] are both recorded after the persistent kernel. m2_step_plan gives the plan
 * without flags (never 2). Returns -1 for a NULL layer or batch <= 0. */
int m2_step_plan(m2_layer layer, int32_t batch);

/* The plan m2_step runs for `batch` sessions with these flags (2 where M2_PERSISTENT is set
 * and plan 2 applies on the current device; -1 as m2_step_plan, or for unknown flags). */
int m2_step_plan_flags(m2_layer layer, int32_t batch, int32_t flags);

/* Workspace bytes m2_prefill needs. */
size_t m2_prefill_workspace(m2_layer layer, int32_t batch, int32_t seqlen, int32_t chunk);

/* Prefill `seqlen` tokens for `batch` sessions with the chunked SSD scan
 * (chunk tokens per chunk, a multiple of 16 in [16, 256]; the last chunk may be
 * partial). x, y fp32 [batch][seqlen][d_model]. Starts from each slot's current
 * state and conv cache and leaves them as seqlen calls of m2_step would. */
int m2_prefill(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch,
               int32_t seqlen, int32_t chunk, const int32_t *slot_ids, int32_t flags, void *ws,
               size_t ws_bytes, void *stream);

/* Output heads (page "NemotronLabs VoiceChat" of the SGLang-Omni cookbook, introduction and
 * "Request parameters": every 80 ms frame yields a token from each of two heads, text and
 * function, chosen greedily). A head is a [vocab][d_model] matrix W; for each
 * session b, logits[b][v] = W[v] . h[b] (times q_gamma for quantized types) and the
 * token is argmax_v logits[b][v]: the lowest index among equal maxima, a NaN logit never
 * chosen, -1 if every logit is NaN. Call once per head. */
typedef struct {
  int32_t d_model;          /* K, at most 8192: a multiple of 4 (f32), 8 (bf16), 16 (int8) or 32 (low-bit) */
  int32_t vocab;            /* rows V, 1 .. 2^24 */
  int32_t wtype;            /* m2_wtype; packing and scales as for the layer's matrices */
  int32_t q_group;          /* quantized types: as m2_config.q_group; must divide d_model */
  float q_gamma;            /* quantized types: per-tensor multiplier (1 = none) */
} m2_head_config;

/* Workspace bytes m2_head_argmax needs (any batch; partial maxima of one launch). */
size_t m2_head_workspace(const m2_head_config *cfg, int32_t batch);

/* Greedy decode of one head for `batch` sessions. w: device [vocab][d_model] (16-byte
 * aligned); scales: quantized types as s_in of m2_weights (else NULL); h: device fp32
 * [batch][d_model], 16-byte aligned; token: device int32 [batch]; logits: device fp32
 * [batch][vocab] or NULL (not written). Asynchronous on `stream`; errors as m2_status. */
int m2_head_argmax(const m2_head_config *cfg, const void *w, const void *scales, const float *h,
                   int32_t batch, int32_t *token, float *logits, void *ws, size_t ws_bytes,
                   void *stream);

/* m2_head_argmax for at most 4 sessions (M2_ERR_UNSUPPORTED above) that also records
 * hipEvent_t events[0..2] on `stream`: before the GEMV kernel, between it and the argmax
 * reduction, and after the reduction. For per-kernel timing; the events must have been
 * created by the caller; NULL events are skipped. */
int m2_head_argmax_timed(const m2_head_config *cfg, const void *w, const void *scales, const float *h,
                         int32_t batch, int32_t *token, float *logits, void *ws, size_t ws_bytes,
                         void *stream, void *const *events);

/* Attention layers of the hybrid backbone (blog page "NemotronLabs VoiceChat 11B" overview,
 * "Key design decisions" item 2: Mamba layers alternate with attention layers; its "Known
 * limitations": a 2-minute audio context; SGLang-Omni cookbook page, "Known limitations":
 * the backbone and its KV cache run in bfloat16). One decode token per session:
 *   qkv = W_qkv u, rows [q: n_q heads x D | k: n_kv heads x D | v: n_kv heads x D] (no bias)
 *   the new k and v, rounded to bf16 (nearest, ties to even), are stored at position pos of
 *   the session's cache; query head h reads key/value head g = h / (n_q / n_kv):
 *   s_j = q_h . K_g[j] / sqrt(D), j = 0 .. pos; o_h = sum_j softmax(s)_j V_g[j]
 *   y = W_o o (o head-major), or u + W_o o under M2_RESIDUAL; pos += 1.
 * A session whose slot id is out of range or whose pos is already max_len gets NaN outputs
 * and its cache and pos are left as they were. */
typedef struct {
  int32_t d_model;          /* a multiple of 4 (f32), 8 (bf16), 16 (int8) or 32 (low-bit) */
  int32_t n_q;              /* query heads; a multiple of n_kv, at most 8 per key/value head */
  int32_t n_kv;             /* key/value heads */
  int32_t head_dim;         /* D: 64 or 128 */
  int32_t max_len;          /* cache positions per session, 1 .. 65536 */
  int32_t wtype;            /* m2_wtype of W_qkv and W_o */
  int32_t q_group;          /* quantized types: as m2_config.q_group; divides d_model and n_q D */
  float q_gamma_qkv;        /* quantized types: per-tensor multipliers (1 = none) */
  float q_gamma_o;
} m2_attn_config;

typedef struct {
  const void *w_qkv;        /* [(n_q + 2 n_kv) D][d_model], formats as m2_weights.w_in */
  const void *s_qkv;        /* quantized types: scales as m2_weights.s_in, else NULL */
  const void *w_o;          /* [d_model][n_q D] */
  const void *s_o;
} m2_attn_weights;

typedef struct m2_attn_s *m2_attn;   /* borrows the m2_attn_weights pointers; immutable */

int m2_attn_create(const m2_attn_config *cfg, const m2_attn_weights *w, m2_attn *out);
void m2_attn_destroy(m2_attn a);

/* Workspace bytes m2_attn_step needs for `batch` sessions (0 if batch <= 0). */
size_t m2_attn_workspace(m2_attn a, int32_t batch);

/* One decode token for `batch` sessions. k_cache, v_cache: device bf16 bits
 * [n_slots][n_kv][max_len][D], 16-byte aligned, caller-owned; pos: device int32 [n_slots]
 * (tokens already cached per slot), advanced in place; x, y: fp32 [batch][d_model] (y may
 * alias x); session b uses slot slot_ids[b] (device int32 [batch]) or b if NULL; flags:
 * M2_RESIDUAL. Asynchronous on `stream`; errors as m2_status. */
int m2_attn_step(m2_attn a, void *k_cache, void *v_cache, int32_t *pos, int32_t n_slots, const float *x,
                 float *y, int32_t batch, const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes,
                 void *stream);

/* m2_attn_step that also records hipEvent_t events[0..4] on `stream`: before the qkv GEMV
 * and after each of its four kernels (qkv GEMV, split attention, combine, o GEMV). For
 * per-kernel timing; NULL events are skipped. */
int m2_attn_step_timed(m2_attn a, void *k_cache, void *v_cache, int32_t *pos, int32_t n_slots,
                       const float *x, float *y, int32_t batch, const int32_t *slot_ids, int32_t flags,
                       void *ws, size_t ws_bytes, void *stream, void *const *events);

/* A hybrid layer stack (blog page "NemotronLabs VoiceChat 11B" overview, "Key design
 * decisions" item 2: Mamba layers alternate with attention layers) stepped by one call: a
 * table of layers in order, each a mixer (m2_layer + its m2_state) or an attention layer
 * (m2_attn + its KV cache and positions). One step for `batch` sessions is the residual
 * chain u_0 = x, u_{l+1} = u_l + layer_l(u_l), y = u_L, enqueued layer by layer on `stream`
 * (capturable into one graph by the caller). Every layer must have the same d_model; all
 * layers' states and caches hold n_slots session slots addressed by the same slot ids. */
enum { M2_LAYER_MIXER = 0, M2_LAYER_ATTN = 1 };

typedef struct {
  int32_t kind;             /* M2_LAYER_MIXER or M2_LAYER_ATTN */
  void *layer;              /* m2_layer or m2_attn (borrowed) */
  void *state;              /* mixer: its m2_state (borrowed); attention: NULL */
  void *k_cache, *v_cache;  /* attention: the layer's caches, as m2_attn_step; mixer: NULL */
  int32_t *pos;             /* attention: the layer's positions [n_slots]; mixer: NULL */
} m2_stack_layer;

typedef struct m2_stack_s *m2_stack;

/* Copies the table (not what it points to). Where a GPU is present it also copies the
 * mixers' arguments into a small table on the current device (for m2_stack_step_flags);
 * m2_stack_destroy frees it. Errors: a NULL or unknown entry, layers of different d_model, a
 * mixer state with fewer than n_slots slots, M2_ERR_HIP if that table cannot be made. */
int m2_stack_create(const m2_stack_layer *layers, int32_t n_layers, int32_t n_slots, m2_stack *out);
void m2_stack_destroy(m2_stack s);

/* Workspace bytes m2_stack_step needs for `batch` sessions: the largest of its layers'. */
size_t m2_stack_workspace(m2_stack s, int32_t batch);

/* One step of every layer in order for `batch` sessions: x, y fp32 [batch][d_model] (y may
 * alias x); session b uses slot slot_ids[b] (device int32 [batch]) or b if NULL. */
int m2_stack_step(m2_stack s, const float *x, float *y, int32_t batch, const int32_t *slot_ids, void *ws,
                  size_t ws_bytes, void *stream);

/* The persistent stack step (blog page "NemotronLabs VoiceChat 11B", "Key design decisions"
 * item 2: the backbone is one deep stack of Mamba-2 layers with attention layers among them,
 * stepped once per 80 ms frame). m2_stack_step with flags: M2_PERSISTENT runs every maximal
 * run of consecutive mixer layers in ONE kernel launch (plus a one-wave launch that clears
 * its barrier words) where the run applies: one session (batch 1), bf16 weights in every
 * layer of the run, each layer within plan 2's shape limits (m2_step_plan), and two
 * workgroups of the kernel resident on every CU of the device that was current at
 * m2_stack_create (the kernel's occupancy is checked on the host before each launch).
 * Inside the launch each layer is three phases with a grid-wide barrier after each:
 * in_proj (the arithmetic of plan 0's GEMV) | the SSD update (plan 2's) | out_proj +
 * residual (plan 2's); the residual stream between the run's layers, zx, v and the sums of
 * squares live in per-layer buffers of the workspace, written once and read past the
 * per-XCD caches. The results are bitwise those of calling m2_step with M2_PERSISTENT |
 * M2_RESIDUAL layer by layer. Every barrier wait is bounded: should the grid not be all
 * resident (another stream's kernels holding CUs; persistent steps on one device are best
 * serialised), the launch still ends, writes NaN over its run's outputs and leaves the run's
 * states undefined. Attention layers, runs where the path does not apply, and steps on a
 * device other than the table's, are stepped as by m2_stack_step. The workspace is
 * m2_stack_workspace_flags bytes: the persistent area (barrier words and per-layer buffers)
 * first, then m2_stack_workspace's. Errors as m2_stack_step, and M2_ERR_UNSUPPORTED for
 * unknown flags; with flags 0 the call is m2_stack_step. */
size_t m2_stack_workspace_flags(m2_stack s, int32_t batch, int32_t flags);
int m2_stack_step_flags(m2_stack s, const float *x, float *y, int32_t batch, const int32_t *slot_ids,
                        int32_t flags, void *ws, size_t ws_bytes, void *stream);
/* How many persistent launches m2_stack_step_flags makes per step for `batch` sessions (0
 * where the path does not apply; -1 for a NULL stack, batch <= 0 or unknown flags). */
int m2_stack_persistent_runs(m2_stack s, int32_t batch, int32_t flags);

#ifdef __cplusplus
}
#endif
#endif
