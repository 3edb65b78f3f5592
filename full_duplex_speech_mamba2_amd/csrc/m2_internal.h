// Internal declarations shared by the C-ABI layer (m2_api.cpp) and the HIP
// kernels (decode.hip, prefill.hip) of libm2.so. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "m2.h"

struct m2_layer_s {
  m2_config cfg;
  m2_weights w;
  // derived sizes
  int d_inner;      // H * P
  int conv_dim;     // d_inner + 2 G N
  int d_in_proj;    // 2 d_inner + 2 G N + H
  int zx_stride;    // d_in_proj rounded up to 4 floats (workspace row stride)
  int hpg;          // heads per B/C group
  int ng;           // channels per RMS group
  int n_norm;       // RMS groups: d_inner / ng
  int prange;       // head_dim rows per SSD workgroup (divides head_dim and ng)
  int psplit;       // head_dim / prange
  int n_partials;   // d_inner / prange sum-of-squares partials per session
};

struct m2_state_s {
  const m2_layer_s *layer;
  int n_slots;
  float *ssm;       // [n_slots][H][P][N]
  float *conv;      // [n_slots][d_conv-1][conv_dim]
};

struct m2_attn_s {
  m2_attn_config cfg;
  m2_attn_weights w;
  int qkv_rows;     // (n_q + 2 n_kv) head_dim
  int o_dim;        // n_q head_dim
  int nsplit;       // 64-position chunks of max_len
};

namespace m2d {

// Workspace carve-up of one decode step for `batch` sessions.
struct StepWs {
  float *zx;        // [B][d_in_proj]: z raw | conv+SiLU(x|B|C) | softplus dt
  float *v;         // [B][d_inner]: gated SSD output
  float *ss;        // [B][n_partials]: sums of squares of v per partial range
  float *part;      // MFMA GEMVs: K-chunk partial sums [KS][B][rows]
  unsigned *bar;    // plan 2: the persistent kernel's grid-barrier words
  size_t bytes;
};
StepWs step_ws_layout(const m2_layer_s &L, int batch, void *base);

hipError_t launch_step(const m2_layer_s &L, const m2_state_s &S, const float *x, float *y, int batch,
                       const int32_t *slots, int flags, const StepWs &ws, hipStream_t stream,
                       hipEvent_t const *events = nullptr);

// Kernel plan of a decode step of `batch` sessions (m2_step_plan); flags may hold
// M2_PERSISTENT, which asks for plan 2 where it applies.
enum { kPlanValu = 0, kPlanMfma = 1, kPlanFused = 2 };
int step_plan(const m2_layer_s &L, int batch, int flags = 0);

// Plan 2's persistent SSD + out_proj kernel (fused.hip): the grid it runs with on the
// current device (0: it cannot), whether the layer's shapes fit it, and its launch.
int fused_grid(const m2_layer_s &L);
bool fused_fits(const m2_layer_s &L, int grid);
hipError_t launch_fused_step(const m2_layer_s &L, const m2_state_s &S, const float *x, float *y,
                             const int32_t *slots, int flags, const StepWs &ws, int grid, hipStream_t stream);
// The persistent stack step (fused.hip): one launch runs a run of consecutive mixer layers
// (one session, bf16). Its workspace area: the barrier words (stack_area_head bytes), then
// stack_area_layer_bytes per layer; a device table holds one stack_rec_bytes record per
// layer of the stack (stack_rec_fill writes a mixer's, `off` its buffers' area offset).
size_t stack_area_head();
size_t stack_area_layer_bytes(const m2_layer_s &L);
size_t stack_rec_bytes();
void stack_rec_fill(const m2_layer_s &L, const m2_state_s &S, size_t off, void *out);
size_t stack_lds_bytes(const m2_layer_s &L);
int stack_grid(size_t lds);
bool stack_fits(const m2_layer_s &L, int grid);
hipError_t launch_stack_run(const void *tab, int l0, int l1, size_t lds, void *area, float *y,
                            const int32_t *slots, int n_slots, int grid, hipStream_t stream);
// Whether a step of `batch` sessions runs its projections as MFMA GEMVs.
bool step_uses_mfma(const m2_layer_s &L, int batch);

hipError_t launch_state_zero(const m2_state_s &S, const int32_t *slots, int n, hipStream_t stream);
// 16-row panel copies of a [rows][K] bf16 or int8 matrix (the batched decode GEMVs' weight
// layout): their size (0 for other types), and the packing kernel.
size_t panels_bytes(int wtype, int rows, int K);
hipError_t launch_pack_panels(int wtype, const void *w, int rows, int K, void *out, hipStream_t stream);

// Output heads: greedy argmax of W h (m2_head_argmax).
size_t head_ws_bytes(int vocab);
hipError_t launch_head(const m2_head_config &c, const void *w, const void *scales, const float *h, int batch,
                       int32_t *token, float *logits, void *ws, hipStream_t stream,
                       hipEvent_t const *events = nullptr);

// y[b] = gamma W act[b] (+ resid[b]) for a [rows][K] matrix in any weight format, with the
// decode step's GEMV kernels (plain epilogue); `part` holds gemv_plain_part_bytes of
// K-chunk partial sums when the MFMA GEMV is used (3-32 sessions, bf16 or int8 g128/g256).
bool gemv_plain_uses_mfma(int wtype, int q_group, int batch);
size_t gemv_plain_part_bytes(int wtype, int q_group, int rows, int K, int batch);
hipError_t launch_gemv_plain(int wtype, const void *W, const void *S, int rows, int K, int q_group, float gamma,
                             const float *act, int batch, float *y, const float *resid, float *part,
                             hipStream_t stream);

// Attention decode step (m2_attn_step).
int attn_nsplit(int max_len);
size_t attn_ws_bytes(const m2_attn_s &A, int batch);
hipError_t launch_attn_step(const m2_attn_s &A, uint16_t *kc, uint16_t *vc, int32_t *pos, int n_slots,
                            const float *x, float *y, int batch, const int32_t *slots, int flags, void *ws,
                            hipStream_t stream, hipEvent_t const *events = nullptr);

// Prefill
size_t prefill_ws_bytes(const m2_layer_s &L, int batch, int seqlen, int chunk);
hipError_t launch_prefill(const m2_layer_s &L, const m2_state_s &S, const float *x, float *y, int batch,
                          int seqlen, int chunk, const int32_t *slots, int flags, void *ws,
                          hipStream_t stream);

}  // namespace m2d
