// Decode step of the Mamba-2 mixer layer on gfx950: three kernels per step.
//
//   gemv_in   zxbcdt = W_in u, weight-streaming GEMV (16-byte loads of W, fp32
//             accumulate); the row epilogue applies softplus to the dt rows.
//   ssd_step  per (session, head, row range): causal conv + SiLU of the item's
//             x channels and of its group's B and C (cache read only), then
//             S = exp(dt A) S + dt x B^T and y = C.S + D x on the state tile held
//             in registers (one read, one write), v = y SiLU(z), written as
//             v * norm_w, and per-range sums of squares of v.
//   gemv_out  RMS factors from the sums of squares, yn = (v norm_w) r staged
//             into LDS, then out = W_out yn (+ residual); the same kernel shifts
//             the conv cache (the SSD kernel, its last reader, has finished).
//
// The operation follows the Mamba-2 layer the backbone of the pages uses (page
// "NemotronLabs VoiceChat 11B: GPTQ 3-bit LLM, MLX", introduction; page
// "NemotronLabs VoiceChat" of the SGLang-Omni cookbook, introduction: one token
// per 80 ms frame). The decode step is bound by streaming the two projection
// matrices from HBM (GPTQ page, introduction: the LLM step is limited by
// memory bandwidth), so the GEMVs are built around full 16-byte coalesced loads
// with several loads in flight per lane; the rest is small.
//
// Two GEMV shapes:
//   gemv_wave   batch <= 2: one wave per weight row, so every load instruction
//               reads 1 KB of one row; the activations of the batch are staged
//               whole into LDS after the first weight loads have been issued.
//   gemv_tiled  any batch: 16-lane row groups, K split inside the workgroup,
//               activations staged in K tiles for tiles of 4 sessions.
#include <hip/hip_fp16.h>

#include <climits>

#include "lanes.h"
#include "m2_internal.h"

namespace m2d {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kNormF4PerThread = 5;          // gemv_wave out_proj: float4 activations held per thread (K <= 10240 at 512 threads)
constexpr int kLdsFloatsPerBatch = 12288;   // tiled kernel: activation tile budget (48 KB at 1 session)

// Activations of the low-bit GEMV sit in LDS with 4 floats of padding after every 64: lane l
// reads the 32 floats of chunk l, and without the padding every lane of an LDS cycle falls
// on the same 4 banks. With it, the 16 lanes of one cycle read 16 distinct 4-bank groups
// (for any chunk of 4 to 32 floats). The bf16 wave GEMV reads 8-float chunks, a 2-way
// conflict that costs it nothing measurable; padding its rows made it slower, so it keeps
// them dense.
__host__ __device__ constexpr int lds_pad(int k) { return k + 4 * (k >> 6); }
__host__ __device__ constexpr int lds_padded(int K) { return lds_pad(K - 1) + 1; }   // a multiple of 4 for K % 4 == 0

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ float softplus(float a) { return a > 20.0f ? a : log1pf(expf(a)); }

__device__ __forceinline__ float i8(uint32_t u, int j) {
  return (float)((int32_t)(u << (24 - 8 * j)) >> 24);
}

// A weight row is read in chunks of EPC elements, CB bytes each: 16 bytes for every type
// but 3-bit codes, whose 32-code runs are 12 bytes.
template <int WT> struct WTraits;
template <> struct WTraits<M2_W_F32> { static constexpr int EPC = 4; static constexpr int CB = 16; using chunk_t = u32x4; };
template <> struct WTraits<M2_W_BF16> { static constexpr int EPC = 8; static constexpr int CB = 16; using chunk_t = u32x4; };
template <> struct WTraits<M2_W_INT8G> { static constexpr int EPC = 16; static constexpr int CB = 16; using chunk_t = u32x4; };
template <> struct WTraits<M2_W_INT4G> { static constexpr int EPC = 32; static constexpr int CB = 16; using chunk_t = u32x4; };
struct W3 { uint32_t x, y, z; };
template <> struct WTraits<M2_W_INT3G> { static constexpr int EPC = 32; static constexpr int CB = 12; using chunk_t = W3; };

template <int NT> __device__ __forceinline__ u32x4 wload(const u32x4 *p) {
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <int NT> __device__ __forceinline__ uint32_t wload1(const uint32_t *p) {
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}

// Chunk c of a row that starts at byte pointer rowp.
template <int WT, int NT>
__device__ __forceinline__ typename WTraits<WT>::chunk_t load_chunk(const char *rowp, int c) {
  if constexpr (WT == M2_W_INT3G) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(rowp + 12 * (size_t)c);
    return W3{wload1<NT>(p), wload1<NT>(p + 1), wload1<NT>(p + 2)};
  } else {
    return wload<NT>(reinterpret_cast<const u32x4 *>(rowp) + c);
  }
}

// Dot product of one 16-byte weight chunk with EPC consecutive fp32 activations.
template <int WT> __device__ __forceinline__ float chunk_dot(const u32x4 &w, const float *a);

template <> __device__ __forceinline__ float chunk_dot<M2_W_F32>(const u32x4 &w, const float *a) {
  const float4 x = *reinterpret_cast<const float4 *>(a);
  float s = __uint_as_float(w.x) * x.x;
  s = fmaf(__uint_as_float(w.y), x.y, s);
  s = fmaf(__uint_as_float(w.z), x.z, s);
  s = fmaf(__uint_as_float(w.w), x.w, s);
  return s;
}

template <> __device__ __forceinline__ float chunk_dot<M2_W_BF16>(const u32x4 &w, const float *a) {
  const float4 x0 = *reinterpret_cast<const float4 *>(a);
  const float4 x1 = *reinterpret_cast<const float4 *>(a + 4);
  float s = bf16_lo(w.x) * x0.x;
  s = fmaf(bf16_hi(w.x), x0.y, s);
  s = fmaf(bf16_lo(w.y), x0.z, s);
  s = fmaf(bf16_hi(w.y), x0.w, s);
  s = fmaf(bf16_lo(w.z), x1.x, s);
  s = fmaf(bf16_hi(w.z), x1.y, s);
  s = fmaf(bf16_lo(w.w), x1.z, s);
  s = fmaf(bf16_hi(w.w), x1.w, s);
  return s;
}

template <> __device__ __forceinline__ float chunk_dot<M2_W_INT8G>(const u32x4 &w, const float *a) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 x = *reinterpret_cast<const float4 *>(a + 4 * q);
    s = fmaf(i8(ws[q], 0), x.x, s);
    s = fmaf(i8(ws[q], 1), x.y, s);
    s = fmaf(i8(ws[q], 2), x.z, s);
    s = fmaf(i8(ws[q], 3), x.w, s);
  }
  return s;
}

// Low-bit chunks: 32 unsigned codes. 4-bit: word j holds codes 8j .. 8j+7, code 2i of the
// word in bits 8i .. 8i+3 and code 2i+1 in bits 8i+4 .. 8i+7. 3-bit: the three words are
// one little-endian 96-bit run, code i in bits 3i .. 3i+2.
__device__ __forceinline__ float lb4_code(const u32x4 &w, int i) {
  const uint32_t word = i < 8 ? w.x : i < 16 ? w.y : i < 24 ? w.z : w.w;
  return (float)((word >> (4 * (i & 7))) & 15u);
}

__device__ __forceinline__ float lb3_code(const W3 &w, int i) {
  const int bit = 3 * i, off = bit & 31;
  const uint32_t lo = bit < 32 ? w.x : bit < 64 ? w.y : w.z;
  if (off <= 29) return (float)__builtin_amdgcn_ubfe(lo, off, 3);
  const uint32_t hi = bit < 32 ? w.y : w.z;                    // the code straddles two words
  return (float)(__builtin_amdgcn_alignbit(hi, lo, off) & 7u);
}

// sum_i code_i a_i and sum_i a_i over the chunk's 32 codes
template <int WT>
__device__ __forceinline__ float2 lowbit_dots(const typename WTraits<WT>::chunk_t &w, const float *a) {
  float dq = 0.0f, dx = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 x = *reinterpret_cast<const float4 *>(a + 4 * q);
    const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float code;
      if constexpr (WT == M2_W_INT4G) code = lb4_code(w, 4 * q + j);
      else code = lb3_code(w, 4 * q + j);
      dq = fmaf(code, xv[j], dq);
      dx += xv[j];
    }
  }
  return make_float2(dq, dx);
}

// Per-chunk quantization parameters: int8 scale, or low-bit (scale, bias) of the chunk's group.
struct QScale { float s, m; };

template <int WT>
__device__ __forceinline__ QScale load_qscale(const void *srow, int c, int q_shift) {
  QScale r{1.0f, 0.0f};
  if constexpr (WT == M2_W_INT8G) {
    r.s = __half2float(static_cast<const __half *>(srow)[c >> q_shift]);
  } else if constexpr (WT == M2_W_INT4G || WT == M2_W_INT3G) {
    const __half2 sm = static_cast<const __half2 *>(srow)[c >> q_shift];
    r.s = __low2float(sm);
    r.m = __high2float(sm);
  }
  return r;
}

// acc += the chunk's contribution (one session)
template <int WT>
__device__ __forceinline__ float chunk_acc(const typename WTraits<WT>::chunk_t &w, const float *a, const QScale &q,
                                           float acc) {
  if constexpr (WT == M2_W_INT4G || WT == M2_W_INT3G) {
    const float2 d = lowbit_dots<WT>(w, a);
    return fmaf(q.s, d.x, fmaf(q.m, d.y, acc));
  } else if constexpr (WT == M2_W_INT8G) {
    return fmaf(q.s, chunk_dot<WT>(w, a), acc);
  } else {
    return acc + chunk_dot<WT>(w, a);
  }
}

// Scale columns of a row (int8: one fp16 per group; low-bit: one (scale, bias) pair).
template <int WT>
__device__ __forceinline__ const void *scale_row(const void *S, size_t row, int ngroups) {
  if constexpr (WT == M2_W_INT4G || WT == M2_W_INT3G) return static_cast<const __half2 *>(S) + row * ngroups;
  return static_cast<const __half *>(S) + row * ngroups;
}

enum { PRO_PLAIN = 0, PRO_NORM = 1 };
enum { EPI_INPROJ = 0, EPI_OUT = 1 };

struct GemvArgs {
  const void *W;          // [rows][K]
  const void *S;          // int8 scales [rows][K / q_group] (fp16), or low-bit (scale, bias) fp16 pairs
  int rows, K;
  int q_shift;            // log2(q_group / EPC): chunk index -> scale column (quantized types)
  float gamma;
  const float *act;       // [B][K]: x (in_proj) or v * norm_w (out_proj)
  int B, KT;              // sessions, activation K tile (tiled kernel)
  // RMSNorm prologue (out_proj)
  const float *ss;        // [B][n_partials]
  int ng, n_partials, n_norm;
  float eps;
  // in_proj epilogue
  float *zx;              // [B][zx_stride]
  int zx_stride, d_inner, conv_dim, d_conv;
  const float *conv_w, *conv_b, *dt_bias;
  float *conv_cache;      // [n_slots][d_conv-1][conv_dim]
  // out_proj epilogue
  float *y;               // [B][rows]
  const float *resid;     // [B][rows] or null
  const int32_t *slots;
  int n_slots;
};

// ---------------------------------------------------------------------------
struct SsdArgs {
  const float *zx;        // [B][zx_stride]: z raw | x|B|C raw (pre-conv) | dt (softplus'd)
  int zx_stride, d_inner, conv_dim, H, P, N, G, hpg;
  float *ssm;             // [n_slots][H][P][N]
  const float *conv_cache;// [n_slots][d_conv-1][conv_dim], read only (shifted by out_proj)
  const float *conv_w, *conv_b;
  int d_conv;
  const float *A_log, *D, *norm_w;
  float *vw;              // [B][d_inner]: v * norm_w
  float *ss;              // [B][n_partials]
  int prange, psplit, n_partials;
  const int32_t *slots;
  int n_slots;
};

// Per-row epilogue inputs, loaded when the row starts so that their latency
// overlaps the weight stream: dt bias (dt rows), residual (out_proj).
struct EpiIn {
  float bias;
  float resid;
  int slot;
  bool sok;
};

template <int EPI>
__device__ __forceinline__ EpiIn epilogue_prefetch(const GemvArgs &a, int row, int b) {
  EpiIn e;
  e.slot = a.slots ? a.slots[b] : b;
  e.sok = e.slot >= 0 && e.slot < a.n_slots;
  e.bias = 0.0f;
  e.resid = 0.0f;
  if (EPI == EPI_INPROJ) {
    if (row >= a.d_inner + a.conv_dim) e.bias = a.dt_bias[row - a.d_inner - a.conv_dim];
  } else if (a.resid) {
    e.resid = a.resid[(size_t)b * a.rows + row];
  }
  return e;
}

// The same inputs with every load unconditional (indices clamped, values selected after),
// for kernels that keep later loads in flight across the epilogue: a conditional load
// would make the compiler wait for all of them.
template <int EPI>
__device__ __forceinline__ EpiIn epilogue_load_all(const GemvArgs &a, int row, int b) {
  EpiIn e;
  const int32_t *sp = a.slots ? a.slots + b : reinterpret_cast<const int32_t *>(a.act);
  const int32_t sv = *sp;
  e.slot = a.slots ? sv : b;
  e.sok = e.slot >= 0 && e.slot < a.n_slots;
  e.bias = 0.0f;
  e.resid = 0.0f;
  if (EPI == EPI_INPROJ) {
    const int j = row - a.d_inner - a.conv_dim;
    const float bv = a.dt_bias[min(max(j, 0), a.rows - a.d_inner - a.conv_dim - 1)];
    e.bias = j >= 0 ? bv : 0.0f;
  } else {
    const float *rp = a.resid ? a.resid + (size_t)b * a.rows + row : a.act;
    const float rv = *rp;
    e.resid = a.resid ? rv : 0.0f;
  }
  return e;
}

// Per-row result -> outputs. in_proj: z and x|B|C raw (the causal conv is applied
// by the SSD kernel), softplus(dt + bias) for the dt rows. out_proj: gamma,
// residual add.
template <int EPI>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs &a, int row, int b, float val, const EpiIn &e) {
  val *= a.gamma;
  const float qnan = __builtin_nanf("");
  if (EPI == EPI_INPROJ) {
    float out = val;
    if (row >= a.d_inner + a.conv_dim) out = softplus(val + e.bias);
    a.zx[(size_t)b * a.zx_stride + row] = e.sok ? out : qnan;
  } else {
    a.y[(size_t)b * a.rows + row] = e.sok ? val + e.resid : qnan;
  }
}

// The conv cache after this step: the last d_conv-1 raw inputs, oldest first.
// Runs in the out_proj kernels, after every reader of the old cache (the SSD
// kernel) has finished. Elements (session, channel) strided over the grid.
__device__ __forceinline__ void conv_cache_shift(const GemvArgs &a, size_t gtid, size_t gthreads) {
  const size_t total = (size_t)a.B * a.conv_dim;
  for (size_t i = gtid; i < total; i += gthreads) {
    const int b = (int)(i / a.conv_dim), c = (int)(i - (size_t)b * a.conv_dim);
    const int slot = a.slots ? a.slots[b] : b;
    if (slot < 0 || slot >= a.n_slots) continue;
    float *cc = a.conv_cache + (size_t)slot * (a.d_conv - 1) * a.conv_dim + c;
    const float raw = a.zx[(size_t)b * a.zx_stride + a.d_inner + c];
    for (int k = 0; k + 1 < a.d_conv - 1; ++k) cc[(size_t)k * a.conv_dim] = cc[(size_t)(k + 1) * a.conv_dim];
    cc[(size_t)(a.d_conv - 2) * a.conv_dim] = raw;
  }
}

// RMS factors r[bb][j] = 1/sqrt(mean_j(v^2) + eps) for sessions b0 .. b0+nb-1,
// summing each group's partials in a fixed order. Uses LDS part[n_partials].
__device__ __forceinline__ void rms_factors(const GemvArgs &a, int b0, int nb, float *part, float *rn,
                                            int tid, int nthreads) {
  const int per = a.n_partials / a.n_norm;
  for (int bb = 0; bb < nb; ++bb) {
    for (int p = tid; p < a.n_partials; p += nthreads) part[p] = a.ss[(size_t)(b0 + bb) * a.n_partials + p];
    __syncthreads();
    for (int j = tid; j < a.n_norm; j += nthreads) {
      float s = 0.0f;
      for (int q = 0; q < per; ++q) s += part[j * per + q];
      rn[bb * a.n_norm + j] = 1.0f / sqrtf(s / (float)a.ng + a.eps);
    }
    __syncthreads();
  }
}

// out_proj activation staging in one memory trip: each thread loads its float4s
// of v * norm_w and one sum-of-squares partial per session together, the RMS
// factors are formed in LDS, then the float4s are scaled by their group's factor.
// LDS: act [BT][K] | part [n_partials] | rn [BT][n_norm]. K/4 <= TPB * kNormF4PerThread.
template <int BT, int TPB>
__device__ __forceinline__ void stage_norm_act(const GemvArgs &a, float *lds, int tid) {
  const int K = a.K;
  const int nb = min(BT, a.B);
  float *act_s = lds;
  float *part = lds + BT * K;
  float *rn = part + a.n_partials;
  constexpr int MAXF = kNormF4PerThread;
  const int nf = K / 4;
  float pv[BT];
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    pv[bb] = (bb < nb && tid < a.n_partials) ? a.ss[(size_t)bb * a.n_partials + tid] : 0.0f;
#pragma unroll
    for (int i = 0; i < MAXF; ++i) {
      const int f = tid + TPB * i;
      if (f < nf)
        reinterpret_cast<float4 *>(act_s + bb * K)[f] =
            bb < nb ? reinterpret_cast<const float4 *>(a.act + (size_t)bb * K)[f] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  const int per = a.n_partials / a.n_norm;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    if (tid < a.n_partials) part[tid] = pv[bb];
    __syncthreads();
    if (tid < a.n_norm) {
      float sum = 0.0f;
      for (int q = 0; q < per; ++q) sum += part[tid * per + q];
      rn[bb * a.n_norm + tid] = 1.0f / sqrtf(sum / (float)a.ng + a.eps);
    }
    __syncthreads();
  }
  // each thread rescales the float4s it staged
  const int ng4 = a.ng / 4;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb)
#pragma unroll
    for (int i = 0; i < MAXF; ++i) {
      const int f = tid + TPB * i;
      if (f < nf) {
        const float r = bb < nb ? rn[bb * a.n_norm + f / ng4] : 0.0f;
        float4 *p4 = reinterpret_cast<float4 *>(act_s + bb * K) + f;
        const float4 x = *p4;
        *p4 = make_float4(x.x * r, x.y * r, x.z * r, x.w * r);
      }
    }
}

// ---------------------------------------------------------------------------
// gemv_wave: one wave per row, whole-K activations of BT (= batch) sessions in LDS.
// LDS: act [BT][K] | part [n_partials] | rn [BT][n_norm]
template <int WT, int BT, int TPB, int U, int NT, int PRO, int EPI>
__global__ __launch_bounds__(TPB) void gemv_wave_kernel(GemvArgs a) {
  extern __shared__ float lds[];
  constexpr int WPB = TPB / 64;
  constexpr int EPC = WTraits<WT>::EPC;
  constexpr int CB = WTraits<WT>::CB;
  using chunk_t = typename WTraits<WT>::chunk_t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x * WPB + (tid >> 6);
  const bool row_ok = row < a.rows;
  const int nb = min(BT, a.B);
  const int K = a.K;
  const int NC = K / EPC;
  const char *wr = static_cast<const char *>(a.W) + (size_t)(row_ok ? row : 0) * NC * CB;
  const void *srow = scale_row<WT>(a.S, (size_t)(row_ok ? row : 0), NC >> a.q_shift);

  // weights do not depend on the activations: put the first U loads in flight first
  chunk_t w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = lane + 64 * u;
    w[u] = (row_ok && c < NC) ? load_chunk<WT, NT>(wr, c) : chunk_t{};
  }
  EpiIn epi{};
  if (row_ok && lane < nb) epi = epilogue_prefetch<EPI>(a, row, lane);

  float *act_s = lds;
  if (PRO == PRO_NORM) {
    stage_norm_act<BT, TPB>(a, lds, tid);
  } else {
#pragma unroll
    for (int bb = 0; bb < BT; ++bb)
      for (int i = tid * 4; i < K; i += TPB * 4) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (bb < nb) v = *reinterpret_cast<const float4 *>(a.act + (size_t)bb * K + i);
        *reinterpret_cast<float4 *>(act_s + bb * K + i) = v;
      }
  }
  __syncthreads();

  float acc[BT];
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) acc[bb] = 0.0f;
  if (row_ok) {
    for (int cb = lane;;) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb + 64 * u;
        if (c < NC) {
          const QScale qs = load_qscale<WT>(srow, c, a.q_shift);
#pragma unroll
          for (int bb = 0; bb < BT; ++bb) acc[bb] = chunk_acc<WT>(w[u], act_s + bb * K + c * EPC, qs, acc[bb]);
        }
      }
      cb += 64 * U;
      if (cb >= NC) break;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb + 64 * u;
        w[u] = c < NC ? load_chunk<WT, NT>(wr, c) : chunk_t{};
      }
    }
  }
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) acc[bb] = group_reduce<64>(acc[bb]);
  if (EPI == EPI_OUT && a.conv_cache)
    conv_cache_shift(a, (size_t)blockIdx.x * TPB + tid, (size_t)gridDim.x * TPB);
  if (!row_ok || lane >= nb) return;
  float val = 0.0f;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb)
    if (lane == bb) val = acc[bb];
  gemv_epilogue<EPI>(a, row, lane, val, epi);
}

// ---------------------------------------------------------------------------
// gemv_lowbit: 4- and 3-bit codes, BT (1 or 2) sessions. A wave takes R rows and walks
// their 32-code chunks together, lane l taking chunk columns l, l + 64, ...: one read of
// an activation chunk from LDS serves the R rows, and each chunk's (scale, bias) pair is
// loaded with the chunk. The activations are staged with all their loads issued before
// any LDS write (the weight loads go out first), then the sum of every 32-element chunk
// of each session is formed once, for the group bias: w = s q + m gives
// sum_k w_k x_k = s sum_k q_k x_k + m sum_k x_k.
// LDS: act [BT][K] | xsum [BT][K/32] (| part [BT][n_partials] | rn [BT][n_norm], out_proj)
constexpr int kLbThreads = 512;

template <int WT, int BT, int PRO>
__device__ __forceinline__ void lb_stage(const GemvArgs &a, float *lds, int tid) {
  constexpr int TPB = kLbThreads;
  constexpr int MAXF = kNormF4PerThread;
  const int K = a.K, nf = K / 4, nb = min(BT, a.B);
  f32x4 v[BT][MAXF];
  float pv[BT];
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    const int sb = min(bb, nb - 1);
    const f32x4 *src = reinterpret_cast<const f32x4 *>(a.act + (size_t)sb * K);
#pragma unroll
    for (int i = 0; i < MAXF; ++i) v[bb][i] = src[min(tid + TPB * i, nf - 1)];   // clamped index
    pv[bb] = PRO != PRO_NORM ? 0.0f : a.ss[(size_t)sb * a.n_partials + min(tid, a.n_partials - 1)];
  }
  const int KP = lds_padded(K);
  float *acts = lds;
  if (PRO == PRO_NORM) {
    float *part = lds + BT * (KP + K / 32);
    float *rn = part + BT * a.n_partials;
    if (tid < a.n_partials) {
#pragma unroll
      for (int bb = 0; bb < BT; ++bb) part[bb * a.n_partials + tid] = pv[bb];
    }
    __syncthreads();
    const int per = a.n_partials / a.n_norm;
    for (int j = tid; j < BT * a.n_norm; j += TPB) {
      const int bb = j / a.n_norm, q = j - bb * a.n_norm;
      float sum = 0.0f;
      for (int k = 0; k < per; ++k) sum += part[bb * a.n_partials + q * per + k];
      rn[j] = 1.0f / sqrtf(sum / (float)a.ng + a.eps);
    }
    __syncthreads();
    const int ng4 = a.ng / 4;
#pragma unroll
    for (int bb = 0; bb < BT; ++bb)
#pragma unroll
      for (int i = 0; i < MAXF; ++i) {
        const int f = min(tid + TPB * i, nf - 1);    // past the row: rewrites the last float4
        *reinterpret_cast<f32x4 *>(acts + bb * KP + lds_pad(4 * f)) = v[bb][i] * rn[bb * a.n_norm + f / ng4];
      }
  } else {
#pragma unroll
    for (int bb = 0; bb < BT; ++bb)
#pragma unroll
      for (int i = 0; i < MAXF; ++i) *reinterpret_cast<f32x4 *>(acts + bb * KP + lds_pad(4 * min(tid + TPB * i, nf - 1))) = v[bb][i];
  }
  __syncthreads();
  // chunk sums, each in a fixed order
  float *xsum = lds + BT * KP;
  const int nc = K / 32;
  for (int j = tid; j < BT * nc; j += TPB) {
    const int bb = j / nc, c = j - bb * nc;
    const f32x4 *p = reinterpret_cast<const f32x4 *>(acts + bb * KP + lds_pad(32 * c));
    f32x4 s4 = p[0];
#pragma unroll
    for (int q = 1; q < 8; ++q) s4 += p[q];
    xsum[j] = (s4.x + s4.y) + (s4.z + s4.w);
  }
  __syncthreads();
}

// sum_i code_i x_i over one chunk of 32 codes, x from LDS; R rows share each x read
template <int WT, int R>
__device__ __forceinline__ void lb_dots(const typename WTraits<WT>::chunk_t (&w)[R], const float *x, float (&dq)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) dq[r] = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 xv = *reinterpret_cast<const float4 *>(x + 4 * q);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float c0, c1, c2, c3;
      if constexpr (WT == M2_W_INT4G) {
        // word q/2 holds codes 8(q/2) .. +7; even codes in the low nibbles
        const uint32_t word = (q >> 1) == 0 ? w[r].x : (q >> 1) == 1 ? w[r].y : (q >> 1) == 2 ? w[r].z : w[r].w;
        const uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
        const int sh = (q & 1) * 16;
        c0 = (float)((lo >> sh) & 0xffu);
        c1 = (float)((hi >> sh) & 0xffu);
        c2 = (float)((lo >> (sh + 8)) & 0xffu);
        c3 = (float)((hi >> (sh + 8)) & 0xffu);
      } else {
        c0 = lb3_code(w[r], 4 * q);
        c1 = lb3_code(w[r], 4 * q + 1);
        c2 = lb3_code(w[r], 4 * q + 2);
        c3 = lb3_code(w[r], 4 * q + 3);
      }
      dq[r] = fmaf(c0, xv.x, dq[r]);
      dq[r] = fmaf(c1, xv.y, dq[r]);
      dq[r] = fmaf(c2, xv.z, dq[r]);
      dq[r] = fmaf(c3, xv.w, dq[r]);
    }
  }
}

// A persistent grid: wave w takes row groups (R rows) w, w + W, w + 2W, ... (W waves in
// all); every chunk column of a group is requested at once (U columns per lane cover the
// row, U * 64 >= K / 32), and the next group's loads are issued before the current group
// is multiplied, so two groups per wave are in flight. Loads are unconditional (group
// and column indices clamped), so that waiting for one group never waits for the next.
template <int WT, int BT, int R, int U, int NT, int PRO, int EPI>
__global__ __launch_bounds__(kLbThreads) void gemv_lowbit_kernel(GemvArgs a) {
  extern __shared__ float lds[];
  constexpr int WPB = kLbThreads / 64;
  constexpr int CB = WTraits<WT>::CB;
  using chunk_t = typename WTraits<WT>::chunk_t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, NC = K / 32, nb = min(BT, a.B);
  const int ngroups = (a.rows + R - 1) / R;
  const int gstride = gridDim.x * WPB;
  const int g0 = blockIdx.x * WPB + wave;

  struct Set {
    chunk_t w[U][R];
    __half2 sm[U][R];
    EpiIn epi[R];
  };
  auto load_group = [&](int g, Set &st) {
    g = min(g, ngroups - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(g * R + r, a.rows - 1);
      st.epi[r] = epilogue_load_all<EPI>(a, row, min(lane, nb - 1));
      const char *wr = static_cast<const char *>(a.W) + (size_t)row * NC * CB;
      const __half2 *sr = static_cast<const __half2 *>(a.S) + (size_t)row * (NC >> a.q_shift);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(lane + 64 * u, NC - 1);   // columns past the row are not used
        st.w[u][r] = load_chunk<WT, NT>(wr, c);
        st.sm[u][r] = sr[c >> a.q_shift];
      }
    }
  };
  Set sa, sb;
  load_group(g0, sa);
  lb_stage<WT, BT, PRO>(a, lds, tid);
  const int KP = lds_padded(K);
  const float *act_s = lds;
  const float *xsum = lds + BT * KP;

  auto run_group = [&](int g, const Set &st) {
    float acc[R][BT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int bb = 0; bb < BT; ++bb) acc[r][bb] = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = lane + 64 * u;
      if (c < NC) {
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) {
          float dq[R];
          lb_dots<WT, R>(st.w[u], act_s + bb * KP + lds_pad(32 * c), dq);
          const float xs = xsum[bb * NC + c];
#pragma unroll
          for (int r = 0; r < R; ++r)
            acc[r][bb] = fmaf(__low2float(st.sm[u][r]), dq[r], fmaf(__high2float(st.sm[u][r]), xs, acc[r][bb]));
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int bb = 0; bb < BT; ++bb)
        acc[r][bb] = group_reduce<64>(acc[r][bb]);
    if (lane < nb) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = g * R + r;
        if (row < a.rows) {
          float val = 0.0f;
#pragma unroll
          for (int bb = 0; bb < BT; ++bb)
            if (lane == bb) val = acc[r][bb];
          gemv_epilogue<EPI>(a, row, lane, val, st.epi[r]);
        }
      }
    }
  };
  // two groups per iteration so that the register sets keep static names
  for (int g = g0; g < ngroups; g += 2 * gstride) {
    load_group(g + gstride, sb);
    run_group(g, sa);
    if (g + gstride >= ngroups) break;
    load_group(g + 2 * gstride, sa);
    run_group(g + gstride, sb);
  }
  if (EPI == EPI_OUT && a.conv_cache)
    conv_cache_shift(a, (size_t)blockIdx.x * kLbThreads + tid, (size_t)gridDim.x * kLbThreads);
}

// ---------------------------------------------------------------------------
// gemv_tiled: one workgroup computes RPW = 16/KS rows for a tile of BT sessions.
// Threads form 16 groups of 16 lanes; group (ks, r) covers row r over the ks-th
// share of each K tile, lanes striding over 16-byte chunks, U chunks in flight.
// LDS: act [BT][KT] | part [n_partials] | rn [BT][n_norm] | red [16][BT]
template <int WT, int BT, int KS, int PRO, int EPI, int U>
__global__ __launch_bounds__(kThreads) void gemv_tiled_kernel(GemvArgs a) {
  extern __shared__ float lds[];
  constexpr int RPW = 16 / KS;
  constexpr int EPC = WTraits<WT>::EPC;
  constexpr int CB = WTraits<WT>::CB;
  using chunk_t = typename WTraits<WT>::chunk_t;
  const int tid = threadIdx.x, lane = tid & 15, gid = tid >> 4;
  const int ks = gid / RPW, rl = gid % RPW;
  const int row = blockIdx.x * RPW + rl;
  const bool row_ok = row < a.rows;
  const int b0 = blockIdx.y * BT;
  const int nb = min(BT, a.B - b0);
  float *act_s = lds;
  float *part = lds + BT * a.KT;
  float *rn = part + (PRO == PRO_NORM ? a.n_partials : 0);
  float *red_s = rn + (PRO == PRO_NORM ? BT * a.n_norm : 0);

  if (PRO == PRO_NORM) rms_factors(a, b0, nb, part, rn, tid, kThreads);

  float acc[BT];
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) acc[bb] = 0.0f;

  const void *srow = scale_row<WT>(a.S, (size_t)(row_ok ? row : 0), (a.K / EPC) >> a.q_shift);
  for (int kt = 0; kt < a.K; kt += a.KT) {
    const int klen = min(a.KT, a.K - kt);
    // stage act[b0 .. b0+BT)[kt .. kt+klen) (times the RMS factor for out_proj); klen % 4 == 0
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) {
      if (PRO == PRO_NORM) {
        const int j0 = kt / a.ng, j1 = (kt + klen - 1) / a.ng;
        for (int j = j0; j <= j1; ++j) {
          const int lo = max(kt, j * a.ng), hi = min(kt + klen, (j + 1) * a.ng);
          const float r = bb < nb ? rn[bb * a.n_norm + j] : 0.0f;
          for (int i = lo + tid * 4; i < hi; i += kThreads * 4) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (bb < nb) v = *reinterpret_cast<const float4 *>(a.act + (size_t)(b0 + bb) * a.K + i);
            *reinterpret_cast<float4 *>(act_s + bb * a.KT + (i - kt)) = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
          }
        }
      } else {
        for (int i = tid * 4; i < klen; i += kThreads * 4) {
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (bb < nb) v = *reinterpret_cast<const float4 *>(a.act + (size_t)(b0 + bb) * a.K + kt + i);
          *reinterpret_cast<float4 *>(act_s + bb * a.KT + i) = v;
        }
      }
    }
    __syncthreads();
    if (row_ok) {
      const int nch = klen / EPC;
      const int per = (nch + KS - 1) / KS;
      const int c0 = ks * per, c1 = min(nch, c0 + per);
      const int cbase = kt / EPC;
      const char *wrow = static_cast<const char *>(a.W) + ((size_t)row * (a.K / EPC) + cbase) * CB;
      for (int cb = c0 + lane; cb < c1; cb += 16 * U) {
        chunk_t wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + 16 * u;
          wv[u] = c < c1 ? load_chunk<WT, 0>(wrow, c) : chunk_t{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + 16 * u;
          if (c < c1) {
            const QScale qs = load_qscale<WT>(srow, cbase + c, a.q_shift);
#pragma unroll
            for (int bb = 0; bb < BT; ++bb) acc[bb] = chunk_acc<WT>(wv[u], act_s + bb * a.KT + c * EPC, qs, acc[bb]);
          }
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int bb = 0; bb < BT; ++bb) acc[bb] = group_reduce<16>(acc[bb]);
  float val = 0.0f;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb)
    if (lane == bb) val = acc[bb];
  if (KS > 1) {
    if (lane < BT) red_s[gid * BT + lane] = val;
    __syncthreads();
    if (ks == 0 && lane < BT) {
      float s = 0.0f;
      for (int q = 0; q < KS; ++q) s += red_s[(q * RPW + rl) * BT + lane];
      val = s;
    }
  }
  if (EPI == EPI_OUT && a.conv_cache && blockIdx.y == 0)
    conv_cache_shift(a, (size_t)blockIdx.x * kThreads + tid, (size_t)gridDim.x * kThreads);
  if (ks != 0 || !row_ok || lane >= nb) return;
  gemv_epilogue<EPI>(a, row, b0 + lane, val, epilogue_prefetch<EPI>(a, row, b0 + lane));
}

// ---------------------------------------------------------------------------

// The SSM state is read once and written once per step: stream it (nontemporal),
// so that it neither evicts nor leaves dirty lines for the weight stream that
// follows.
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float4 *p) {
  const f32x4v t = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st_stream(float4 *p, const float4 &v) {
  const f32x4v t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4v *>(p));
}

// One SSD work item = (session b, head h, rows [ps*prange, (ps+1)*prange)),
// done by the NW waves of a workgroup. A state row (N floats) is read by N/4
// lanes as float4; every slice of the tile is loaded before any is used,
// updated in registers and written once. wsum: LDS float[NW]. Must be called by
// every thread of the workgroup.
// Causal conv + SiLU of 4 consecutive conv channels c0..c0+3 of one session
// (cache slot `slot`): bias + sum_k w[c][k] in(t-K+1+k), the last K-1 inputs from
// the cache, the newest the raw in_proj output.
__device__ __forceinline__ float4 conv4(const SsdArgs &a, const float *zb, int slot, int c0) {
  const float4 raw = *reinterpret_cast<const float4 *>(zb + a.d_inner + c0);
  const float4 bias = *reinterpret_cast<const float4 *>(a.conv_b + c0);
  const float *cache = a.conv_cache + (size_t)slot * (a.d_conv - 1) * a.conv_dim + c0;
  const float r[4] = {raw.x, raw.y, raw.z, raw.w};
  float acc[4] = {bias.x, bias.y, bias.z, bias.w};
  if (a.d_conv == 4) {
    const float4 *w4 = reinterpret_cast<const float4 *>(a.conv_w + (size_t)c0 * 4);
    const float4 w[4] = {w4[0], w4[1], w4[2], w4[3]};
    const float4 h0 = *reinterpret_cast<const float4 *>(cache);
    const float4 h1 = *reinterpret_cast<const float4 *>(cache + a.conv_dim);
    const float4 h2 = *reinterpret_cast<const float4 *>(cache + 2 * (size_t)a.conv_dim);
    const float x0[4] = {h0.x, h0.y, h0.z, h0.w}, x1[4] = {h1.x, h1.y, h1.z, h1.w}, x2[4] = {h2.x, h2.y, h2.z, h2.w};
    const float wt[4][4] = {{w[0].x, w[0].y, w[0].z, w[0].w}, {w[1].x, w[1].y, w[1].z, w[1].w},
                            {w[2].x, w[2].y, w[2].z, w[2].w}, {w[3].x, w[3].y, w[3].z, w[3].w}};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = fmaf(wt[e][0], x0[e], acc[e]);
      acc[e] = fmaf(wt[e][1], x1[e], acc[e]);
      acc[e] = fmaf(wt[e][2], x2[e], acc[e]);
      acc[e] = fmaf(wt[e][3], r[e], acc[e]);
    }
  } else {
    const float *w = a.conv_w + (size_t)c0 * a.d_conv;
    for (int k = 0; k < a.d_conv - 1; ++k) {
      const float4 hv = *reinterpret_cast<const float4 *>(cache + (size_t)k * a.conv_dim);
      const float hh[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(w[e * a.d_conv + k], hh[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(w[e * a.d_conv + a.d_conv - 1], r[e], acc[e]);
  }
  return make_float4(silu(acc[0]), silu(acc[1]), silu(acc[2]), silu(acc[3]));
}

template <int NW, int MAXI>
__device__ __forceinline__ void ssd_item(const SsdArgs &a, int h, int ps, int b, int wave, int lane,
                                         float *wsum, float *cx) {
  const int g = h / a.hpg;
  const int lpr = a.N >> 2;                 // lanes per state row
  const int rpi = 64 / lpr;                 // rows per wave instruction
  const int n_inst = (a.prange + rpi - 1) / rpi;
  const int r_in = lane / lpr, q = lane - r_in * lpr;
  const float *zb = a.zx + (size_t)b * a.zx_stride;
  const int slot = a.slots ? a.slots[b] : b;
  const bool sok = slot >= 0 && slot < a.n_slots;
  float4 *S = reinterpret_cast<float4 *>(a.ssm + ((size_t)(sok ? slot : 0) * a.H + h) * a.P * a.N);

  float4 st[MAXI];
  int prow[MAXI];
  float zg[MAXI], nw[MAXI];                 // gate input and norm weight of the row (lane q == 0)
#pragma unroll
  for (int k = 0; k < MAXI; ++k) {
    const int i = wave + NW * k;
    const int pl = i * rpi + r_in;
    prow[k] = (i < n_inst && pl < a.prange) ? ps * a.prange + pl : -1;
    st[k] = (sok && prow[k] >= 0) ? ld_stream(S + (size_t)prow[k] * lpr + q) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // the epilogue's loads go out with the state's, not after the readout
#pragma unroll
  for (int k = 0; k < MAXI; ++k) {
    const bool need = q == 0 && prow[k] >= 0;
    zg[k] = need ? zb[h * a.P + prow[k]] : 0.0f;
    nw[k] = need ? a.norm_w[h * a.P + prow[k]] : 0.0f;
  }
  const float dt = zb[a.d_inner + a.conv_dim + h];
  const float dA = expf(-expf(a.A_log[h]) * dt);
  const float Dh = a.D[h];
  // conv outputs, each channel once per workgroup: B and C of the group and the
  // item's x rows, one float4 of channels per thread, through LDS (cx = [B | C | x])
  {
    const int n4 = a.N / 4;
    for (int t = wave * 64 + lane; t < 2 * n4 + a.prange / 4; t += NW * 64) {
      const int c0 = t < n4 ? a.d_inner + g * a.N + 4 * t
                   : t < 2 * n4 ? a.d_inner + (a.G + g) * a.N + 4 * (t - n4)
                   : h * a.P + ps * a.prange + 4 * (t - 2 * n4);
      reinterpret_cast<float4 *>(cx)[t] = conv4(a, zb, sok ? slot : 0, c0);
    }
    __syncthreads();
  }
  const float4 Bq = reinterpret_cast<const float4 *>(cx)[q];
  const float4 Cq = reinterpret_cast<const float4 *>(cx + a.N)[q];
  const float *xs = cx + 2 * a.N;
  float ssacc = 0.0f;
#pragma unroll
  for (int k = 0; k < MAXI; ++k) {
    if (wave + NW * k >= n_inst) break;     // uniform across the wave
    const int p = prow[k];
    const float xp = p >= 0 ? xs[p - ps * a.prange] : 0.0f;
    const float dtx = dt * xp;
    float4 sv = st[k];
    sv.x = fmaf(dA, sv.x, dtx * Bq.x);
    sv.y = fmaf(dA, sv.y, dtx * Bq.y);
    sv.z = fmaf(dA, sv.z, dtx * Bq.z);
    sv.w = fmaf(dA, sv.w, dtx * Bq.w);
    st[k] = sv;
    float r = sv.x * Cq.x;
    r = fmaf(sv.y, Cq.y, r);
    r = fmaf(sv.z, Cq.z, r);
    r = fmaf(sv.w, Cq.w, r);
    r = group_sum_rt(r, lpr);
    if (q == 0 && p >= 0) {
      const int ch = h * a.P + p;
      const float yv = fmaf(Dh, xp, r);
      float vv = yv * silu(zg[k]);
      if (!sok) vv = __builtin_nanf("");
      a.vw[(size_t)b * a.d_inner + ch] = vv * nw[k];
      ssacc = fmaf(vv, vv, ssacc);
    }
  }
  if (sok) {
#pragma unroll
    for (int k = 0; k < MAXI; ++k)
      if (prow[k] >= 0) st_stream(S + (size_t)prow[k] * lpr + q, st[k]);
  }
  // sum of squares of this item's rows, in a fixed order
  ssacc = group_reduce<64>(ssacc);
  if (lane == 0) wsum[wave] = ssacc;
  __syncthreads();
  if (wave == 0 && lane == 0) {
    float t = 0.0f;
    for (int i = 0; i < NW; ++i) t += wsum[i];
    a.ss[(size_t)b * a.n_partials + (h * a.P + ps * a.prange) / a.prange] = t;
  }
  __syncthreads();
}

// NW waves per item, up to MAXI state slices per wave (NW * MAXI >= the item's
// wave instructions).
template <int NW, int MAXI>
__global__ __launch_bounds__(NW * 64) void ssd_step_kernel(SsdArgs a) {
  __shared__ float wsum[NW];
  __shared__ float cx[2 * 256 + 32];   // conv outputs: B [N] | C [N] | x rows [prange]
  const int h = blockIdx.x / a.psplit, ps = blockIdx.x - h * a.psplit;
  ssd_item<NW, MAXI>(a, h, ps, blockIdx.y, threadIdx.x >> 6, threadIdx.x & 63, wsum, cx);
}


// ---------------------------------------------------------------------------
// gemv_mfma: batch 3..32 with bf16 weights, or int8 weights with q_group 128 or
// 256. A workgroup of 8 waves owns 128 rows (16 per wave) over one K chunk
// (blockIdx.y) of whole 256-wide tiles and writes its partial sums
// part[chunk][b][row]. Per 32-wide k-step: A = 16 weight rows x 32 k straight
// from HBM (one 16- or 8-byte load per lane and step), B = 32 k x 16 sessions
// from LDS as bf16 hi + lo (an fp32 value is hi + lo to 2^-16 relative; bf16 and
// int8 weights are exact in bf16), two 16x16x32 bf16 MFMAs per product. The tiles
// are software-pipelined: while one tile's MFMAs run, the next tile's weights are
// in flight into a second register set and its activations into registers, which
// are then converted into the second LDS buffer; one barrier per tile. With RMS
// (out_proj) the workgroup first forms the RMS factors of the norm groups its
// chunk covers from the sums of squares (fixed order) and scales the activations
// by them while staging. gemv_mfma_reduce sums the chunks in a fixed order and
// applies the row epilogue, so results do not depend on scheduling.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kMKT = 256;          // K tile
constexpr int kMLD = kMKT + 8;     // LDS row stride (bf16)
constexpr int kMRows = 128;        // rows per workgroup (8 waves x 16)

struct MfmaArgs {
  const void *W;
  const __half *S;
  int rows, K, q_group, kchunk;
  const float *act;                // [B][K]
  int B;
  // RMS prologue (out_proj): act[b][k] *= 1/sqrt(sum_j ss[b][g*per + j] / ng + eps), g = k / ng
  const float *ss;
  int n_partials, n_norm, ng;
  float eps;
  float *part;                     // [KS][B][rows]
};

// Raw weights of one tile for one lane: 8 k-steps of 8 values.
template <int WT> struct MRaw;
template <> struct MRaw<M2_W_BF16> { bf16x8 v[8]; };
template <> struct MRaw<M2_W_INT8G> { uint2 v[8]; };

template <int WT>
__device__ __forceinline__ void mfma_load_w(const MfmaArgs &a, int arow, int kt, int klen, int kq, MRaw<WT> &w) {
  const bool arow_ok = arow < a.rows;
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const bool ok = arow_ok && 32 * st + kq < klen;
    const size_t off = (size_t)arow * a.K + kt + 32 * st + kq;
    if constexpr (WT == M2_W_BF16)
      w.v[st] = ok ? *reinterpret_cast<const bf16x8 *>(static_cast<const unsigned short *>(a.W) + off) : bf16x8{};
    else
      w.v[st] = ok ? *reinterpret_cast<const uint2 *>(static_cast<const int8_t *>(a.W) + off) : make_uint2(0u, 0u);
  }
}

// int8 scales of the tile's q_group groups (at most 2) for this lane's 4 C rows.
__device__ __forceinline__ void mfma_load_s(const MfmaArgs &a, int rbase, int lane, int kt, float (&sc)[2][4]) {
  const int ngrp = a.K / a.q_group;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int g = (kt + q * a.q_group) / a.q_group;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = rbase + (lane >> 4) * 4 + r;
      sc[q][r] = (rr < a.rows && g < ngrp && q * a.q_group < kMKT) ? __half2float(a.S[(size_t)rr * ngrp + g]) : 0.0f;
    }
  }
}

template <int WT> __device__ __forceinline__ bf16x8 mfma_a(const MRaw<WT> &w, int st);
template <> __device__ __forceinline__ bf16x8 mfma_a<M2_W_BF16>(const MRaw<M2_W_BF16> &w, int st) { return w.v[st]; }
// int8 -> bf16 is exact; the conversions vectorise to byte-select converts and packed
// bf16 converts (1.5 instructions per value).
template <> __device__ __forceinline__ bf16x8 mfma_a<M2_W_INT8G>(const MRaw<M2_W_INT8G> &w, int st) {
  f32x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const unsigned wd = e < 4 ? w.v[st].x : w.v[st].y;
    f[e] = (float)((int32_t)(wd << (24 - 8 * (e & 3))) >> 24);
  }
  return __builtin_convertvector(f, bf16x8);
}

// Activations of one tile (NBT*16 sessions x 256 k, zero-filled) into registers.
template <int NBT>
__device__ __forceinline__ void mfma_load_x(const MfmaArgs &a, int kt, int klen, int tid, float4 (&xv)[NBT * 2]) {
#pragma unroll
  for (int q = 0; q < NBT * 2; ++q) {
    const int i = tid + 512 * q;
    const int b = i / (kMKT / 4), k4 = (i - b * (kMKT / 4)) * 4;
    xv[q] = (b < a.B && k4 < klen) ? *reinterpret_cast<const float4 *>(a.act + (size_t)b * a.K + kt + k4)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ... scaled by the RMS factors (RMS) and stored as bf16 hi / lo.
template <int NBT, bool RMS>
__device__ __forceinline__ void mfma_store_x(const MfmaArgs &a, int kt, int tid, const float4 (&xv)[NBT * 2],
                                             unsigned short *xh, unsigned short *xl, const float *rn_s, int g0,
                                             int ngc) {
#pragma unroll
  for (int q = 0; q < NBT * 2; ++q) {
    const int i = tid + 512 * q;
    const int b = i / (kMKT / 4), k4 = (i - b * (kMKT / 4)) * 4;
    f32x4 vv = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
    if (RMS) {
      const float r = b < a.B ? rn_s[b * ngc + (kt + k4) / a.ng - g0] : 0.0f;
      vv *= r;
    }
    // hi = bf16(v) and lo = bf16(v - hi), both rounded to nearest even
    const bf16x4 h = __builtin_convertvector(vv, bf16x4);
    const bf16x4 l = __builtin_convertvector(vv - __builtin_convertvector(h, f32x4), bf16x4);
    *reinterpret_cast<bf16x4 *>(&xh[b * kMLD + k4]) = h;
    *reinterpret_cast<bf16x4 *>(&xl[b * kMLD + k4]) = l;
  }
}

// The MFMAs of one tile; each k-step's weight registers are refilled with the same
// k-step of the next tile (kn < k_end) as soon as its MFMAs are issued, so 8 loads
// per lane stay in flight without a second register set.
template <int WT, int NBT>
__device__ __forceinline__ void mfma_tile(const MfmaArgs &a, MRaw<WT> &w, const float (&sc)[2][4], int klen,
                                          int lane, int kq, const unsigned short *xh, const unsigned short *xl,
                                          f32x4 (&acc)[NBT], int arow, int kn, int k_end) {
  const bool arow_ok = arow < a.rows;
  const int nlen = min(kMKT, k_end - kn);
  auto refill = [&](int st) {
    if (kn < k_end) {
      const bool ok = arow_ok && 32 * st + kq < nlen;
      const size_t off = (size_t)arow * a.K + kn + 32 * st + kq;
      if constexpr (WT == M2_W_BF16)
        w.v[st] = ok ? *reinterpret_cast<const bf16x8 *>(static_cast<const unsigned short *>(a.W) + off) : bf16x8{};
      else
        w.v[st] = ok ? *reinterpret_cast<const uint2 *>(static_cast<const int8_t *>(a.W) + off) : make_uint2(0u, 0u);
    }
  };
  if (WT == M2_W_BF16) {
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (32 * st < klen) {
        const bf16x8 av = mfma_a<WT>(w, st);
#pragma unroll
        for (int j = 0; j < NBT; ++j) {
          const int b = 16 * j + (lane & 15);
          const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&xh[b * kMLD + 32 * st + kq]);
          const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&xl[b * kMLD + 32 * st + kq]);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, acc[j], 0, 0, 0);
        }
      }
      refill(st);
    }
  } else {
    // one scale group = q_group / 32 k-steps (4 or 8): its products gathered, then scaled
    const int spg = a.q_group / 32;
    f32x4 gacc[NBT];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (32 * st < klen) {
        if (st % spg == 0) {
#pragma unroll
          for (int j = 0; j < NBT; ++j) gacc[j] = f32x4{};
        }
        const bf16x8 av = mfma_a<WT>(w, st);
#pragma unroll
        for (int j = 0; j < NBT; ++j) {
          const int b = 16 * j + (lane & 15);
          const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&xh[b * kMLD + 32 * st + kq]);
          const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&xl[b * kMLD + 32 * st + kq]);
          gacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, gacc[j], 0, 0, 0);
          gacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, gacc[j], 0, 0, 0);
        }
        if (st % spg == spg - 1 || 32 * (st + 1) >= klen) {
          const int q = st / spg;
#pragma unroll
          for (int j = 0; j < NBT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(q == 0 ? sc[0][r] : sc[1][r], gacc[j][r], acc[j][r]);
        }
      }
      refill(st);
    }
  }
}

template <int WT, int NBT, bool RMS>
__global__ __launch_bounds__(512) void gemv_mfma_kernel(MfmaArgs a) {
  extern __shared__ unsigned short xs[];            // [2 buffers][hi, lo][NBT*16][kMLD], then rn
  constexpr int XB = NBT * 16 * kMLD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rbase = blockIdx.x * kMRows + wave * 16;
  const int arow = rbase + (lane & 15);             // A-operand row of this lane
  const int k_begin = blockIdx.y * a.kchunk, k_end = min(a.K, k_begin + a.kchunk);
  const int kq = (lane >> 4) * 8;                   // this lane's 8 k within a 32-wide step
  float *rn_s = reinterpret_cast<float *>(xs + 4 * XB);
  const int g0 = RMS ? k_begin / a.ng : 0;
  const int ngc = RMS ? (k_end - 1) / a.ng - g0 + 1 : 1;

  MRaw<WT> w;
  float s0[2][4] = {}, s1[2][4] = {};
  float4 xv[NBT * 2];
  mfma_load_w<WT>(a, arow, k_begin, min(kMKT, k_end - k_begin), kq, w);
  if (WT == M2_W_INT8G) mfma_load_s(a, rbase, lane, k_begin, s0);
  mfma_load_x<NBT>(a, k_begin, min(kMKT, k_end - k_begin), tid, xv);
  if (RMS) {
    // RMS factors of the chunk's groups: 8 lanes per (session, group), strided sums
    // combined in a fixed order
    const int per = a.n_partials / a.n_norm;
    for (int base = 0; base < a.B * ngc * 8; base += 512) {
      const int i = base + tid, pair = i >> 3, j = i & 7;
      float sum = 0.0f;
      if (pair < a.B * ngc) {
        const int b = pair / ngc, g = g0 + pair % ngc;
        for (int q = j; q < per; q += 8) sum += a.ss[(size_t)b * a.n_partials + g * per + q];
      }
      sum = group_reduce<8>(sum);
      if (pair < a.B * ngc && j == 0) rn_s[pair] = 1.0f / sqrtf(sum / (float)a.ng + a.eps);
    }
    __syncthreads();
  }
  mfma_store_x<NBT, RMS>(a, k_begin, tid, xv, xs, xs + XB, rn_s, g0, ngc);
  __syncthreads();

  f32x4 acc[NBT];
#pragma unroll
  for (int j = 0; j < NBT; ++j) acc[j] = f32x4{};
  int buf = 0;
  for (int kt = k_begin; kt < k_end; kt += kMKT) {
    const int kn = kt + kMKT;
    if (kn < k_end) {
      mfma_load_x<NBT>(a, kn, min(kMKT, k_end - kn), tid, xv);
      if (WT == M2_W_INT8G) mfma_load_s(a, rbase, lane, kn, s1);
    }
    mfma_tile<WT, NBT>(a, w, s0, min(kMKT, k_end - kt), lane, kq, xs + 2 * buf * XB, xs + (2 * buf + 1) * XB, acc,
                       arow, kn, k_end);
    if (kn >= k_end) break;
    mfma_store_x<NBT, RMS>(a, kn, tid, xv, xs + 2 * (buf ^ 1) * XB, xs + (2 * (buf ^ 1) + 1) * XB, rn_s, g0, ngc);
    if (WT == M2_W_INT8G) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) s0[q][r] = s1[q][r];
    }
    __syncthreads();
    buf ^= 1;
  }
  // lane l, reg r -> row rbase + (l/16)*4 + r, session 16 j + l % 16
  float *part = a.part + (size_t)blockIdx.y * a.B * a.rows;
#pragma unroll
  for (int j = 0; j < NBT; ++j) {
    const int b = 16 * j + (lane & 15);
    if (b >= a.B) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = rbase + (lane >> 4) * 4 + r;
      if (rr < a.rows) part[(size_t)b * a.rows + rr] = acc[j][r];
    }
  }
}

// Sum of the K-chunk partials in chunk order, then the row epilogue.
template <int EPI>
__global__ void gemv_mfma_reduce_kernel(GemvArgs a, const float *part, int ks) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (EPI == EPI_OUT && a.conv_cache) conv_cache_shift(a, idx, (size_t)gridDim.x * blockDim.x);
  if (idx >= a.rows * a.B) return;
  const int b = idx / a.rows, row = idx - b * a.rows;
  const EpiIn e = epilogue_prefetch<EPI>(a, row, b);
  float v = 0.0f;
  for (int s = 0; s < ks; ++s) v += part[((size_t)s * a.B + b) * a.rows + row];
  gemv_epilogue<EPI>(a, row, b, v, e);
}

__global__ void state_zero_kernel(float *ssm, float *conv, size_t ssm_per, size_t conv_per,
                                  const int32_t *slots, int n, int n_slots) {
  const int i = blockIdx.y;
  const int slot = slots ? slots[i] : i;
  if (slot < 0 || slot >= n_slots) return;
  float *s = ssm + (size_t)slot * ssm_per;
  float *c = conv + (size_t)slot * conv_per;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < ssm_per + conv_per;
       e += (size_t)gridDim.x * blockDim.x) {
    if (e < ssm_per) s[e] = 0.0f;
    else c[e - ssm_per] = 0.0f;
  }
}

// ---------------------------------------------------------------------------
// launch helpers

template <typename F>
hipError_t allow_lds(F *kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

constexpr size_t kWaveLdsMax = 96 * 1024;

size_t wave_lds_bytes(const GemvArgs &a, int BT, int PRO) {
  return sizeof(float) * ((size_t)BT * a.K + (PRO == PRO_NORM ? (size_t)a.n_partials + (size_t)BT * a.n_norm : 0));
}

template <int WT, int BT, int TPB, int U, int NT, int PRO, int EPI>
hipError_t launch_wave(const GemvArgs &a, hipStream_t stream) {
  constexpr int WPB = TPB / 64;
  const size_t lds = wave_lds_bytes(a, BT, PRO);
  auto *k = gemv_wave_kernel<WT, BT, TPB, U, NT, PRO, EPI>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((a.rows + WPB - 1) / WPB), dim3(TPB), lds, stream, a);
  return hipGetLastError();
}

template <int WT, int BT, int KS, int PRO, int EPI, int U>
hipError_t launch_tiled(const GemvArgs &a, hipStream_t stream) {
  constexpr int RPW = 16 / KS;
  dim3 grid((a.rows + RPW - 1) / RPW, (a.B + BT - 1) / BT);
  const size_t lds = sizeof(float) * ((size_t)BT * a.KT +
                                      (PRO == PRO_NORM ? (size_t)a.n_partials + (size_t)BT * a.n_norm : 0) +
                                      16 * BT);
  auto *k = gemv_tiled_kernel<WT, BT, KS, PRO, EPI, U>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

int pick_kt(int K, int BT) {
  const int kt = (kLdsFloatsPerBatch / BT) & ~255;
  return K <= kt ? K : kt;
}

size_t lowbit_lds_bytes(const GemvArgs &a, int BT, int PRO) {
  return sizeof(float) * ((size_t)BT * (lds_padded(a.K) + a.K / 32) +
                          (PRO == PRO_NORM ? (size_t)BT * (a.n_partials + a.n_norm) : 0));
}

template <int WT, int BT, int R, int U, int NT, int PRO, int EPI>
hipError_t launch_lowbit(const GemvArgs &a, hipStream_t stream) {
  const size_t lds = lowbit_lds_bytes(a, BT, PRO);
  auto *k = gemv_lowbit_kernel<WT, BT, R, U, NT, PRO, EPI>;
  hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  // persistent: at most the workgroups resident at once (two per CU), at least one group each
  const int rows_per_block = (kLbThreads / 64) * R;
  const int blocks = std::min((a.rows + rows_per_block - 1) / rows_per_block, 2 * 256);
  hipLaunchKernelGGL(k, dim3(blocks), dim3(kLbThreads), lds, stream, a);
  return hipGetLastError();
}

// in_proj: U=5 nontemporal loads; out_proj: U=8 cached loads (measured best on gfx950).
// Low-bit codes at 1-2 sessions: the persistent low-bit GEMV, one row per wave group
// (two for in_proj at 2 sessions), 3 or 5 chunk columns per lane (rows of up to 6144 or
// 10240 codes).
template <int WT, int PRO, int EPI>
hipError_t dispatch_bt(GemvArgs a, hipStream_t stream) {
  constexpr bool LOWBIT = WT == M2_W_INT4G || WT == M2_W_INT3G;
  if constexpr (LOWBIT) {
    const bool fits = a.K / 4 <= kLbThreads * kNormF4PerThread && (PRO != PRO_NORM || a.n_partials <= kLbThreads) &&
                      lowbit_lds_bytes(a, a.B, PRO) <= kWaveLdsMax && a.K / 32 <= 64 * 5;
    if (a.B <= 2 && fits) {
      const bool u3 = a.K / 32 <= 64 * 3;
      if (EPI == EPI_INPROJ) {
        if (a.B == 1) return u3 ? launch_lowbit<WT, 1, 1, 3, 1, PRO, EPI>(a, stream) : launch_lowbit<WT, 1, 1, 5, 1, PRO, EPI>(a, stream);
        return u3 ? launch_lowbit<WT, 2, 2, 3, 1, PRO, EPI>(a, stream) : launch_lowbit<WT, 2, 2, 5, 1, PRO, EPI>(a, stream);
      }
      if (a.B == 1) return u3 ? launch_lowbit<WT, 1, 1, 3, 0, PRO, EPI>(a, stream) : launch_lowbit<WT, 1, 1, 5, 0, PRO, EPI>(a, stream);
      return u3 ? launch_lowbit<WT, 2, 1, 3, 0, PRO, EPI>(a, stream) : launch_lowbit<WT, 2, 1, 5, 0, PRO, EPI>(a, stream);
    }
  }
  constexpr int KS = EPI == EPI_INPROJ ? 1 : 4;
  const bool regs_ok = PRO != PRO_NORM || (a.K / 4 <= 512 * kNormF4PerThread && a.n_partials <= 512 && a.n_norm <= 512);
  if (a.B <= 2 && regs_ok && wave_lds_bytes(a, a.B, PRO) <= kWaveLdsMax) {
    if (EPI == EPI_INPROJ) {
      if (a.B == 1) return launch_wave<WT, 1, 512, 5, 1, PRO, EPI>(a, stream);
      return launch_wave<WT, 2, 512, 5, 1, PRO, EPI>(a, stream);
    }
    if (a.B == 1) return launch_wave<WT, 1, 512, 8, 0, PRO, EPI>(a, stream);
    return launch_wave<WT, 2, 512, 8, 0, PRO, EPI>(a, stream);
  }
  if (a.B >= 4) {
    a.KT = pick_kt(a.K, 4);
    return launch_tiled<WT, 4, KS, PRO, EPI, 8>(a, stream);
  }
  if (a.B >= 2) {
    a.KT = pick_kt(a.K, 2);
    return launch_tiled<WT, 2, KS, PRO, EPI, 8>(a, stream);
  }
  a.KT = pick_kt(a.K, 1);
  return launch_tiled<WT, 1, KS, PRO, EPI, 8>(a, stream);
}

template <int PRO, int EPI>
hipError_t dispatch_wt(int wtype, const GemvArgs &a, hipStream_t stream) {
  switch (wtype) {
    case M2_W_F32: return dispatch_bt<M2_W_F32, PRO, EPI>(a, stream);
    case M2_W_BF16: return dispatch_bt<M2_W_BF16, PRO, EPI>(a, stream);
    case M2_W_INT4G: return dispatch_bt<M2_W_INT4G, PRO, EPI>(a, stream);
    case M2_W_INT3G: return dispatch_bt<M2_W_INT3G, PRO, EPI>(a, stream);
    default: return dispatch_bt<M2_W_INT8G, PRO, EPI>(a, stream);
  }
}

// ---------------------------------------------------------------------------
// MFMA GEMV planning: 128-row workgroups over K chunks of whole 256-wide tiles, at
// most as many workgroups as are resident at once on the 256 CUs of an MI355X (2
// per CU), so that no second, partial round of workgroups forms a tail.
struct MfmaPlan {
  int ks, kchunk, nbt;
  size_t lds;
};

MfmaPlan mfma_plan(int rows, int K, int B, int ng) {
  MfmaPlan p;
  p.nbt = B <= 16 ? 1 : 2;
  const int rb = (rows + kMRows - 1) / kMRows;
  const int ntiles = (K + kMKT - 1) / kMKT;
  const int target = 512;                              // 2 resident workgroups per CU
  int ks = target / rb;
  if (ks > ntiles) ks = ntiles;
  if (ks < 1) ks = 1;
  const int tiles_per = (ntiles + ks - 1) / ks;
  p.kchunk = tiles_per * kMKT;
  p.ks = (K + p.kchunk - 1) / p.kchunk;
  const int ngc = ng > 0 ? p.kchunk / ng + 2 : 0;      // norm groups a chunk can touch
  p.lds = 4 * sizeof(unsigned short) * (size_t)p.nbt * 16 * kMLD + sizeof(float) * (size_t)B * ngc;
  return p;
}

template <int WT, int NBT, bool RMS>
hipError_t launch_mfma_k(const MfmaArgs &m, const MfmaPlan &p, hipStream_t stream) {
  auto *k = gemv_mfma_kernel<WT, NBT, RMS>;
  hipError_t e = allow_lds(k, p.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((m.rows + kMRows - 1) / kMRows, p.ks), dim3(512), p.lds, stream, m);
  return hipGetLastError();
}

template <int WT, bool RMS>
hipError_t launch_mfma(const MfmaArgs &m, const MfmaPlan &p, hipStream_t stream) {
  return p.nbt == 1 ? launch_mfma_k<WT, 1, RMS>(m, p, stream) : launch_mfma_k<WT, 2, RMS>(m, p, stream);
}

// One MFMA GEMV + reduce for the arguments of a gemv_* launch; out_proj (EPI_OUT)
// also forms the RMS factors from g.ss.
template <int EPI>
hipError_t run_mfma_gemv(const m2_config &c, const GemvArgs &g, float *part, hipStream_t stream) {
  constexpr bool RMS = EPI == EPI_OUT;
  const MfmaPlan p = mfma_plan(g.rows, g.K, g.B, RMS ? g.ng : 0);
  MfmaArgs m{};
  m.W = g.W;
  m.S = static_cast<const __half *>(g.S);
  m.rows = g.rows;
  m.K = g.K;
  m.q_group = c.wtype == M2_W_INT8G ? c.q_group : g.K;
  m.kchunk = p.kchunk;
  m.act = g.act;
  m.B = g.B;
  m.ss = g.ss;
  m.n_partials = g.n_partials;
  m.n_norm = g.n_norm;
  m.ng = g.ng;
  m.eps = g.eps;
  m.part = part;
  hipError_t e = c.wtype == M2_W_BF16 ? launch_mfma<M2_W_BF16, RMS>(m, p, stream)
                                      : launch_mfma<M2_W_INT8G, RMS>(m, p, stream);
  if (e != hipSuccess) return e;
  const int n = g.rows * g.B;
  hipLaunchKernelGGL(gemv_mfma_reduce_kernel<EPI>, dim3((n + 255) / 256), dim3(256), 0, stream, g, part, p.ks);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int log2i(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// ---------------------------------------------------------------------------
// Output heads (text head, function head): logits = gamma * W h for a [V][K] matrix and
// the greedy token argmax_v logits (the lowest index among equal maxima; a NaN logit never
// wins), per session. head_wave_kernel: one row per wave as in gemv_wave_kernel (U chunks
// in flight, activations staged once per workgroup), then the workgroup's best (logit,
// index) per session into part[session][workgroup]; head_reduce_kernel: one workgroup per
// session takes the best over the partials. Both reductions keep the winner by value,
// then by index, so the result does not depend on the order in which they combine.
struct HeadArgs {
  const void *W;
  const void *S;
  int rows, K, q_shift;
  float gamma;
  const float *h;         // [B][K]
  int B;
  float *logits;          // [B][rows] or null
  int32_t *token;         // [B]
  float2 *part;           // [4][gridDim]: per session the workgroups' (logit, index bits)
  int nparts;
};

__device__ __forceinline__ bool head_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int WT, int BT, int U>
__global__ __launch_bounds__(512) void head_wave_kernel(HeadArgs a) {
  extern __shared__ float lds[];
  constexpr int TPB = 512, WPB = TPB / 64;
  constexpr int EPC = WTraits<WT>::EPC;
  constexpr int CB = WTraits<WT>::CB;
  using chunk_t = typename WTraits<WT>::chunk_t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x * WPB + wave;
  const bool row_ok = row < a.rows;
  const int nb = min(BT, a.B);
  const int K = a.K, NC = K / EPC;
  const char *wr = static_cast<const char *>(a.W) + (size_t)(row_ok ? row : 0) * NC * CB;
  const void *srow = scale_row<WT>(a.S, (size_t)(row_ok ? row : 0), NC >> a.q_shift);
  chunk_t w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = lane + 64 * u;
    w[u] = (row_ok && c < NC) ? load_chunk<WT, 1>(wr, c) : chunk_t{};
  }
  float *act_s = lds;
  float2 *best = reinterpret_cast<float2 *>(lds + BT * K);   // [WPB][BT]
#pragma unroll
  for (int bb = 0; bb < BT; ++bb)
    for (int i = tid * 4; i < K; i += TPB * 4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (bb < nb) v = *reinterpret_cast<const float4 *>(a.h + (size_t)bb * K + i);
      *reinterpret_cast<float4 *>(act_s + bb * K + i) = v;
    }
  __syncthreads();
  float acc[BT];
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) acc[bb] = 0.0f;
  if (row_ok) {
    for (int cb = lane;;) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb + 64 * u;
        if (c < NC) {
          const QScale qs = load_qscale<WT>(srow, c, a.q_shift);
#pragma unroll
          for (int bb = 0; bb < BT; ++bb) acc[bb] = chunk_acc<WT>(w[u], act_s + bb * K + c * EPC, qs, acc[bb]);
        }
      }
      cb += 64 * U;
      if (cb >= NC) break;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb + 64 * u;
        w[u] = c < NC ? load_chunk<WT, 1>(wr, c) : chunk_t{};
      }
    }
  }
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    acc[bb] = group_reduce<64>(acc[bb]);
  }
  if (lane < BT) {
    float val = 0.0f;
#pragma unroll
    for (int bb = 0; bb < BT; ++bb)
      if (lane == bb) val = acc[bb];
    val *= a.gamma;
    const bool ok = row_ok && lane < nb;
    if (ok && a.logits) a.logits[(size_t)lane * a.rows + row] = val;
    best[wave * BT + lane] = ok ? make_float2(val, __int_as_float(row)) : make_float2(-INFINITY, __int_as_float(INT_MAX));
  }
  __syncthreads();
  if (tid < BT) {                       // rows rise with the wave index
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int w8 = 0; w8 < WPB; ++w8) {
      const float2 e = best[w8 * BT + tid];
      if (head_better(e.x, __float_as_int(e.y), bv, bi)) {
        bv = e.x;
        bi = __float_as_int(e.y);
      }
    }
    a.part[(size_t)tid * a.nparts + blockIdx.x] = make_float2(bv, __int_as_float(bi));
  }
}

// One workgroup of 1024 threads per session; every thread first issues all of its (up to 16
// per pass) loads of the session's contiguous partials, then combines them, so that a pass
// costs one memory latency rather than one per partial.
__global__ __launch_bounds__(1024) void head_reduce_kernel(HeadArgs a) {
  constexpr int TPB = 1024, L = 16;
  __shared__ float sv[TPB / 64];
  __shared__ int si[TPB / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float2 *part = a.part + (size_t)b * a.nparts;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int p0 = tid; p0 < a.nparts; p0 += TPB * L) {
    float2 e[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int p = p0 + j * TPB;
      e[j] = p < a.nparts ? part[p] : make_float2(-INFINITY, __int_as_float(INT_MAX));
    }
#pragma unroll
    for (int j = 0; j < L; ++j)
      if (head_better(e[j].x, __float_as_int(e[j].y), bv, bi)) {
        bv = e[j].x;
        bi = __float_as_int(e[j].y);
      }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (head_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < TPB / 64; ++w)
      if (head_better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    a.token[b] = bi == INT_MAX ? -1 : bi;
  }
}

hipError_t record(hipEvent_t const *ev, int i, hipStream_t stream) {
  return (ev && ev[i]) ? hipEventRecord(ev[i], stream) : hipSuccess;
}

template <int WT, int BT>
hipError_t launch_head_bt(const HeadArgs &a, hipStream_t stream, hipEvent_t const *ev) {
  const size_t lds = sizeof(float) * ((size_t)BT * a.K + 2 * 8 * BT);
  auto *k = head_wave_kernel<WT, BT, 5>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipError_t e = record(ev, 0, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(a.nparts), dim3(512), lds, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = record(ev, 1, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_reduce_kernel, dim3(a.B), dim3(1024), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = record(ev, 2, stream);
  return e;
}

template <int WT>
hipError_t launch_head_wt(const HeadArgs &a, hipStream_t stream, hipEvent_t const *ev) {
  if (a.B == 1) return launch_head_bt<WT, 1>(a, stream, ev);
  if (a.B == 2) return launch_head_bt<WT, 2>(a, stream, ev);
  return launch_head_bt<WT, 4>(a, stream, ev);
}

}  // namespace

StepWs step_ws_layout(const m2_layer_s &L, int batch, void *base) {
  StepWs w{};
  char *p = static_cast<char *>(base);
  size_t off = 0;
  const size_t zx = align256(sizeof(float) * (size_t)batch * L.zx_stride);
  const size_t v = align256(sizeof(float) * (size_t)batch * L.d_inner);
  const size_t ss = align256(sizeof(float) * (size_t)batch * L.n_partials);
  w.zx = p ? reinterpret_cast<float *>(p + off) : nullptr;
  off += zx;
  w.v = p ? reinterpret_cast<float *>(p + off) : nullptr;
  off += v;
  w.ss = p ? reinterpret_cast<float *>(p + off) : nullptr;
  off += ss;
  if (step_uses_mfma(L, batch)) {
    const MfmaPlan pi = mfma_plan(L.d_in_proj, L.cfg.d_model, batch, 0);
    const MfmaPlan po = mfma_plan(L.cfg.d_model, L.d_inner, batch, L.ng);
    const size_t n_in = (size_t)pi.ks * batch * L.d_in_proj, n_out = (size_t)po.ks * batch * L.cfg.d_model;
    w.part = p ? reinterpret_cast<float *>(p + off) : nullptr;
    off += align256(sizeof(float) * (n_in > n_out ? n_in : n_out));
  }
  w.bytes = off;
  return w;
}

// SSD item shapes (measured on gfx950): one or two sessions are latency-bound, and
// 8 waves with at most 2 slices each finish an item soonest; larger batches are
// bound by the state stream, where small items with few registers (many items
// resident) move it fastest.
hipError_t launch_ssd(const SsdArgs &sa, int items, int batch, hipStream_t stream) {
  const int rpi = 64 / (sa.N / 4);
  const int n_inst = (sa.prange + rpi - 1) / rpi;
  const dim3 grid(items, batch);
  if (batch <= 2 && n_inst <= 16)
    hipLaunchKernelGGL((ssd_step_kernel<8, 2>), grid, dim3(512), 0, stream, sa);
  else if (n_inst <= 10)
    hipLaunchKernelGGL((ssd_step_kernel<2, 5>), grid, dim3(128), 0, stream, sa);
  else if (n_inst <= 16)
    hipLaunchKernelGGL((ssd_step_kernel<4, 4>), grid, dim3(256), 0, stream, sa);
  else
    hipLaunchKernelGGL((ssd_step_kernel<4, 8>), grid, dim3(256), 0, stream, sa);
  return hipGetLastError();
}

hipError_t launch_step(const m2_layer_s &L, const m2_state_s &S, const float *x, float *y, int batch,
                       const int32_t *slots, int flags, const StepWs &ws, hipStream_t stream,
                       hipEvent_t const *events) {
  const m2_config &c = L.cfg;
  auto mark = [&](int i) -> hipError_t {
    return (events && events[i]) ? hipEventRecord(events[i], stream) : hipSuccess;
  };
  const bool quantized = c.wtype == M2_W_INT8G || c.wtype == M2_W_INT4G || c.wtype == M2_W_INT3G;
  const int epc = c.wtype == M2_W_F32 ? 4 : c.wtype == M2_W_BF16 ? 8 : c.wtype == M2_W_INT8G ? 16 : 32;
  const int q_shift = quantized ? log2i(c.q_group / epc) : 30;
  hipError_t e = mark(0);
  if (e != hipSuccess) return e;
  // 1. in_proj + conv + dt
  GemvArgs gi{};
  gi.W = L.w.w_in;
  gi.S = L.w.s_in;
  gi.rows = L.d_in_proj;
  gi.K = c.d_model;
  gi.q_shift = q_shift;
  gi.gamma = quantized ? c.q_gamma_in : 1.0f;
  gi.act = x;
  gi.B = batch;
  gi.zx = ws.zx;
  gi.zx_stride = L.zx_stride;
  gi.d_inner = L.d_inner;
  gi.conv_dim = L.conv_dim;
  gi.d_conv = c.d_conv;
  gi.dt_bias = L.w.dt_bias;
  gi.slots = slots;
  gi.n_slots = S.n_slots;
  const bool mfma = step_uses_mfma(L, batch);
  e = mfma ? run_mfma_gemv<EPI_INPROJ>(c, gi, ws.part, stream)
           : dispatch_wt<PRO_PLAIN, EPI_INPROJ>(c.wtype, gi, stream);
  if (e == hipSuccess) e = mark(1);
  if (e != hipSuccess) return e;

  // 2. SSD update + readout + gate + sums of squares
  SsdArgs sa{};
  sa.zx = ws.zx;
  sa.zx_stride = L.zx_stride;
  sa.d_inner = L.d_inner;
  sa.conv_dim = L.conv_dim;
  sa.H = c.n_heads;
  sa.P = c.head_dim;
  sa.N = c.d_state;
  sa.G = c.n_groups;
  sa.hpg = L.hpg;
  sa.ssm = S.ssm;
  sa.conv_cache = S.conv;
  sa.conv_w = L.w.conv_w;
  sa.conv_b = L.w.conv_b;
  sa.d_conv = c.d_conv;
  sa.A_log = L.w.A_log;
  sa.D = L.w.D;
  sa.norm_w = L.w.norm_w;
  sa.vw = ws.v;
  sa.ss = ws.ss;
  sa.prange = L.prange;
  sa.psplit = L.psplit;
  sa.n_partials = L.n_partials;
  sa.slots = slots;
  sa.n_slots = S.n_slots;

  // 3. RMSNorm + out_proj (+ residual)
  GemvArgs go{};
  go.W = L.w.w_out;
  go.S = L.w.s_out;
  go.rows = c.d_model;
  go.K = L.d_inner;
  go.q_shift = q_shift;
  go.gamma = quantized ? c.q_gamma_out : 1.0f;
  go.act = ws.v;
  go.B = batch;
  go.ss = ws.ss;
  go.ng = L.ng;
  go.n_partials = L.n_partials;
  go.n_norm = L.n_norm;
  go.eps = c.norm_eps;
  go.y = y;
  go.resid = (flags & M2_RESIDUAL) ? x : nullptr;
  go.slots = slots;
  go.n_slots = S.n_slots;
  go.zx = ws.zx;                 // raw x|B|C of this step, for the conv-cache shift
  go.zx_stride = L.zx_stride;
  go.d_inner = L.d_inner;
  go.conv_dim = L.conv_dim;
  go.d_conv = c.d_conv;
  go.conv_cache = S.conv;
  e = launch_ssd(sa, c.n_heads * L.psplit, batch, stream);
  if (e == hipSuccess) e = mark(2);
  if (e != hipSuccess) return e;
  if (mfma) {
    e = run_mfma_gemv<EPI_OUT>(c, go, ws.part, stream);
  } else {
    e = dispatch_wt<PRO_NORM, EPI_OUT>(c.wtype, go, stream);
  }
  if (e == hipSuccess) e = mark(3);
  return e;
}

// Batches of 3..32 sessions with bf16 weights, or int8 weights in groups of 128 or
// 256, run the projections as MFMA GEMVs; the rest as VALU GEMVs.
int step_plan(const m2_layer_s &L, int batch) {
  const m2_config &c = L.cfg;
  if (batch < 3 || batch > 32) return kPlanValu;
  if (c.wtype == M2_W_BF16) return kPlanMfma;
  return c.wtype == M2_W_INT8G && (c.q_group == 128 || c.q_group == 256) ? kPlanMfma : kPlanValu;
}

bool step_uses_mfma(const m2_layer_s &L, int batch) { return step_plan(L, batch) == kPlanMfma; }


hipError_t launch_state_zero(const m2_state_s &S, const int32_t *slots, int n, hipStream_t stream) {
  const m2_layer_s &L = *S.layer;
  const size_t ssm_per = (size_t)L.d_inner * L.cfg.d_state;
  const size_t conv_per = (size_t)(L.cfg.d_conv - 1) * L.conv_dim;
  const size_t per = ssm_per + conv_per;
  const unsigned gx = (unsigned)((per + 256 * 16 - 1) / (256 * 16));
  hipLaunchKernelGGL(state_zero_kernel, dim3(gx, n), dim3(256), 0, stream, S.ssm, S.conv, ssm_per,
                     conv_per, slots, n, S.n_slots);
  return hipGetLastError();
}

bool gemv_plain_uses_mfma(int wtype, int q_group, int batch) {
  if (batch < 3 || batch > 32) return false;
  return wtype == M2_W_BF16 || (wtype == M2_W_INT8G && (q_group == 128 || q_group == 256));
}

size_t gemv_plain_part_bytes(int wtype, int q_group, int rows, int K, int batch) {
  if (!gemv_plain_uses_mfma(wtype, q_group, batch)) return 0;
  const MfmaPlan p = mfma_plan(rows, K, batch, 0);
  return sizeof(float) * (size_t)p.ks * batch * rows;
}

hipError_t launch_gemv_plain(int wtype, const void *W, const void *S, int rows, int K, int q_group, float gamma,
                             const float *act, int batch, float *y, const float *resid, float *part,
                             hipStream_t stream) {
  const bool quantized = wtype == M2_W_INT8G || wtype == M2_W_INT4G || wtype == M2_W_INT3G;
  const int epc = wtype == M2_W_F32 ? 4 : wtype == M2_W_BF16 ? 8 : wtype == M2_W_INT8G ? 16 : 32;
  GemvArgs a{};
  a.W = W;
  a.S = S;
  a.rows = rows;
  a.K = K;
  a.q_shift = quantized ? log2i(q_group / epc) : 30;
  a.gamma = quantized ? gamma : 1.0f;
  a.act = act;
  a.B = batch;
  a.y = y;
  a.resid = resid;
  a.slots = nullptr;
  a.n_slots = batch;
  // 3-32 sessions with bf16 (or int8 g128/g256) weights: the MFMA GEMV over K chunks, then
  // the reduction with the plain epilogue (as the decode step's MFMA plan, without RMS).
  if (gemv_plain_uses_mfma(wtype, q_group, batch)) {
    const MfmaPlan p = mfma_plan(rows, K, batch, 0);
    MfmaArgs m{};
    m.W = W;
    m.S = static_cast<const __half *>(S);
    m.rows = rows;
    m.K = K;
    m.q_group = wtype == M2_W_INT8G ? q_group : K;
    m.kchunk = p.kchunk;
    m.act = act;
    m.B = batch;
    m.part = part;
    hipError_t e = wtype == M2_W_BF16 ? launch_mfma<M2_W_BF16, false>(m, p, stream)
                                      : launch_mfma<M2_W_INT8G, false>(m, p, stream);
    if (e != hipSuccess) return e;
    const int n = rows * batch;
    hipLaunchKernelGGL(gemv_mfma_reduce_kernel<EPI_OUT>, dim3((n + 255) / 256), dim3(256), 0, stream, a, part, p.ks);
    return hipGetLastError();
  }
  // 1-2 sessions, 2- and 4-byte weights: the in_proj configuration (5 nontemporal loads in
  // flight); otherwise the decode step's choice for out_proj.
  if (batch <= 2 && (wtype == M2_W_BF16 || wtype == M2_W_F32) && wave_lds_bytes(a, batch, PRO_PLAIN) <= kWaveLdsMax) {
    if (wtype == M2_W_BF16)
      return batch == 1 ? launch_wave<M2_W_BF16, 1, 512, 5, 1, PRO_PLAIN, EPI_OUT>(a, stream)
                        : launch_wave<M2_W_BF16, 2, 512, 5, 1, PRO_PLAIN, EPI_OUT>(a, stream);
    return batch == 1 ? launch_wave<M2_W_F32, 1, 512, 5, 1, PRO_PLAIN, EPI_OUT>(a, stream)
                      : launch_wave<M2_W_F32, 2, 512, 5, 1, PRO_PLAIN, EPI_OUT>(a, stream);
  }
  return dispatch_wt<PRO_PLAIN, EPI_OUT>(wtype, a, stream);
}

size_t head_ws_bytes(int vocab) { return sizeof(float2) * 4 * (size_t)((vocab + 7) / 8); }

hipError_t launch_head(const m2_head_config &c, const void *w, const void *scales, const float *h, int batch,
                       int32_t *token, float *logits, void *ws, hipStream_t stream, hipEvent_t const *events) {
  const int epc = c.wtype == M2_W_F32 ? 4 : c.wtype == M2_W_BF16 ? 8 : c.wtype == M2_W_INT8G ? 16 : 32;
  const bool quantized = c.wtype == M2_W_INT8G || c.wtype == M2_W_INT4G || c.wtype == M2_W_INT3G;
  HeadArgs a{};
  a.W = w;
  a.S = scales;
  a.rows = c.vocab;
  a.K = c.d_model;
  a.q_shift = quantized ? log2i(c.q_group / epc) : 30;
  a.gamma = quantized ? c.q_gamma : 1.0f;
  a.part = static_cast<float2 *>(ws);
  a.nparts = (c.vocab + 7) / 8;
  for (int b0 = 0; b0 < batch; b0 += 4) {      // up to 4 sessions per launch, in stream order
    a.h = h + (size_t)b0 * c.d_model;
    a.B = batch - b0 < 4 ? batch - b0 : 4;
    a.logits = logits ? logits + (size_t)b0 * c.vocab : nullptr;
    a.token = token + b0;
    hipError_t e;
    switch (c.wtype) {
      case M2_W_F32: e = launch_head_wt<M2_W_F32>(a, stream, events); break;
      case M2_W_BF16: e = launch_head_wt<M2_W_BF16>(a, stream, events); break;
      case M2_W_INT4G: e = launch_head_wt<M2_W_INT4G>(a, stream, events); break;
      case M2_W_INT3G: e = launch_head_wt<M2_W_INT3G>(a, stream, events); break;
      default: e = launch_head_wt<M2_W_INT8G>(a, stream, events); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace m2d
