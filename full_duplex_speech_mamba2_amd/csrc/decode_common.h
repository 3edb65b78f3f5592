// Device helpers shared by the decode kernels (decode.hip) and the persistent one-launch
// decode step (fused.hip): weight chunk loads and dot products for every storage format,
// the GEMV argument blocks and row epilogues, the RMS staging of out_proj's activations,
// the causal conv of the SSD items and the SSD item itself.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

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

// A buffer offset past every resource the kernels build: a raw buffer load there returns
// zeros without a memory access, so a load that must not read can still be issued without
// a branch, and the compiler's wait counts for the loads around it stay exact.
constexpr int kBufOutOfRange = 0x7ffffff0;
__host__ __device__ constexpr int lds_padded(int K) { return lds_pad(K - 1) + 1; }   // a multiple of 4 for K % 4 == 0

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ float softplus(float a) { return a > 20.0f ? a : log1pf(expf(a)); }

// Loads and stores of data that workgroups hand to each other inside one launch (COH): they
// go past the per-XCD caches (agent-scope relaxed atomics: the sc1 policy), so a store
// completed before a grid barrier is seen by a load after it on any XCD, with no cache
// write-back or invalidation. Without COH: plain accesses (the data crosses a kernel
// boundary instead).
template <bool COH>
__device__ __forceinline__ float ldc(const float *p) {
  if constexpr (COH) return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH>
__device__ __forceinline__ void stc(float *p, float v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ float4 ldc4(const float *p) {
  if constexpr (COH) return make_float4(ldc<true>(p), ldc<true>(p + 1), ldc<true>(p + 2), ldc<true>(p + 3));
  else return *reinterpret_cast<const float4 *>(p);
}

// Grid-barrier words of the persistent SSD + out_proj kernel, one per 128-byte line (their
// atomics and polls then go to different memory channels): a counter per group of
// workgroups (blockIdx % 8, the XCD the dispatcher sends a workgroup to), the count of
// groups complete, a release flag per group, and a flag raised when a bounded wait ran out.
// All zero before the kernel starts (the in_proj kernel before it zeroes them).
constexpr int kBarStride = 32;          // words per line
constexpr int kBarGroups = 8;
constexpr int kBarCount = 0, kBarTop = kBarGroups, kBarFlag = kBarGroups + 1, kBarError = 2 * kBarGroups + 1;
constexpr int kBarWords = 2 * kBarGroups + 2;
constexpr int kBarBytes = kBarWords * kBarStride * 4;

// A workgroup barrier that orders LDS accesses only: unlike __syncthreads it does not wait
// for the waves' global loads in flight (weights requested for a later phase).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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
  unsigned *bar_clear;    // in_proj: the grid-barrier words of the kernel after it, zeroed here (or null)
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
template <bool ZC = false>
__device__ __forceinline__ void conv_cache_shift(const GemvArgs &a, size_t gtid, size_t gthreads) {
  const size_t total = (size_t)a.B * a.conv_dim;
  const int nk = a.d_conv - 1;                      // 1..7 cached inputs
  for (size_t i = gtid; i < total; i += gthreads) {
    const int b = (int)(i / a.conv_dim), c = (int)(i - (size_t)b * a.conv_dim);
    const int slot = a.slots ? a.slots[b] : b;
    if (slot < 0 || slot >= a.n_slots) continue;
    float *cc = a.conv_cache + (size_t)slot * nk * a.conv_dim + c;
    // every old value first, then the stores: a store between the loads would make each
    // load wait for the one before it
    float v[7];
#pragma unroll
    for (int k = 0; k < 6; ++k) v[k] = k + 1 < nk ? cc[(size_t)(k + 1) * a.conv_dim] : 0.0f;
    v[6] = ldc<ZC>(a.zx + (size_t)b * a.zx_stride + a.d_inner + c);
#pragma unroll
    for (int k = 0; k < 6; ++k)
      if (k + 1 < nk) cc[(size_t)k * a.conv_dim] = v[k];
    cc[(size_t)(nk - 1) * a.conv_dim] = v[6];
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

// out_proj activation staging in one memory trip: each thread loads its float4s of
// v * norm_w (kept in registers) and, with them, its lanes' share of the sums-of-squares
// partials; wave w reduces norm groups w, w + W, ... (each lane a strided part of the
// group's partials, then a cross-lane tree: a fixed order) into their RMS factors, and after
// one barrier every thread writes its float4s scaled by their group's factor.
// LDS: act [BT][K] | rn [BT][n_norm]. K/4 <= 512 * kNormF4PerThread (each thread holds
// ceil(512 * kNormF4PerThread / TPB) float4s).
template <int BT, int TPB>
__device__ __forceinline__ void stage_norm_act(const GemvArgs &a, float *lds, int tid) {
  constexpr int MAXF = (kNormF4PerThread * 512 + TPB - 1) / TPB, W = TPB / 64;   // K/4 <= 512 * kNormF4PerThread
  const int K = a.K, nb = min(BT, a.B), nf = K / 4;
  const int lane = tid & 63, wave = tid >> 6;
  float *act_s = lds;
  float *rn = lds + BT * K;
  float4 v[BT][MAXF];
#pragma unroll
  for (int bb = 0; bb < BT; ++bb)
#pragma unroll
    for (int i = 0; i < MAXF; ++i) {
      const int f = tid + TPB * i;
      v[bb][i] = (bb < nb && f < nf) ? reinterpret_cast<const float4 *>(a.act + (size_t)bb * K)[f]
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  const int per = a.n_partials / a.n_norm;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    const float *ssb = a.ss + (size_t)min(bb, nb - 1) * a.n_partials;
    for (int g = wave; g < a.n_norm; g += W) {
      float sum = 0.0f;
      for (int q = lane; q < per; q += 64) sum += ssb[g * per + q];
      sum = group_reduce<64>(sum);
      if (lane == 0) rn[bb * a.n_norm + g] = 1.0f / sqrtf(sum / (float)a.ng + a.eps);
    }
  }
  __syncthreads();
  const int ng4 = a.ng / 4;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb)
#pragma unroll
    for (int i = 0; i < MAXF; ++i) {
      const int f = tid + TPB * i;
      if (f < nf) {
        const float r = bb < nb ? rn[bb * a.n_norm + f / ng4] : 0.0f;
        const float4 x = v[bb][i];
        reinterpret_cast<float4 *>(act_s + bb * K)[f] = make_float4(x.x * r, x.y * r, x.z * r, x.w * r);
      }
    }
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


// Causal conv + SiLU of 4 consecutive conv channels c0..c0+3 of one session
// (cache slot `slot`): bias + sum_k w[c][k] in(t-K+1+k), the last K-1 inputs from
// the cache, the newest the raw in_proj output.
// ZC: zx was written inside the same launch (read past the per-XCD caches).
template <bool ZC = false>
__device__ __forceinline__ float4 conv4(const SsdArgs &a, const float *zb, int slot, int c0) {
  const float4 raw = ldc4<ZC>(zb + a.d_inner + c0);
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

// The state slices of one SSD item held by one wave: MAXI float4s per lane, and the state
// row (p) each belongs to (-1: none).
template <int MAXI>
struct SsdTile {
  float4 st[MAXI];
  int prow[MAXI];
};

// First half of an item: the rows of the item's state tile this wave owns and their loads
// (the tile does not depend on the step's in_proj results, so a caller may issue this
// before they exist).
// `slot`: the session's state slot (slots[b], or b), read once by the caller.
template <int NW, int MAXI>
__device__ __forceinline__ void ssd_load(const SsdArgs &a, int h, int ps, int slot, int wave, int lane,
                                         SsdTile<MAXI> &t) {
  const int lpr = a.N >> 2;                 // lanes per state row
  const int rpi = 64 / lpr;                 // rows per wave instruction
  const int n_inst = (a.prange + rpi - 1) / rpi;
  const int r_in = lane / lpr, q = lane - r_in * lpr;
  const bool sok = slot >= 0 && slot < a.n_slots;
  const float4 *S = reinterpret_cast<const float4 *>(a.ssm + ((size_t)(sok ? slot : 0) * a.H + h) * a.P * a.N);
  // Every slice is loaded, unconditionally (rows past the item from its first row, an
  // out-of-range slot from slot 0): a load under a condition is joined to the other path
  // by register moves that wait for it at once. What such a slice holds is never stored
  // or read out (its readout lanes and its v are discarded; a bad slot's v is NaN).
#pragma unroll
  for (int k = 0; k < MAXI; ++k) {
    const int i = wave + NW * k;
    const int pl = i * rpi + r_in;
    t.prow[k] = (i < n_inst && pl < a.prange) ? ps * a.prange + pl : -1;
    t.st[k] = ld_stream(S + (size_t)(t.prow[k] >= 0 ? t.prow[k] : ps * a.prange) * lpr + q);
  }
}

// The updated tile back to the session's slot (nothing for an out-of-range slot).
template <int MAXI>
__device__ __forceinline__ void ssd_store(const SsdArgs &a, int h, int slot, int lane, const SsdTile<MAXI> &t) {
  const int lpr = a.N >> 2;
  const int q = lane - (lane / lpr) * lpr;
  if (slot < 0 || slot >= a.n_slots) return;
  float4 *S = reinterpret_cast<float4 *>(a.ssm + ((size_t)slot * a.H + h) * a.P * a.N);
#pragma unroll
  for (int k = 0; k < MAXI; ++k)
    if (t.prow[k] >= 0) st_stream(S + (size_t)t.prow[k] * lpr + q, t.st[k]);
}

// Second half: conv + SiLU of the item's channels, the update and readout on the tile (left
// updated in t), the gate, v * norm_w and the item's sum of squares. Must be called by every
// thread of the workgroup. STORE: write the tile back here (else the caller does, with
// ssd_store). active = false: compute, but write nothing (a workgroup without an item of
// its own runs a copy of another's, so that no branch around the call leaves the tile's
// loads unaccounted for).
struct NoOp {
  __device__ void operator()() const {}
};

// mid(): called by every wave once the item's own loads have all been issued and the conv
// outputs are in LDS (a caller's loads for a later phase, which then cannot delay these).
// ZC: zx was written inside the same launch, so its reads go past the per-XCD caches too.
template <int NW, int MAXI, bool STORE, bool COH = false, bool ZC = false, typename Mid = NoOp>
__device__ __forceinline__ void ssd_finish(const SsdArgs &a, int h, int ps, int b, int slot, int wave, int lane,
                                           SsdTile<MAXI> &t, float *wsum, float *cx, bool active = true,
                                           Mid &&mid = Mid()) {
  // COH: v and the sum of squares are read by other workgroups of the same launch, so they
  // are stored past the per-XCD caches, and the workgroup's barriers order LDS only (the
  // waves may have later weights in flight)
  auto wg_sync = [] {
    if constexpr (COH) lds_barrier();
    else __syncthreads();
  };
  const int g = h / a.hpg;
  const int lpr = a.N >> 2;                 // lanes per state row
  const int rpi = 64 / lpr;                 // rows per wave instruction
  const int n_inst = (a.prange + rpi - 1) / rpi;
  const int q = lane - (lane / lpr) * lpr;
  const float *zb = a.zx + (size_t)b * a.zx_stride;
  const bool sok = slot >= 0 && slot < a.n_slots;
  float zg[MAXI], nw[MAXI];                 // gate input and norm weight of the row (lane q == 0)
  // the epilogue's loads go out with the state's, not after the readout
#pragma unroll
  for (int k = 0; k < MAXI; ++k) {
    const bool need = q == 0 && t.prow[k] >= 0;
    zg[k] = need ? ldc<ZC>(zb + h * a.P + t.prow[k]) : 0.0f;
    nw[k] = need ? a.norm_w[h * a.P + t.prow[k]] : 0.0f;
  }
  const float dt = ldc<ZC>(zb + a.d_inner + a.conv_dim + h);
  const float dA = expf(-expf(a.A_log[h]) * dt);
  const float Dh = a.D[h];
  // conv outputs, each channel once per workgroup: B and C of the group and the
  // item's x rows, one float4 of channels per thread, through LDS (cx = [B | C | x])
  {
    const int n4 = a.N / 4;
    for (int i = wave * 64 + lane; i < 2 * n4 + a.prange / 4; i += NW * 64) {
      const int c0 = i < n4 ? a.d_inner + g * a.N + 4 * i
                   : i < 2 * n4 ? a.d_inner + (a.G + g) * a.N + 4 * (i - n4)
                   : h * a.P + ps * a.prange + 4 * (i - 2 * n4);
      reinterpret_cast<float4 *>(cx)[i] = conv4<ZC>(a, zb, sok ? slot : 0, c0);
    }
    wg_sync();
  }
  mid();
  const float4 Bq = reinterpret_cast<const float4 *>(cx)[q];
  const float4 Cq = reinterpret_cast<const float4 *>(cx + a.N)[q];
  const float *xs = cx + 2 * a.N;
  float ssacc = 0.0f;
#pragma unroll
  for (int k = 0; k < MAXI; ++k) {
    if (wave + NW * k >= n_inst) break;     // uniform across the wave
    const int p = t.prow[k];
    const float xp = p >= 0 ? xs[p - ps * a.prange] : 0.0f;
    const float dtx = dt * xp;
    float4 sv = t.st[k];
    sv.x = fmaf(dA, sv.x, dtx * Bq.x);
    sv.y = fmaf(dA, sv.y, dtx * Bq.y);
    sv.z = fmaf(dA, sv.z, dtx * Bq.z);
    sv.w = fmaf(dA, sv.w, dtx * Bq.w);
    t.st[k] = sv;
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
      if (active) stc<COH>(a.vw + (size_t)b * a.d_inner + ch, vv * nw[k]);
      ssacc = fmaf(vv, vv, ssacc);
    }
  }
  if (STORE && active) ssd_store<MAXI>(a, h, slot, lane, t);
  // sum of squares of this item's rows, in a fixed order
  ssacc = group_reduce<64>(ssacc);
  if (lane == 0) wsum[wave] = ssacc;
  wg_sync();
  if (wave == 0 && lane == 0 && active) {
    float s = 0.0f;
    for (int i = 0; i < NW; ++i) s += wsum[i];
    stc<COH>(a.ss + (size_t)b * a.n_partials + (h * a.P + ps * a.prange) / a.prange, s);
  }
  wg_sync();
}

// One SSD work item = (session b, head h, rows [ps*prange, (ps+1)*prange)), done by the NW
// waves of a workgroup: a state row (N floats) is read by N/4 lanes as float4; every slice
// of the tile is loaded before any is used, updated in registers and written once. wsum:
// LDS float[NW]. Must be called by every thread of the workgroup.
template <int NW, int MAXI>
__device__ __forceinline__ void ssd_item(const SsdArgs &a, int h, int ps, int b, int wave, int lane,
                                         float *wsum, float *cx) {
  SsdTile<MAXI> t;
  const int slot = a.slots ? a.slots[b] : b;
  ssd_load<NW, MAXI>(a, h, ps, slot, wave, lane, t);
  ssd_finish<NW, MAXI, true>(a, h, ps, b, slot, wave, lane, t, wsum, cx);
}

}  // namespace
}  // namespace m2d
