// Attention layers of the hybrid Mamba-2/attention backbone: one decode token per
// session with a bf16 KV cache (blog page "NemotronLabs VoiceChat 11B", "Key design
// decisions" item 2 and "Known limitations": attention layers between the Mamba layers,
// a 2-minute context; SGLang-Omni cookbook page, "Known limitations": the backbone and
// its KV cache run in bfloat16).
//
// One step, four kernels on the caller's stream:
//   qkv GEMV         qkv = W_qkv u (the mixer's GEMV kernels with a plain epilogue)
//   attn_split       per (64-position chunk, key/value head, session): the chunk's scores
//                    for every query head of the group, their softmax terms relative to
//                    the chunk maximum, and the weighted sum of the chunk's values; the new
//                    key and value (rounded to bf16) stand in for the cache row at the
//                    session's position and are stored there by the chunk that holds it
//   attn_combine     per (query head, session): rescales the chunk partials to the common
//                    maximum, normalises, and advances the session's position (chunks past
//                    the session's length are marked empty by attn_split)
//   o GEMV           y = W_o o (+ u)
// Scores are kept in log2 units (q pre-scaled by log2(e)/sqrt(D)) so that every
// exponential is one exp2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "lanes.h"
#include "m2_internal.h"

namespace m2d {
namespace {

constexpr int kC = 64;      // cache positions per split workgroup
constexpr int kT = 256;     // threads per split workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const float *qkv;         // [B][(Hq + 2 Hk) D]
  uint16_t *kc, *vc;        // [n_slots][Hk][max_len][D] bf16 bits
  int32_t *pos;             // [n_slots]
  const int32_t *slots;     // [B] or null (session b uses slot b)
  int n_slots, B, Hq, Hk, max_len, nsplit;
  float scale;              // log2(e) / sqrt(D)
  float *part_o;            // [B][Hq][nsplit][D]: sum over the chunk of 2^(s_j - m) v_j
  float2 *part_ml;          // [B][Hq][nsplit]: (m, sum over the chunk of 2^(s_j - m))
  int *lens;                // [B]: positions attended (pos + 1), -1 for a session not run
  float *o;                 // [B][Hq D]
};

// bf16 bits of the nearest value (ties to even); NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Scores on the matrix cores: wave w takes the chunk's positions 16w .. 16w + 15 as the A
// operand of bf16 16x16x32 MFMAs (lane l holds 8 dimensions of position l % 16, octet l / 16,
// loaded straight from the cache) and the group's queries as the B operand (head l % 16, the
// same octet), split into bf16 hi and lo parts (q = hi + lo to 2^-16 relative; keys are exact
// in bf16), two MFMAs per 32-dimension step; the product tile gives head l % 16 the scores
// of positions 4 (l / 16) + r in register r. Values: each wave takes positions w, w + 4, ...
// and each lane D/64 dimensions of a row, so a load instruction reads one whole row and the
// weighted sum over positions stays in the lane. Every cache load is issued first.
template <int D, int HPG>
__global__ __launch_bounds__(kT) void attn_split_kernel(AttnArgs a) {
  constexpr int WPB = kT / 64, KS = D / 32;
  constexpr int DPL = D / 64, VPW = kC / WPB;
  static_assert(kC == 16 * WPB && HPG <= 16, "layout");
  constexpr int QLD = D + 8;                         // padded row: 16 lanes hit distinct banks
  __shared__ float sc[HPG][kC];
  __shared__ float red[WPB][HPG][D];
  __shared__ float2 ml[HPG];
  __shared__ unsigned short qhl[2][16][QLD];          // scaled queries as bf16 hi and lo, rows >= HPG zero
  __shared__ unsigned short kns[D];                   // the new key in bf16

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = a.slots ? a.slots[b] : b;
  const bool sok = slot >= 0 && slot < a.n_slots;
  const int p = sok ? a.pos[slot] : -1;
  const bool live = sok && p >= 0 && p < a.max_len;
  if (split == 0 && g == 0 && tid == 0) a.lens[b] = live ? p + 1 : -1;
  const int j0 = split * kC;
  if (!live) return;                                 // uniform over the workgroup
  if (j0 > p) {                                      // a chunk past the session's length: empty
    if (tid < HPG) a.part_ml[((size_t)b * a.Hq + (size_t)g * HPG + tid) * a.nsplit + split] = make_float2(-INFINITY, 0.0f);
    return;
  }

  const size_t cache_off = ((size_t)slot * a.Hk + g) * (size_t)a.max_len * D;
  const uint16_t *kg = a.kc + cache_off;
  const uint16_t *vg = a.vc + cache_off;
  const int r16 = lane & 15, oct = lane >> 4;
  const int jk = j0 + 16 * wave + r16;               // this lane's key row
  u32x4v kr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kr[ks] = *reinterpret_cast<const u32x4v *>(kg + (size_t)min(jk, p) * D + 32 * ks + 8 * oct);
  uint32_t vr[VPW];
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int j = min(j0 + wave + WPB * i, p);
    const uint16_t *vp = vg + (size_t)j * D + lane * DPL;
    vr[i] = DPL == 2 ? *reinterpret_cast<const uint32_t *>(vp) : (uint32_t)*vp;
  }
  const float *qkv = a.qkv + (size_t)b * (a.Hq + 2 * a.Hk) * D;
  const float *kn = qkv + (size_t)(a.Hq + g) * D;                   // the new key
  const float *vnl = qkv + (size_t)(a.Hq + a.Hk + g) * D + lane * DPL;   // the new value, this lane's dims
  // queries split by truncation (hi = the top 16 bits, lo = the top 16 bits of the rest:
  // q = hi + lo to 2^-16 relative), the new key rounded to nearest even as it is stored
  for (int i = tid; i < 16 * D; i += kT) {
    const int h = i / D, d = i - h * D;
    const float v = h < HPG ? qkv[(size_t)(g * HPG + h) * D + d] * a.scale : 0.0f;
    const uint32_t hb = __float_as_uint(v) & 0xFFFF0000u;
    qhl[0][h][d] = (unsigned short)(hb >> 16);
    qhl[1][h][d] = (unsigned short)(__float_as_uint(v - __uint_as_float(hb)) >> 16);
  }
  for (int i = tid; i < D; i += kT) kns[i] = (unsigned short)to_bf16(kn[i]);
  __syncthreads();
  bf16x8 qhi[KS], qlo[KS];
  u32x4v knew[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qhi[ks] = *reinterpret_cast<const bf16x8 *>(&qhl[0][r16][32 * ks + 8 * oct]);
    qlo[ks] = *reinterpret_cast<const bf16x8 *>(&qhl[1][r16][32 * ks + 8 * oct]);
    knew[ks] = *reinterpret_cast<const u32x4v *>(&kns[32 * ks + 8 * oct]);
  }
  float vfresh[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) vfresh[e] = __uint_as_float(to_bf16(vnl[e]) << 16);

  // scores: rows at and past p take the new key (finite; past p they are masked)
  f32x4v c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4v kk = jk >= p ? knew[ks] : kr[ks];
    const bf16x8 av = __builtin_bit_cast(bf16x8, kk);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qhi[ks], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qlo[ks], c, 0, 0, 0);
  }
  if (r16 < HPG) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jl = 16 * wave + 4 * oct + r;
      sc[r16][jl] = j0 + jl <= p ? c[r] : -INFINITY;
    }
  }
  __syncthreads();

  // per head: the chunk maximum, the terms 2^(s - m) and their sum (one wave per head)
  for (int h = wave; h < HPG; h += WPB) {
    const float s = sc[h][lane];
    const float m = group_reduce<64, true>(s);
    const float e = exp2f(s - m);
    const float l = group_reduce<64>(e);
    sc[h][lane] = e;
    if (lane == 0) ml[h] = make_float2(m, l);
  }
  __syncthreads();

  // weighted values: the lane's DPL dimensions over the wave's positions, then over the waves
  float acc[HPG][DPL];
#pragma unroll
  for (int h = 0; h < HPG; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.0f;
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int jl = wave + WPB * i, j = j0 + jl;
    float vf[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float c = __uint_as_float(e == 0 ? vr[i] << 16 : vr[i] & 0xFFFF0000u);
      vf[e] = j >= p ? vfresh[e] : c;             // the new row at p; past p (weight 0) also finite
    }
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const float w = sc[h][jl];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(w, vf[e], acc[h][e]);
    }
  }
#pragma unroll
  for (int h = 0; h < HPG; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) red[wave][h][lane * DPL + e] = acc[h][e];
  __syncthreads();
  const size_t hq0 = (size_t)b * a.Hq + (size_t)g * HPG;
  for (int i = tid; i < HPG * D; i += kT) {
    const int h = i / D, d = i % D;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WPB; ++w) v += red[w][h][d];
    a.part_o[((hq0 + h) * a.nsplit + split) * D + d] = v;
  }
  if (tid < HPG) a.part_ml[(hq0 + tid) * a.nsplit + split] = ml[tid];
  // the chunk holding the session's position stores the new key (the lanes whose key row
  // is p, 8 dimensions per step each) and the new value (wave 0, D/64 dimensions per lane)
  if (jk == p) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      *reinterpret_cast<u32x4v *>(a.kc + cache_off + (size_t)p * D + 32 * ks + 8 * oct) = knew[ks];
  }
  if (p < j0 + kC && wave == 0) {
    uint32_t vb = 0;
#pragma unroll
    for (int e = 0; e < DPL; ++e) vb |= (__float_as_uint(vfresh[e]) >> 16) << (16 * e);
    if (DPL == 2)
      *reinterpret_cast<uint32_t *>(a.vc + cache_off + (size_t)p * D + lane * 2) = vb;
    else
      a.vc[cache_off + (size_t)p * D + lane] = (uint16_t)vb;
  }
}

// One workgroup of D threads per (query head, session). The chunk statistics are copied to
// LDS with one vector load per thread and this thread's dimension of the first 32 chunks'
// partials is requested in the same round trip; chunks past the session's length carry
// m = -inf and are skipped by selection, so their stale partials never enter. The session's
// length is needed only at the end.
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs a) {
  constexpr int NB = 32;
  __shared__ float2 mls[1024];                     // nsplit <= 1024 (max_len <= 65536)
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = a.lens[b];
  const size_t hq = (size_t)b * a.Hq + h;
  const float2 *ml = a.part_ml + hq * a.nsplit;
  const float *po = a.part_o + hq * a.nsplit * D + d;
  const int ns = a.nsplit;
  float v[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) v[i] = po[(size_t)min(i, ns - 1) * D];
  for (int s = d; s < ns; s += D) mls[s] = ml[s];
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, mls[s].x);
  float l = 0.0f, acc = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += NB) {
    if (s0 > 0)
#pragma unroll
      for (int i = 0; i < NB; ++i) v[i] = po[(size_t)min(s0 + i, ns - 1) * D];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float2 e = mls[min(s0 + i, ns - 1)];
      const bool use = s0 + i < ns && e.x != -INFINITY;
      const float w = exp2f(e.x - M);
      l = use ? fmaf(w, e.y, l) : l;
      acc = use ? fmaf(w, v[i], acc) : acc;
    }
  }
  float *o = a.o + hq * D;
  o[d] = L < 0 ? __builtin_nanf("") : acc / l;
  if (L >= 0 && h == 0 && d == 0) a.pos[a.slots ? a.slots[b] : b] = L;
}

template <int D, int HPG>
hipError_t launch_split(const AttnArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_split_kernel<D, HPG>), dim3(a.nsplit, a.Hk, a.B), dim3(kT), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const AttnArgs &a, int hpg, hipStream_t stream) {
  switch (hpg) {
    case 1: return launch_split<D, 1>(a, stream);
    case 2: return launch_split<D, 2>(a, stream);
    case 3: return launch_split<D, 3>(a, stream);
    case 4: return launch_split<D, 4>(a, stream);
    case 5: return launch_split<D, 5>(a, stream);
    case 6: return launch_split<D, 6>(a, stream);
    case 7: return launch_split<D, 7>(a, stream);
    default: return launch_split<D, 8>(a, stream);
  }
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct AttnWs {
  float *qkv, *o, *part_o, *gemv_part;
  float2 *part_ml;
  int *lens;
  size_t bytes;
};

AttnWs attn_ws_layout(const m2_attn_s &A, int B, void *base) {
  const m2_attn_config &c = A.cfg;
  char *p = static_cast<char *>(base);
  AttnWs w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    char *r = p ? p + off : nullptr;
    off += al256(n);
    return r;
  };
  w.qkv = reinterpret_cast<float *>(take(sizeof(float) * (size_t)B * A.qkv_rows));
  w.o = reinterpret_cast<float *>(take(sizeof(float) * (size_t)B * A.o_dim));
  w.part_o = reinterpret_cast<float *>(take(sizeof(float) * (size_t)B * c.n_q * A.nsplit * c.head_dim));
  w.part_ml = reinterpret_cast<float2 *>(take(sizeof(float2) * (size_t)B * c.n_q * A.nsplit));
  w.lens = reinterpret_cast<int *>(take(sizeof(int) * (size_t)B));
  const size_t gp = std::max(gemv_plain_part_bytes(c.wtype, c.q_group, A.qkv_rows, c.d_model, B),
                             gemv_plain_part_bytes(c.wtype, c.q_group, c.d_model, A.o_dim, B));
  w.gemv_part = gp ? reinterpret_cast<float *>(take(gp)) : nullptr;
  w.bytes = off;
  return w;
}

}  // namespace

int attn_nsplit(int max_len) { return (max_len + kC - 1) / kC; }

size_t attn_ws_bytes(const m2_attn_s &A, int batch) { return attn_ws_layout(A, batch, nullptr).bytes; }

hipError_t launch_attn_step(const m2_attn_s &A, uint16_t *kc, uint16_t *vc, int32_t *pos, int n_slots,
                            const float *x, float *y, int batch, const int32_t *slots, int flags, void *ws,
                            hipStream_t stream, hipEvent_t const *events) {
  const m2_attn_config &c = A.cfg;
  auto mark = [&](int i) -> hipError_t {
    return (events && events[i]) ? hipEventRecord(events[i], stream) : hipSuccess;
  };
  const AttnWs w = attn_ws_layout(A, batch, ws);
  hipError_t e = mark(0);
  if (e == hipSuccess)
    e = launch_gemv_plain(c.wtype, A.w.w_qkv, A.w.s_qkv, A.qkv_rows, c.d_model, c.q_group, c.q_gamma_qkv, x,
                          batch, w.qkv, nullptr, w.gemv_part, stream);
  if (e == hipSuccess) e = mark(1);
  if (e != hipSuccess) return e;
  AttnArgs a{};
  a.qkv = w.qkv;
  a.kc = kc;
  a.vc = vc;
  a.pos = pos;
  a.slots = slots;
  a.n_slots = n_slots;
  a.B = batch;
  a.Hq = c.n_q;
  a.Hk = c.n_kv;
  a.max_len = c.max_len;
  a.nsplit = A.nsplit;
  a.scale = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  a.part_o = w.part_o;
  a.part_ml = w.part_ml;
  a.lens = w.lens;
  a.o = w.o;
  const int hpg = c.n_q / c.n_kv;
  e = c.head_dim == 128 ? launch_split_d<128>(a, hpg, stream) : launch_split_d<64>(a, hpg, stream);
  if (e == hipSuccess) e = mark(2);
  if (e != hipSuccess) return e;
  if (c.head_dim == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(c.n_q, batch), dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(c.n_q, batch), dim3(64), 0, stream, a);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess)
    e = launch_gemv_plain(c.wtype, A.w.w_o, A.w.s_o, c.d_model, A.o_dim, c.q_group, c.q_gamma_o, w.o, batch, y,
                          (flags & M2_RESIDUAL) ? x : nullptr, w.gemv_part, stream);
  if (e == hipSuccess) e = mark(4);
  return e;
}

}  // namespace m2d
