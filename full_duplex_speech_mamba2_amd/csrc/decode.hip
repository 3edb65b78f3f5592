// Decode step of the Mamba-2 mixer layer on gfx950: three kernels per step.
//
//   gemv_in   zxbcdt = W_in u, weight-streaming GEMV (16-byte loads of W, fp32
//             accumulate), with the per-row epilogue fused in: causal conv +
//             SiLU and the conv-cache shift for the x|B|C rows, softplus for the
//             dt rows, the raw value for the z rows.
//   ssd_step  per (session, head, row range): S = exp(dt A) S + dt x B^T and
//             y = C.S + D x on the state tile held in registers (one read, one
//             write), then v = y SiLU(z) and per-range sums of squares.
//   gemv_out  RMS factors from the sums of squares, yn = v r norm_w staged into
//             LDS, then out = W_out yn (+ residual).
//
// The operation follows the Mamba-2 layer the backbone of the pages uses (page
// "NemotronLabs VoiceChat 11B: GPTQ 3-bit LLM, MLX", introduction; page
// "NemotronLabs VoiceChat" of the SGLang-Omni cookbook, introduction: one token
// per 80 ms frame). The decode step is bound by streaming the two projection
// matrices from HBM (GPTQ page, introduction: the LLM step is limited by
// memory bandwidth), so the GEMVs are built around full 16-byte coalesced loads
// with several loads in flight per lane; the rest is small.
#include <hip/hip_fp16.h>

#include "m2_internal.h"

namespace m2d {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsFloatsPerBatch = 12288;   // activation tile budget: 48 KB at batch tile 1

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ float softplus(float a) { return a > 20.0f ? a : log1pf(expf(a)); }

__device__ __forceinline__ float i8(uint32_t u, int j) {
  return (float)((int32_t)(u << (24 - 8 * j)) >> 24);
}

template <int WT> struct WTraits;
template <> struct WTraits<M2_W_F32> { static constexpr int EPC = 4; static constexpr int ESZ = 4; };
template <> struct WTraits<M2_W_BF16> { static constexpr int EPC = 8; static constexpr int ESZ = 2; };
template <> struct WTraits<M2_W_INT8G> { static constexpr int EPC = 16; static constexpr int ESZ = 1; };

// Dot product of one 16-byte weight chunk with EPC consecutive fp32 activations.
template <int WT> __device__ __forceinline__ float chunk_dot(const uint4 &w, const float *a);

template <> __device__ __forceinline__ float chunk_dot<M2_W_F32>(const uint4 &w, const float *a) {
  const float4 x = *reinterpret_cast<const float4 *>(a);
  float s = __uint_as_float(w.x) * x.x;
  s = fmaf(__uint_as_float(w.y), x.y, s);
  s = fmaf(__uint_as_float(w.z), x.z, s);
  s = fmaf(__uint_as_float(w.w), x.w, s);
  return s;
}

template <> __device__ __forceinline__ float chunk_dot<M2_W_BF16>(const uint4 &w, const float *a) {
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

template <> __device__ __forceinline__ float chunk_dot<M2_W_INT8G>(const uint4 &w, const float *a) {
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

enum { PRO_PLAIN = 0, PRO_NORM = 1 };
enum { EPI_INPROJ = 0, EPI_OUT = 1 };

struct GemvArgs {
  const void *W;          // [rows][K]
  const __half *S;        // int8 scales [rows][K / q_group]
  int rows, K, q_group;
  float gamma;
  const float *act;       // [B][K]
  int B, KT;              // sessions, activation K tile
  // RMSNorm prologue (gemv_out)
  const float *ss;        // [B][n_partials]
  const float *norm_w;    // [K]
  int ng, prange, n_partials, n_norm;
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

// One workgroup computes RPW = 16/KS rows for a tile of BT sessions. Threads
// form 16 groups of 16 lanes; group (ks, r) covers row r over the ks-th share
// of each K tile, lanes striding over 16-byte weight chunks, U chunks in flight.
template <int WT, int BT, int KS, int PRO, int EPI, int U>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  extern __shared__ float lds[];
  constexpr int RPW = 16 / KS;
  constexpr int EPC = WTraits<WT>::EPC;
  constexpr int ESZ = WTraits<WT>::ESZ;
  const int tid = threadIdx.x, lane = tid & 15, gid = tid >> 4;
  const int ks = gid / RPW, rl = gid % RPW;
  const int row = blockIdx.x * RPW + rl;
  const bool row_ok = row < a.rows;
  const int b0 = blockIdx.y * BT;
  const int nb = min(BT, a.B - b0);
  float *act_s = lds;                       // [BT][KT]
  float *rn_s = lds + BT * a.KT;            // [BT][n_norm]
  float *red_s = rn_s + (PRO == PRO_NORM ? BT * a.n_norm : 0);   // [16][BT]

  if (PRO == PRO_NORM) {
    const int per = a.ng / a.prange;
    for (int i = tid; i < nb * a.n_norm; i += kThreads) {
      const int bb = i / a.n_norm, j = i - bb * a.n_norm;
      const float *p = a.ss + (size_t)(b0 + bb) * a.n_partials + (size_t)j * per;
      float s = 0.0f;
      for (int q = 0; q < per; ++q) s += p[q];
      rn_s[bb * a.n_norm + j] = 1.0f / sqrtf(s / (float)a.ng + a.eps);
    }
    __syncthreads();
  }

  float acc[BT];
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) acc[bb] = 0.0f;

  const int ngrp = a.K / a.q_group;
  for (int kt = 0; kt < a.K; kt += a.KT) {
    const int klen = min(a.KT, a.K - kt);
    for (int i = tid; i < BT * klen; i += kThreads) {
      const int bb = i / klen, k = i - bb * klen;
      float v = 0.0f;
      if (bb < nb) {
        v = a.act[(size_t)(b0 + bb) * a.K + kt + k];
        if (PRO == PRO_NORM) v *= rn_s[bb * a.n_norm + (kt + k) / a.ng] * a.norm_w[kt + k];
      }
      act_s[bb * a.KT + k] = v;
    }
    __syncthreads();
    if (row_ok) {
      const int nch = klen / EPC;
      const int per = (nch + KS - 1) / KS;
      const int c0 = ks * per, c1 = min(nch, c0 + per);
      const uint4 *wrow =
          reinterpret_cast<const uint4 *>(static_cast<const char *>(a.W) + ((size_t)row * a.K + kt) * ESZ);
      for (int cb = c0 + lane; cb < c1; cb += 16 * U) {
        uint4 wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + 16 * u;
          wv[u] = c < c1 ? wrow[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + 16 * u;
          if (c < c1) {
            float sc = 1.0f;
            if (WT == M2_W_INT8G) sc = __half2float(a.S[(size_t)row * ngrp + (kt + c * EPC) / a.q_group]);
#pragma unroll
            for (int bb = 0; bb < BT; ++bb) {
              const float d = chunk_dot<WT>(wv[u], act_s + bb * a.KT + c * EPC);
              acc[bb] = WT == M2_W_INT8G ? fmaf(sc, d, acc[bb]) : acc[bb] + d;
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // reduce over the 16 lanes of the group (every lane ends with the total)
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc[bb] += __shfl_xor(acc[bb], off, 16);
  }
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
  if (ks != 0 || !row_ok || lane >= nb) return;

  const int b = b0 + lane;
  val *= a.gamma;
  const int slot = a.slots ? a.slots[b] : b;
  const bool sok = slot >= 0 && slot < a.n_slots;
  const float qnan = __builtin_nanf("");
  if (EPI == EPI_INPROJ) {
    float out = val;
    if (row >= a.d_inner && row < a.d_inner + a.conv_dim) {
      const int c = row - a.d_inner;
      if (!sok) {
        out = qnan;
      } else {
        float *cc = a.conv_cache + (size_t)slot * (a.d_conv - 1) * a.conv_dim + c;
        const float *w = a.conv_w + (size_t)c * a.d_conv;
        float hist[8];
        float s = a.conv_b[c];
        for (int k = 0; k < a.d_conv - 1; ++k) {
          hist[k] = cc[(size_t)k * a.conv_dim];
          s = fmaf(w[k], hist[k], s);
        }
        s = fmaf(w[a.d_conv - 1], val, s);
        for (int k = 0; k + 1 < a.d_conv - 1; ++k) cc[(size_t)k * a.conv_dim] = hist[k + 1];
        cc[(size_t)(a.d_conv - 2) * a.conv_dim] = val;
        out = silu(s);
      }
    } else if (row >= a.d_inner + a.conv_dim) {
      out = softplus(val + a.dt_bias[row - a.d_inner - a.conv_dim]);
    }
    a.zx[(size_t)b * a.zx_stride + row] = out;
  } else {
    float out = val + (a.resid ? a.resid[(size_t)b * a.rows + row] : 0.0f);
    a.y[(size_t)b * a.rows + row] = sok ? out : qnan;
  }
}

struct SsdArgs {
  const float *zx;        // [B][zx_stride]
  int zx_stride, d_inner, conv_dim, H, P, N, G, hpg;
  float *ssm;             // [n_slots][H][P][N]
  const float *A_log, *D;
  float *v;               // [B][d_inner]
  float *ss;              // [B][n_partials]
  int prange, psplit, n_partials;
  const int32_t *slots;
  int n_slots;
};

constexpr int kSsdMaxInst = 8;   // float4 row-slices per lane: prange <= 32 rows

// One workgroup = (session b, head h, rows [ps*prange, (ps+1)*prange)). A row of
// the state (N floats) is read by N/4 lanes as float4; every slice of the tile
// is loaded before any is used, updated in registers and written once.
__global__ __launch_bounds__(kThreads) void ssd_step_kernel(SsdArgs a) {
  const int h = blockIdx.x / a.psplit, ps = blockIdx.x - h * a.psplit, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = h / a.hpg;
  const int lpr = a.N >> 2;                 // lanes per state row
  const int rpi = 64 / lpr;                 // rows per wave instruction
  const int n_inst = (a.prange + rpi - 1) / rpi;
  const int r_in = lane / lpr, q = lane - r_in * lpr;
  const float *zb = a.zx + (size_t)b * a.zx_stride;
  const int slot = a.slots ? a.slots[b] : b;
  const bool sok = slot >= 0 && slot < a.n_slots;
  const float dt = zb[a.d_inner + a.conv_dim + h];
  const float dA = expf(-expf(a.A_log[h]) * dt);
  const float Dh = a.D[h];
  const float4 Bq = reinterpret_cast<const float4 *>(zb + 2 * a.d_inner + (size_t)g * a.N)[q];
  const float4 Cq = reinterpret_cast<const float4 *>(zb + 2 * a.d_inner + (size_t)(a.G + g) * a.N)[q];
  float4 *S = reinterpret_cast<float4 *>(a.ssm + ((size_t)(sok ? slot : 0) * a.H + h) * a.P * a.N);

  float4 st[kSsdMaxInst];
  int prow[kSsdMaxInst];
#pragma unroll
  for (int k = 0; k < kSsdMaxInst; ++k) {
    const int i = wave + 4 * k;
    const int pl = i * rpi + r_in;
    prow[k] = (i < n_inst && pl < a.prange) ? ps * a.prange + pl : -1;
    st[k] = (sok && prow[k] >= 0) ? S[(size_t)prow[k] * lpr + q] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float ssacc = 0.0f;
#pragma unroll
  for (int k = 0; k < kSsdMaxInst; ++k) {
    if (wave + 4 * k >= n_inst) break;      // uniform across the wave
    const int p = prow[k];
    const float xp = p >= 0 ? zb[a.d_inner + h * a.P + p] : 0.0f;
    const float dtx = dt * xp;
    float4 s = st[k];
    s.x = fmaf(dA, s.x, dtx * Bq.x);
    s.y = fmaf(dA, s.y, dtx * Bq.y);
    s.z = fmaf(dA, s.z, dtx * Bq.z);
    s.w = fmaf(dA, s.w, dtx * Bq.w);
    st[k] = s;
    float r = s.x * Cq.x;
    r = fmaf(s.y, Cq.y, r);
    r = fmaf(s.z, Cq.z, r);
    r = fmaf(s.w, Cq.w, r);
    for (int off = lpr >> 1; off >= 1; off >>= 1) r += __shfl_xor(r, off, 64);
    if (q == 0 && p >= 0) {
      const float yv = fmaf(Dh, xp, r);
      float vv = yv * silu(zb[h * a.P + p]);
      if (!sok) vv = __builtin_nanf("");
      a.v[(size_t)b * a.d_inner + h * a.P + p] = vv;
      ssacc = fmaf(vv, vv, ssacc);
    }
  }
  if (sok) {
#pragma unroll
    for (int k = 0; k < kSsdMaxInst; ++k)
      if (prow[k] >= 0) S[(size_t)prow[k] * lpr + q] = st[k];
  }
  // sum of squares of this workgroup's rows, in a fixed order
  for (int off = 32; off >= 1; off >>= 1) ssacc += __shfl_xor(ssacc, off, 64);
  __shared__ float wsum[4];
  if (lane == 0) wsum[wave] = ssacc;
  __syncthreads();
  if (threadIdx.x == 0)
    a.ss[(size_t)b * a.n_partials + (h * a.P + ps * a.prange) / a.prange] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
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

template <int WT, int BT, int KS, int PRO, int EPI, int U>
hipError_t launch_gemv(const GemvArgs &a, hipStream_t stream) {
  constexpr int RPW = 16 / KS;
  dim3 grid((a.rows + RPW - 1) / RPW, (a.B + BT - 1) / BT);
  size_t lds = sizeof(float) * ((size_t)BT * a.KT + (PRO == PRO_NORM ? (size_t)BT * a.n_norm : 0) + 16 * BT);
  hipLaunchKernelGGL((gemv_kernel<WT, BT, KS, PRO, EPI, U>), grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

int pick_kt(int K, int BT) {
  int kt = (kLdsFloatsPerBatch / BT) & ~255;
  return K <= kt ? K : kt;
}

template <int WT, int PRO, int EPI, int KS>
hipError_t dispatch_bt(GemvArgs a, hipStream_t stream) {
  if (a.B >= 4) {
    a.KT = pick_kt(a.K, 4);
    return launch_gemv<WT, 4, KS, PRO, EPI, 8>(a, stream);
  }
  if (a.B >= 2) {
    a.KT = pick_kt(a.K, 2);
    return launch_gemv<WT, 2, KS, PRO, EPI, 8>(a, stream);
  }
  a.KT = pick_kt(a.K, 1);
  return launch_gemv<WT, 1, KS, PRO, EPI, 8>(a, stream);
}

template <int PRO, int EPI, int KS>
hipError_t dispatch_wt(int wtype, const GemvArgs &a, hipStream_t stream) {
  switch (wtype) {
    case M2_W_F32: return dispatch_bt<M2_W_F32, PRO, EPI, KS>(a, stream);
    case M2_W_BF16: return dispatch_bt<M2_W_BF16, PRO, EPI, KS>(a, stream);
    default: return dispatch_bt<M2_W_INT8G, PRO, EPI, KS>(a, stream);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

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
  w.bytes = off;
  return w;
}

hipError_t launch_step(const m2_layer_s &L, const m2_state_s &S, const float *x, float *y, int batch,
                       const int32_t *slots, int flags, const StepWs &ws, hipStream_t stream,
                       hipEvent_t const *events) {
  const m2_config &c = L.cfg;
  auto mark = [&](int i) -> hipError_t {
    return (events && events[i]) ? hipEventRecord(events[i], stream) : hipSuccess;
  };
  hipError_t e = mark(0);
  if (e != hipSuccess) return e;
  // 1. in_proj + conv + dt
  GemvArgs gi{};
  gi.W = L.w.w_in;
  gi.S = static_cast<const __half *>(L.w.s_in);
  gi.rows = L.d_in_proj;
  gi.K = c.d_model;
  gi.q_group = c.wtype == M2_W_INT8G ? c.q_group : c.d_model;
  gi.gamma = c.wtype == M2_W_INT8G ? c.q_gamma_in : 1.0f;
  gi.act = x;
  gi.B = batch;
  gi.zx = ws.zx;
  gi.zx_stride = L.zx_stride;
  gi.d_inner = L.d_inner;
  gi.conv_dim = L.conv_dim;
  gi.d_conv = c.d_conv;
  gi.conv_w = L.w.conv_w;
  gi.conv_b = L.w.conv_b;
  gi.dt_bias = L.w.dt_bias;
  gi.conv_cache = S.conv;
  gi.slots = slots;
  gi.n_slots = S.n_slots;
  e = dispatch_wt<PRO_PLAIN, EPI_INPROJ, 1>(c.wtype, gi, stream);
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
  sa.A_log = L.w.A_log;
  sa.D = L.w.D;
  sa.v = ws.v;
  sa.ss = ws.ss;
  sa.prange = L.prange;
  sa.psplit = L.psplit;
  sa.n_partials = L.n_partials;
  sa.slots = slots;
  sa.n_slots = S.n_slots;
  hipLaunchKernelGGL(ssd_step_kernel, dim3(c.n_heads * L.psplit, batch), dim3(kThreads), 0, stream, sa);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(2);
  if (e != hipSuccess) return e;

  // 3. RMSNorm + out_proj (+ residual)
  GemvArgs go{};
  go.W = L.w.w_out;
  go.S = static_cast<const __half *>(L.w.s_out);
  go.rows = c.d_model;
  go.K = L.d_inner;
  go.q_group = c.wtype == M2_W_INT8G ? c.q_group : L.d_inner;
  go.gamma = c.wtype == M2_W_INT8G ? c.q_gamma_out : 1.0f;
  go.act = ws.v;
  go.B = batch;
  go.ss = ws.ss;
  go.norm_w = L.w.norm_w;
  go.ng = L.ng;
  go.prange = L.prange;
  go.n_partials = L.n_partials;
  go.n_norm = L.n_norm;
  go.eps = c.norm_eps;
  go.y = y;
  go.resid = (flags & M2_RESIDUAL) ? x : nullptr;
  go.slots = slots;
  go.n_slots = S.n_slots;
  e = dispatch_wt<PRO_NORM, EPI_OUT, 4>(c.wtype, go, stream);
  if (e == hipSuccess) e = mark(3);
  return e;
}

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

}  // namespace m2d
