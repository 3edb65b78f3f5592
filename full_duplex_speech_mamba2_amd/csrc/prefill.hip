// Chunked prefill of the Mamba-2 mixer layer on gfx950.
//
// A prompt of T tokens per session is processed in one pass before streaming
// starts (page "NemotronLabs VoiceChat 11B: GPTQ 3-bit LLM, MLX", "Recipe":
// system-prompt prefill, then the user's speech; page "NemotronLabs VoiceChat"
// of the SGLang-Omni cookbook, "Known limitations": the system-prompt region is
// walked before frame 0). The result equals T decode steps; the chunked form
// only reorders the arithmetic of the SSD recurrence
//     S_t = exp(dt_t A) S_{t-1} + dt_t x_t B_t^T,   y_t = C_t . S_t + D x_t
// into, per chunk of Q tokens with cs_t = sum_{r<=t in chunk} dt_r A:
//     y_t   = sum_{s<=t} (C_t.B_s) exp(cs_t - cs_s) dt_s x_s      (intra-chunk, MFMA)
//           + exp(cs_t) C_t . H_{c-1}                             (entering state, MFMA)
//           + D x_t
//     S_c   = sum_s exp(cs_end - cs_s) dt_s x_s B_s^T             (chunk state, MFMA)
//     H_c   = exp(cs_end) H_{c-1} + S_c                           (sequential over chunks)
//
// Kernels, in stream order:
//   gemm (in_proj)   ZX[BT][d_in_proj] = X W_in^T: bf16 MFMA 32x32x16, fp32 activations
//                    split into bf16 hi + lo so that bf16 weights multiply exactly
//   conv_dt          causal conv + SiLU over T (halo from the conv cache), softplus dt
//   cb               per (t-tile, chunk, group, session): C B^T tiles (f32 MFMA 16x16x4), s-tile <= t-tile
//   chunk_state      per (session, chunk, head): cumsum of dt A, S_c
//   state_pass       per (session, head): H_c recurrence; entering states; final state -> slot
//   chunk_out        per (session, chunk, head): y, gate, v * norm_w, per-head sum of squares
//   rms              RMS factor per (token, norm group)
//   gemm (out_proj)  Y = (v norm_w r) W_out^T (+ residual), same GEMM with a row-group scale on A
//   cache_update     conv cache <- last d_conv-1 raw inputs (mixing with the old cache if T is short)
// Weights stored as fp32, int8 or 4/3-bit codes use a fp32 VALU GEMM instead of the MFMA GEMM.
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include "m2_internal.h"

namespace m2d {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }
__device__ __forceinline__ float softplus(float a) { return a > 20.0f ? a : log1pf(expf(a)); }

__device__ __forceinline__ float bf16_to_f(unsigned short h) { return __uint_as_float((unsigned)h << 16); }

// ---------------------------------------------------------------------------
// MFMA GEMM: C[M][N] = A[M][K] W[N][K]^T (+ R), A fp32 (optionally scaled by
// rs[m][k / ng]), W bf16. Block tile 128 x 128 x 32, 4 waves in 2 x 2, each wave
// 64 x 64 = 2 x 2 MFMA 32x32x16 tiles, two MFMAs (hi, lo) per tile and k-step.
// LDS rows padded to 40 bf16 (80 B). Global loads of the next K tile are held in
// registers while the current tile is multiplied out of LDS.

constexpr int GBM = 128, GBN = 256, GBK = 32, GLD = 40;
constexpr int kGemmGroupM = 4;     // row tiles per group of the tile order
constexpr size_t kGemmLds = sizeof(unsigned short) * 2 * (2 * GBM + GBN) * GLD;   // 80 KB

struct GemmArgs {
  const float *A;
  int lda;
  const unsigned short *W;   // bf16 [N][K], or its 16-row panels (PANEL)
  int S;                     // panels: 32-wide k-steps per panel, ceil(K / 32)
  float *C;
  int ldc;
  const float *R;            // residual [M][ldr] or null
  int ldr;
  const float *rs;           // row-group scale [M][n_rs] or null
  int n_rs, ng;
  int M, N, K;
};

// Block tile 128 x 256, 4 waves in 2 x 2, each wave 64 x 128 = 2 x 4 MFMA 32x32x16
// tiles: per 16-wide k-step a wave reads 2 A fragments (x hi, lo) and 4 W fragments
// from LDS for 16 MFMAs. LDS (dynamic, 80 KB, so two workgroups per CU): double-
// buffered A hi, A lo [128][40] and W [256][40] bf16 (rows padded to 80 B). The next
// K tile's global loads are held in registers while the current one is multiplied.
// PANEL: W is read from its 16-row panels (m2_pack_panels), where the tile's 32 k of 16
// rows are one contiguous 1 KB (row-major, each of the 256 rows gives 64 B of a 128-byte
// line per tile).
template <bool PANEL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_bf16_kernel(GemmArgs g) {
  extern __shared__ unsigned short gsm[];
  unsigned short *sAh = gsm;                          // [2][GBM * GLD]
  unsigned short *sAl = gsm + 2 * GBM * GLD;          // [2][GBM * GLD]
  unsigned short *sW = gsm + 4 * GBM * GLD;           // [2][GBN * GLD]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Tile order. Workgroup ids are dealt to the 8 XCDs in turn (id % 8), each XCD with its
  // own L2: XCD x takes the x-th contiguous range of a grouped tile order, which walks
  // groups of kGemmGroupM row tiles across all column tiles, so that the workgroups
  // resident on one XCD at a time share the A rows and W columns they stream through L2.
  const int nbn = (g.N + GBN - 1) / GBN, nbm = (g.M + GBM - 1) / GBM;
  const int T = nbn * nbm, id = blockIdx.x;
  const int xcd = id & 7, per = T >> 3, rem = T & 7;
  const int v = xcd * per + min(xcd, rem) + (id >> 3);
  const int gsz = kGemmGroupM * nbn, grp = v / gsz, first = grp * kGemmGroupM;
  const int gm = min(kGemmGroupM, nbm - first), w = v - grp * gsz;
  const int m0 = (first + w % gm) * GBM, n0 = (w / gm) * GBN;
  // A loader: row lr, 16 consecutive k from lk; W loader: row tid, all 32 k. Rows past
  // the matrix are read from its last row (their results are never stored); K % 16 == 0,
  // so a 16-wide (A) or 8-wide (W) group lies wholly inside or wholly past K: a group
  // past K is read from the last group and zeroed when stored to LDS. No branches, so
  // the next tile's loads stay in flight while the current tile is multiplied.
  const int lr = tid >> 1, lk = (tid & 1) * 16;
  const int am = min(m0 + lr, g.M - 1), wnr = min(n0 + tid, g.N - 1);
  const float *arow = g.A + (size_t)am * g.lda;
  const unsigned short *wrow = g.W + (size_t)wnr * g.K;
  const float *rsrow = g.rs ? g.rs + (size_t)am * g.n_rs : nullptr;

  f32x4 ra[4];
  u32x4 rw[4];
  float rsc = 1.0f;
  auto load_tile = [&](int k0) {
    const int ka = min(k0 + lk, g.K - 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) ra[q] = *reinterpret_cast<const f32x4 *>(arow + ka + 4 * q);
    // the out_proj scale per (row, norm group): one group covers the 16 values (ng % 16 == 0)
    if (rsrow) rsc = rsrow[ka / g.ng];
    if constexpr (PANEL) {
      static_assert(GBK == 32 && GBN == 256, "one k-step of 16 panels per tile");
      // fragment f = tid + 256 q: panel f / 64 of the tile (past the matrix: its last
      // panel, whose results are never stored), lane f % 64 of the tile's k-step; the
      // panels are zero past K
      const int npan = (g.N + 15) / 16, s = k0 >> 5;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = tid + 256 * q, p = min(n0 / 16 + (f >> 6), npan - 1);
        rw[q] = *reinterpret_cast<const u32x4 *>(g.W + (((size_t)p * g.S + s) * 64 + (f & 63)) * 8);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) rw[q] = *reinterpret_cast<const u32x4 *>(wrow + min(k0 + 8 * q, g.K - 8));
    }
  };
  auto store_tile = [&](int buf, int k0) {
    // hi = bf16(v), lo = bf16(v - hi), both rounded to nearest even (packed converts)
    const bool a_in = k0 + lk < g.K;
    bf16x8 *ph = reinterpret_cast<bf16x8 *>(&sAh[buf * GBM * GLD + lr * GLD + lk]);
    bf16x8 *pl = reinterpret_cast<bf16x8 *>(&sAl[buf * GBM * GLD + lr * GLD + lk]);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f32x8 v = {ra[2 * q].x, ra[2 * q].y, ra[2 * q].z, ra[2 * q].w,
                 ra[2 * q + 1].x, ra[2 * q + 1].y, ra[2 * q + 1].z, ra[2 * q + 1].w};
      v = a_in ? v * rsc : f32x8{};
      const bf16x8 h = __builtin_convertvector(v, bf16x8);
      ph[q] = h;
      pl[q] = __builtin_convertvector(v - __builtin_convertvector(h, f32x8), bf16x8);
    }
    if constexpr (PANEL) {
      // fragment lane l holds row l % 16 of its panel, k 8 (l / 16) .. + 7
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = tid + 256 * q, row = 16 * (f >> 6) + (f & 15), col = 8 * ((f & 63) >> 4);
        *reinterpret_cast<u32x4 *>(&sW[buf * GBN * GLD + row * GLD + col]) = rw[q];
      }
    } else {
      u32x4 *pw = reinterpret_cast<u32x4 *>(&sW[buf * GBN * GLD + tid * GLD]);
#pragma unroll
      for (int q = 0; q < 4; ++q) pw[q] = k0 + 8 * q < g.K ? rw[q] : u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nk = (g.K + GBK - 1) / GBK;
  load_tile(0);
  store_tile(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * GBK);
    const unsigned short *bAh = sAh + buf * GBM * GLD, *bAl = sAl + buf * GBM * GLD, *bW = sW + buf * GBN * GLD;
#pragma unroll
    for (int ks = 0; ks < GBK; ks += 16) {
      const int kofs = ks + (lane >> 5) * 8;
      bf16x8 ah[2], al[2], bw[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        ah[i] = *reinterpret_cast<const bf16x8 *>(&bAh[r * GLD + kofs]);
        al[i] = *reinterpret_cast<const bf16x8 *>(&bAl[r * GLD + kofs]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + j * 32 + (lane & 31);
        bw[j] = *reinterpret_cast<const bf16x8 *>(&bW[r * GLD + kofs]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bw[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bw[j], acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) store_tile(buf ^ 1, (kt + 1) * GBK);
    __syncthreads();
  }
  // epilogue: lane l, reg r -> row (r/4)*8 + (l/32)*4 + r%4, col l%32 of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < g.M) {
          float v = acc[i][j][r];
          if (g.R) v += g.R[(size_t)row * g.ldr + col];
          g.C[(size_t)row * g.ldc + col] = v;
        }
      }
    }
}

// ---------------------------------------------------------------------------
// fp32 VALU GEMM for weights stored as fp32 or int8 (and any shape): 64 x 64
// tiles, 256 threads, 4 x 4 outputs per thread, K tiles of 16 in LDS.
struct GemmValuArgs {
  const float *A;
  int lda;
  const void *W;             // [N][K] fp32, bf16 or int8
  const __half *S;           // int8 scales [N][K / q_group]
  int wtype, q_group;
  float gamma;
  float *C;
  int ldc;
  const float *R;
  int ldr;
  const float *rs;
  int n_rs, ng;
  int M, N, K;
};

__device__ __forceinline__ float weight_at(const GemmValuArgs &g, int n, int k) {
  if (g.wtype == M2_W_F32) return static_cast<const float *>(g.W)[(size_t)n * g.K + k];
  if (g.wtype == M2_W_BF16) return bf16_to_f(static_cast<const unsigned short *>(g.W)[(size_t)n * g.K + k]);
  if (g.wtype == M2_W_INT8G) {
    const float q = (float)static_cast<const int8_t *>(g.W)[(size_t)n * g.K + k];
    return q * __half2float(g.S[(size_t)n * (g.K / g.q_group) + k / g.q_group]);
  }
  // low-bit codes: 4-bit two per byte (even code low), 3-bit 32 per 12-byte little-endian run
  const unsigned char *row = static_cast<const unsigned char *>(g.W);
  unsigned code;
  if (g.wtype == M2_W_INT4G) {
    const unsigned byte = row[(size_t)n * (g.K / 2) + k / 2];
    code = (k & 1) ? byte >> 4 : byte & 15u;
  } else {
    const unsigned char *run = row + (size_t)n * (g.K / 32) * 12 + (k / 32) * 12;
    const int bit = 3 * (k & 31), b = bit >> 3;
    const unsigned v = run[b] | (b < 11 ? (unsigned)run[b + 1] << 8 : 0u);
    code = (v >> (bit & 7)) & 7u;
  }
  const __half2 sm = reinterpret_cast<const __half2 *>(g.S)[(size_t)n * (g.K / g.q_group) + k / g.q_group];
  return fmaf(__low2float(sm), (float)code, __high2float(sm));
}

__global__ __launch_bounds__(256) void gemm_valu_kernel(GemmValuArgs g) {
  __shared__ float sA[16][65];
  __shared__ float sB[16][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    for (int i = tid; i < 64 * 16; i += 256) {
      const int r = i >> 4, k = i & 15;
      const int m = m0 + r, n = n0 + r, kk = k0 + k;
      float a = 0.0f, b = 0.0f;
      if (m < g.M && kk < g.K) {
        a = g.A[(size_t)m * g.lda + kk];
        if (g.rs) a *= g.rs[(size_t)m * g.n_rs + kk / g.ng];
      }
      if (n < g.N && kk < g.K) b = weight_at(g, n, kk);
      sA[k][r] = a;
      sB[k][r] = b;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = sB[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < g.M && n < g.N) {
        float v = acc[i][j] * g.gamma;
        if (g.R) v += g.R[(size_t)m * g.ldr + n];
        g.C[(size_t)m * g.ldc + n] = v;
      }
    }
}

// ---------------------------------------------------------------------------
struct ScanArgs {
  int B, T, Q, nch;                 // sessions, tokens, chunk length, chunks
  int H, P, N, G, hpg;
  int d_inner, conv_dim, d_conv, zx_stride;
  const float *zx;                  // [B*T][zx_stride]: z | raw x|B|C | raw dt (in_proj output)
  float *xc;                        // [B*T][conv_dim]: conv + SiLU
  float *dt;                        // [B*T][H]: softplus(dt_raw + bias)
  float *cs;                        // [B*T][H]: cumsum of dt A within the chunk
  float *cse;                       // [B][nch][H]: chunk-end cumsum
  float *sc;                        // [B][nch][H][P][N]: chunk states, then entering states
  float *cbt;                       // [B][nch][G][npair][64][4]: C B^T tiles
  float *vw;                        // [B*T][d_inner]: v * norm_w
  float *ssh;                       // [B*T][H]: per-head sum of squares of v
  float *rn;                        // [B*T][n_norm]
  int n_norm, ng;
  float eps;
  const float *conv_w, *conv_b, *dt_bias, *A_log, *D, *norm_w;
  float *ssm;                       // [n_slots][H][P][N]
  float *conv;                      // [n_slots][d_conv-1][conv_dim]
  const int32_t *slots;
  int n_slots;
};

__device__ __forceinline__ int slot_of(const ScanArgs &a, int b, bool &ok) {
  const int s = a.slots ? a.slots[b] : b;
  ok = s >= 0 && s < a.n_slots;
  return ok ? s : 0;
}

// conv over T with the cache as left halo, SiLU; softplus dt. A thread owns one
// channel of one session over a segment of kConvSeg tokens and slides a register
// window of the last d_conv - 1 raw inputs along it, so every raw input is read once
// (plus a d_conv - 1 halo per segment). grid: (channel blocks of conv_dim + H, B,
// segments of T).
constexpr int kConvSeg = 64;
constexpr int kMaxConv = 8;

__global__ __launch_bounds__(256) void conv_dt_kernel(ScanArgs a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  const int t0 = blockIdx.z * kConvSeg, t1 = min(a.T, t0 + kConvSeg);
  if (c >= a.conv_dim + a.H) return;
  bool ok;
  const int slot = slot_of(a, b, ok);
  const size_t row0 = (size_t)b * a.T;
  if (c >= a.conv_dim) {
    const int h = c - a.conv_dim;
    const float bias = a.dt_bias[h];
    for (int t = t0; t < t1; ++t)
      a.dt[(row0 + t) * a.H + h] = softplus(a.zx[(row0 + t) * a.zx_stride + a.d_inner + a.conv_dim + h] + bias);
    return;
  }
  const int K = a.d_conv;
  float w[kMaxConv], win[kMaxConv];                 // win[k]: the input k steps before t (k = 1 .. K-1)
#pragma unroll
  for (int k = 0; k < kMaxConv; ++k) w[k] = k < K ? a.conv_w[(size_t)c * K + k] : 0.0f;
  const float bias = a.conv_b[c];
#pragma unroll
  for (int k = 1; k < kMaxConv; ++k) {
    float v = 0.0f;
    if (k < K) {
      const int tau = t0 - k;
      v = tau >= 0 ? a.zx[(row0 + tau) * a.zx_stride + a.d_inner + c]
                   : a.conv[((size_t)slot * (K - 1) + (K - 1 + tau)) * a.conv_dim + c];
    }
    win[k] = v;
  }
  // 8 tokens at a time: their loads are issued together
  constexpr int TB = 8;
  for (int tb = t0; tb < t1; tb += TB) {
    float in[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j)
      in[j] = tb + j < t1 ? a.zx[(row0 + tb + j) * a.zx_stride + a.d_inner + c] : 0.0f;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if (tb + j >= t1) break;
      // tap K-1 multiplies the newest input, tap K-1-k the input k steps back
      float s = fmaf(w[K - 1], in[j], bias);
#pragma unroll
      for (int k = 1; k < kMaxConv; ++k)
        if (k < K) s = fmaf(w[K - 1 - k], win[k], s);
      a.xc[(row0 + tb + j) * a.conv_dim + c] = ok ? silu(s) : __builtin_nanf("");
#pragma unroll
      for (int k = kMaxConv - 1; k > 1; --k) win[k] = win[k - 1];
      win[1] = in[j];
    }
  }
}

__device__ __forceinline__ int npairs(int nt) { return nt * (nt + 1) / 2; }
// tile pair (si <= ti) -> index, row-major over ti
__device__ __forceinline__ int pair_index(int si, int ti) { return ti * (ti + 1) / 2 + si; }

// C B^T tiles: CBT[s][t] = sum_n B_s[n] C_t[n] for 16 x 16 tiles with s-tile <= t-tile,
// stored in MFMA accumulator order (lane l, reg r -> s = 16 si + 4 (l/16) + r,
// t = 16 ti + l % 16). One workgroup per (t-tile, chunk, group, session), its 4 waves
// striding over the s-tiles. The k index of the 16x16x4 MFMA runs over n in the order
// that makes each lane read 4 consecutive n of its row with one 16-byte load (lane group
// j = l/16 takes n = 16 kb + 4 j + e at k-step (kb, e)), so a load instruction covers 16
// rows x 64 contiguous bytes.
__global__ __launch_bounds__(256) void cb_kernel(ScanArgs a) {
  const int ti = blockIdx.x, c = blockIdx.y, g = blockIdx.z % a.G, b = blockIdx.z / a.G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = c * a.Q;
  const int Qc = min(a.Q, a.T - t0);
  if (16 * ti >= Qc) return;
  const int np = npairs(a.Q / 16);
  const size_t rowbase = (size_t)b * a.T + t0;
  const int j4 = 4 * (lane >> 4);
  const int t = 16 * ti + (lane & 15);
  const bool t_ok = t < Qc;
  const float *ct = a.xc + (rowbase + (t_ok ? t : 0)) * a.conv_dim + a.d_inner + a.G * a.N + g * a.N + j4;
  float *out = a.cbt + (((size_t)b * a.nch + c) * a.G + g) * (size_t)np * 256;
  for (int si = wave; si <= ti; si += 4) {
    const int s = 16 * si + (lane & 15);
    const bool s_ok = s < Qc;
    const float *bs = a.xc + (rowbase + (s_ok ? s : 0)) * a.conv_dim + a.d_inner + g * a.N + j4;
    f32x4 acc = {};
    for (int kb = 0; kb < a.N; kb += 16) {
      const f32x4 bv = s_ok ? *reinterpret_cast<const f32x4 *>(bs + kb) : f32x4{};
      const f32x4 cv = t_ok ? *reinterpret_cast<const f32x4 *>(ct + kb) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[e], cv[e], acc, 0, 0, 0);
    }
    reinterpret_cast<f32x4 *>(out)[(size_t)pair_index(si, ti) * 64 + lane] = acc;
  }
}

// Per (session, chunk, head): cs (inclusive cumsum of dt A), chunk-end cumsum, and
// the chunk state S_c[p][n] = sum_s exp(cs_end - cs_s) dt_s x_s[p] B_s[n].
// One wave per 16-row p-tile (P/16 waves); B of the chunk is staged in LDS and x is
// read from global one k-step ahead. LDS: bs [Q][N + 4], w [Q], cs [Q].
template <int NT>
__global__ __launch_bounds__(512) void chunk_state_kernel(ScanArgs a) {
  extern __shared__ float lds[];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x;
  const int g = h / a.hpg;
  const int t0 = c * a.Q;
  const int Qc = min(a.Q, a.T - t0);
  const int NN = a.N + 4;
  float *bs = lds;
  float *ws = bs + (size_t)a.Q * NN;
  float *css = ws + a.Q;
  const size_t rowbase = (size_t)b * a.T + t0;
  const float A = -expf(a.A_log[h]);
  // inclusive scan of dt A over the chunk (Hillis-Steele in LDS); Q <= 4 * nthr
  for (int s = tid; s < a.Q; s += nthr) css[s] = s < Qc ? a.dt[(rowbase + s) * a.H + h] * A : 0.0f;
  __syncthreads();
  for (int off = 1; off < a.Q; off <<= 1) {
    float v[4];
    int n = 0;
    for (int s = tid; s < a.Q; s += nthr) v[n++] = s >= off ? css[s - off] : 0.0f;
    __syncthreads();
    n = 0;
    for (int s = tid; s < a.Q; s += nthr) css[s] += v[n++];
    __syncthreads();
  }
  const float cend = css[Qc - 1];
  for (int s = tid; s < a.Q; s += nthr) {
    float w = 0.0f;
    if (s < Qc) {
      a.cs[(rowbase + s) * a.H + h] = css[s];
      w = expf(cend - css[s]) * a.dt[(rowbase + s) * a.H + h];
    }
    ws[s] = w;
  }
  if (tid == 0) a.cse[((size_t)b * a.nch + c) * a.H + h] = cend;
  const int boff = a.d_inner + g * a.N;
  const int n4 = a.N / 4;
  for (int i = tid; i < a.Q * n4; i += nthr) {
    const int s = i / n4, q = i - s * n4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s < Qc) v = *reinterpret_cast<const float4 *>(a.xc + (rowbase + s) * a.conv_dim + boff + 4 * q);
    *reinterpret_cast<float4 *>(bs + s * NN + 4 * q) = v;
  }
  __syncthreads();
  // wave = p-tile i; k index of lane group l/16 at step kk of block s0 is s = s0 + 4 (l/16) + kk
  const int p = 16 * wave + (lane & 15);
  const float *xcol = a.xc + rowbase * a.conv_dim + h * a.P + p;
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{};
  float xa[4], xn[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int s = 4 * (lane >> 4) + kk;
    xa[kk] = s < Qc ? xcol[(size_t)s * a.conv_dim] : 0.0f;
  }
  for (int s0 = 0; s0 < Qc; s0 += 16) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int s = s0 + 16 + 4 * (lane >> 4) + kk;
      xn[kk] = s < Qc ? xcol[(size_t)s * a.conv_dim] : 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int s = s0 + 4 * (lane >> 4) + kk;
      const float av = xa[kk] * ws[s];
      const float *brow = bs + s * NN + (lane & 15);
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, brow[16 * j], acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xa[kk] = xn[kk];
  }
  // lane l, reg r -> p = 16 wave + 4 (l/16) + r, n = 16 j + l % 16
  float *out = a.sc + (((size_t)b * a.nch + c) * a.H + h) * (size_t)a.P * a.N;
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
        out[(size_t)(16 * wave + 4 * (lane >> 4) + r) * a.N + 16 * j + (lane & 15)] = acc[j][r];
}

// The same for all heads of a group at once (one workgroup per (session, chunk,
// group), 8 waves): the group's B chunk is staged in LDS once instead of once per
// head. Each wave scans dt A of its heads (4 tokens per lane, prefix over the wave by
// shuffles) into the weights w[head][s] = exp(cs_end - cs_s) dt_s, then the waves take
// (head, p-tile) tasks in turn. LDS: bs [Q][N + 4], w [hpg][Q].
template <int NT>
__global__ __launch_bounds__(512) void chunk_state_group_kernel(ScanArgs a) {
  extern __shared__ float lds[];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = c * a.Q;
  const int Qc = min(a.Q, a.T - t0);
  const int NN = a.N + 4;
  float *bs = lds;
  float *ws = bs + (size_t)a.Q * NN;
  const size_t rowbase = (size_t)b * a.T + t0;
  // 1. per head: inclusive cumsum of dt A (Q <= 256: 4 tokens per lane)
  for (int hh = wave; hh < a.hpg; hh += 8) {
    const int h = g * a.hpg + hh;
    const float A = -expf(a.A_log[h]);
    float v[4], dtv[4];
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * lane + i;
      dtv[i] = s < Qc ? a.dt[(rowbase + s) * a.H + h] : 0.0f;
      run += dtv[i] * A;
      v[i] = run;
    }
    float pre = run;   // inclusive prefix of the lane totals
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(pre, off, 64);
      if (lane >= off) pre += o;
    }
    const float base = pre - run;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += base;
    const int le = (Qc - 1) >> 2, ie = (Qc - 1) & 3;
    float ve = v[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) if (ie == i) ve = v[i];
    const float cend = __shfl(ve, le, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * lane + i;
      if (s < a.Q) ws[hh * a.Q + s] = s < Qc ? expf(cend - v[i]) * dtv[i] : 0.0f;
      if (s < Qc) a.cs[(rowbase + s) * a.H + h] = v[i];
    }
    if (lane == 0) a.cse[((size_t)b * a.nch + c) * a.H + h] = cend;
  }
  // 2. the group's B chunk
  const int boff = a.d_inner + g * a.N;
  const int n4 = a.N / 4;
  for (int i = tid; i < a.Q * n4; i += 512) {
    const int s = i / n4, q = i - s * n4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s < Qc) v = *reinterpret_cast<const float4 *>(a.xc + (rowbase + s) * a.conv_dim + boff + 4 * q);
    *reinterpret_cast<float4 *>(bs + s * NN + 4 * q) = v;
  }
  __syncthreads();
  // 3. tasks (head, p-tile); k index of lane group l/16 at step kk of block s0 is s = s0 + 4 (l/16) + kk
  const int npt = a.P / 16;
#pragma unroll 1
  for (int task = wave; task < a.hpg * npt; task += 8) {
    const int hh = task / npt, pt = task - hh * npt;
    const int h = g * a.hpg + hh;
    const float *wh = ws + hh * a.Q;
    const int p = 16 * pt + (lane & 15);
    const float *xcol = a.xc + rowbase * a.conv_dim + h * a.P + p;
    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{};
    // x two blocks ahead of its use
    float xa[4], xb[4], xn[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int s = 4 * (lane >> 4) + kk;
      xa[kk] = s < Qc ? xcol[(size_t)s * a.conv_dim] : 0.0f;
      xb[kk] = s + 16 < Qc ? xcol[(size_t)(s + 16) * a.conv_dim] : 0.0f;
    }
    for (int s0 = 0; s0 < Qc; s0 += 16) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int s = s0 + 32 + 4 * (lane >> 4) + kk;
        xn[kk] = s < Qc ? xcol[(size_t)s * a.conv_dim] : 0.0f;
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int s = s0 + 4 * (lane >> 4) + kk;
        const float av = xa[kk] * wh[s];
        const float *brow = bs + s * NN + (lane & 15);
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, brow[16 * j], acc[j], 0, 0, 0);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        xa[kk] = xb[kk];
        xb[kk] = xn[kk];
      }
    }
    // lane l, reg r -> p = 16 pt + 4 (l/16) + r, n = 16 j + l % 16
    float *out = a.sc + (((size_t)b * a.nch + c) * a.H + h) * (size_t)a.P * a.N;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(size_t)(16 * pt + 4 * (lane >> 4) + r) * a.N + 16 * j + (lane & 15)] = acc[j][r];
  }
}

// Per (session, head, state element): H_c = exp(cs_end_c) H_{c-1} + S_c over the
// chunks; sc[c] is overwritten with the state entering chunk c; the final state
// goes to the session's slot.
__global__ void state_pass_kernel(ScanArgs a) {
  const size_t PN = (size_t)a.P * a.N;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)a.B * a.H * PN) return;
  const size_t e = idx % PN;
  const int h = (int)((idx / PN) % a.H), b = (int)(idx / PN / a.H);
  bool ok;
  const int slot = slot_of(a, b, ok);
  float *st = a.ssm + ((size_t)slot * a.H + h) * PN + e;
  float Hs = *st;
  for (int c = 0; c < a.nch; ++c) {
    float *p = a.sc + (((size_t)b * a.nch + c) * a.H + h) * PN + e;
    const float S = *p;
    *p = Hs;
    Hs = fmaf(expf(a.cse[((size_t)b * a.nch + c) * a.H + h]), Hs, S);
  }
  if (ok) *st = Hs;
}

constexpr int kOutThreads = 512;

// Per (session, chunk, head): y = intra-chunk + entering-state terms + D x, the
// gate, v * norm_w and per-token sums of squares of v over the head. Computed as
// y^T tiles (p x t): lane l, reg r -> p = 16 i + 4 (l/16) + r, t = 16 ti + l % 16.
// Operands held in LDS: xs [Q][P + 4], hs [P][N + 4] (entering state); the C.B^T
// tiles and C rows come from global memory one step ahead of their use.
template <int NP>
__global__ __launch_bounds__(kOutThreads) void chunk_out_kernel(ScanArgs a) {
  extern __shared__ float lds[];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = h / a.hpg;
  const int t0 = c * a.Q;
  const int Qc = min(a.Q, a.T - t0);
  const int PP = a.P + 4, NN = a.N + 4;
  float *xs = lds;
  float *hs = xs + (size_t)a.Q * PP;
  float *css = hs + (size_t)a.P * NN;
  float *dts = css + a.Q;
  const size_t rowbase = (size_t)b * a.T + t0;
  const int p4 = a.P / 4;
  for (int i = tid; i < a.Q * p4; i += kOutThreads) {
    const int s = i / p4, q = i - s * p4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s < Qc) v = *reinterpret_cast<const float4 *>(a.xc + (rowbase + s) * a.conv_dim + h * a.P + 4 * q);
    *reinterpret_cast<float4 *>(xs + s * PP + 4 * q) = v;
  }
  const float *hsrc = a.sc + (((size_t)b * a.nch + c) * a.H + h) * (size_t)a.P * a.N;
  const int n4 = a.N / 4;
  for (int i = tid; i < a.P * n4; i += kOutThreads) {
    const int p = i / n4, q = i - p * n4;
    *reinterpret_cast<float4 *>(hs + p * NN + 4 * q) = reinterpret_cast<const float4 *>(hsrc)[i];
  }
  for (int s = tid; s < a.Q; s += kOutThreads) {
    css[s] = s < Qc ? a.cs[(rowbase + s) * a.H + h] : 0.0f;
    dts[s] = s < Qc ? a.dt[(rowbase + s) * a.H + h] : 0.0f;
  }
  __syncthreads();
  const int nt = (Qc + 15) / 16, np = npairs(a.Q / 16);
  const f32x4 *cbt = reinterpret_cast<const f32x4 *>(a.cbt + (((size_t)b * a.nch + c) * a.G + g) * (size_t)np * 256);
  const int coff = a.d_inner + a.G * a.N + g * a.N;
  const float Dh = a.D[h];
  // 8 waves; tile rounds alternate direction (tiles w, 15 - w, 16 + w, ...), so the
  // triangular intra-chunk work is shared evenly
#pragma unroll 1
  for (int r = 0; 8 * r < nt; ++r) {
    const int ti = (r & 1) ? 8 * r + 7 - wave : 8 * r + wave;
    if (ti >= nt) continue;
    f32x4 acc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = f32x4{};
    const int t = 16 * ti + (lane & 15);
    const bool t_ok = t < Qc;
    const float cst = t_ok ? css[t] : 0.0f;
    // intra-chunk: B (s x t) = CB^T[s][t] exp(cs_t - cs_s) dt_s for s <= t, straight from the
    // tile registers; A (p x s) = x_s[p] from LDS
    f32x4 mnext = cbt[(size_t)pair_index(0, ti) * 64 + lane];
#pragma unroll 1
    for (int si = 0; si <= ti; ++si) {
      f32x4 m = mnext;
      if (si < ti) mnext = cbt[(size_t)pair_index(si + 1, ti) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 16 * si + 4 * (lane >> 4) + r;
        m[r] = (t_ok && s <= t) ? m[r] * expf(cst - css[s]) * dts[s] : 0.0f;
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float *xrow = xs + (16 * si + 4 * (lane >> 4) + kk) * PP + (lane & 15);
#pragma unroll
        for (int i = 0; i < NP; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(xrow[16 * i], m[kk], acc[i], 0, 0, 0);
      }
    }
    // entering state: A (p x n) = H[p][n] from LDS, B (n x t) = C_t[n] exp(cs_t), in blocks of
    // 16 n (N % 16 == 0), the next block's C values loaded while this one is multiplied
    const float ecs = t_ok ? expf(cst) : 0.0f;
    const float *ct = a.xc + (rowbase + (t_ok ? t : 0)) * a.conv_dim + coff + (lane >> 4);
    float cv[4], cn[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) cv[q] = ct[4 * q];
#pragma unroll 1
    for (int n0 = 0; n0 < a.N; n0 += 16) {
      const bool more = n0 + 16 < a.N;
#pragma unroll
      for (int q = 0; q < 4; ++q) cn[q] = more ? ct[n0 + 16 + 4 * q] : 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float *hrow = hs + (lane & 15) * NN + n0 + 4 * q + (lane >> 4);
        const float bv = cv[q] * ecs;
#pragma unroll
        for (int i = 0; i < NP; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(hrow[16 * i * NN], bv, acc[i], 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) cv[q] = cn[q];
    }
    // epilogue
    float ssq = 0.0f;
    const size_t row = rowbase + (t_ok ? t : 0);
    const float *zrow = a.zx + row * a.zx_stride + h * a.P;
    const float *xrow = xs + (t_ok ? t : 0) * PP;
#pragma unroll
    for (int i = 0; i < NP; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
          const int p = 16 * i + 4 * (lane >> 4) + r;
          const float y = fmaf(Dh, xrow[p], acc[i][r]);
          const float v = y * silu(zrow[p]);
          if (t_ok) a.vw[row * a.d_inner + h * a.P + p] = v * a.norm_w[h * a.P + p];
          ssq = fmaf(v, v, ssq);
        }
    ssq += __shfl_xor(ssq, 16, 64);
    ssq += __shfl_xor(ssq, 32, 64);
    if (t_ok && lane < 16) a.ssh[row * a.H + h] = ssq;
  }
}

// RMS factor per (token, norm group) from per-head sums of squares (ng % P == 0).
__global__ void rms_kernel(ScanArgs a) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)a.B * a.T * a.n_norm) return;
  const int j = (int)(idx % a.n_norm);
  const size_t bt = idx / a.n_norm;
  const int hg = a.ng / a.P;
  float s = 0.0f;
  for (int q = 0; q < hg; ++q) s += a.ssh[bt * a.H + j * hg + q];
  a.rn[bt * a.n_norm + j] = 1.0f / sqrtf(s / (float)a.ng + a.eps);
}

// conv cache <- the last d_conv-1 raw inputs; one thread per (session, channel) so
// every old value is read before any is overwritten.
__global__ void cache_update_kernel(ScanArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.B * a.conv_dim) return;
  const int c = idx % a.conv_dim, b = idx / a.conv_dim;
  bool ok;
  const int slot = slot_of(a, b, ok);
  if (!ok) return;
  const int K1 = a.d_conv - 1;
  float *cc = a.conv + (size_t)slot * K1 * a.conv_dim + c;
  float nv[8];
  for (int k = 0; k < K1; ++k) {
    const int tau = a.T - K1 + k;           // position of the k-th newest-but-(K1-1-k) input
    nv[k] = tau >= 0 ? a.zx[((size_t)b * a.T + tau) * a.zx_stride + a.d_inner + c]
                     : cc[(size_t)(K1 + tau) * a.conv_dim];
  }
  for (int k = 0; k < K1; ++k) cc[(size_t)k * a.conv_dim] = nv[k];
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr size_t kLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950

struct PrefillWs {
  float *zx, *xc, *dt, *cs, *cse, *sc, *cbt, *vw, *ssh, *rn;
  size_t bytes;
};

PrefillWs prefill_layout(const m2_layer_s &L, int B, int T, int Q, void *base) {
  const size_t BT = (size_t)B * T;
  const int nch = (T + Q - 1) / Q;
  const int nt = Q / 16;
  const size_t sizes[10] = {
      BT * L.zx_stride, BT * L.conv_dim, BT * L.cfg.n_heads, BT * L.cfg.n_heads,
      (size_t)B * nch * L.cfg.n_heads,
      (size_t)B * nch * L.cfg.n_heads * L.cfg.head_dim * L.cfg.d_state,
      (size_t)B * nch * L.cfg.n_groups * (size_t)(nt * (nt + 1) / 2) * 256,
      BT * L.d_inner, BT * L.cfg.n_heads, BT * L.n_norm};
  PrefillWs w{};
  float **ptrs[10] = {&w.zx, &w.xc, &w.dt, &w.cs, &w.cse, &w.sc, &w.cbt, &w.vw, &w.ssh, &w.rn};
  size_t off = 0;
  for (int i = 0; i < 10; ++i) {
    *ptrs[i] = base ? reinterpret_cast<float *>(static_cast<char *>(base) + off) : nullptr;
    off += align256(sizes[i] * sizeof(float));
  }
  w.bytes = off;
  return w;
}

bool prefill_supported(const m2_layer_s &L) {
  return L.cfg.head_dim % 16 == 0 && L.cfg.head_dim <= 128 && L.cfg.d_state % 16 == 0 &&
         L.cfg.d_state <= 256 && L.ng % L.cfg.head_dim == 0;
}

size_t scan_lds_state(const m2_layer_s &L, int Q) {
  return sizeof(float) * ((size_t)Q * (L.cfg.d_state + 4) + 2 * (size_t)Q);
}
size_t scan_lds_out(const m2_layer_s &L, int Q) {
  return sizeof(float) *
         ((size_t)Q * (L.cfg.head_dim + 4) + (size_t)L.cfg.head_dim * (L.cfg.d_state + 4) + 2 * (size_t)Q);
}

template <typename F>
hipError_t allow_lds(F *kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int NT>
hipError_t launch_chunk_state_t(const ScanArgs &a, size_t lds, dim3 grid, dim3 block, hipStream_t stream) {
  hipError_t e = allow_lds(chunk_state_kernel<NT>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_state_kernel<NT>, grid, block, lds, stream, a);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_chunk_state_group_t(const ScanArgs &a, size_t lds, dim3 grid, hipStream_t stream) {
  hipError_t e = allow_lds(chunk_state_group_kernel<NT>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_state_group_kernel<NT>, grid, dim3(512), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_chunk_state_group(int nt, const ScanArgs &a, size_t lds, dim3 grid, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_chunk_state_group_t<1>(a, lds, grid, stream);
    case 2: return launch_chunk_state_group_t<2>(a, lds, grid, stream);
    case 4: return launch_chunk_state_group_t<4>(a, lds, grid, stream);
    case 8: return launch_chunk_state_group_t<8>(a, lds, grid, stream);
    case 16: return launch_chunk_state_group_t<16>(a, lds, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// n-tiles of the state: d_state / 16 in {1, 2, 4, 8, 16}
hipError_t launch_chunk_state(int nt, const ScanArgs &a, size_t lds, dim3 grid, dim3 block, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_chunk_state_t<1>(a, lds, grid, block, stream);
    case 2: return launch_chunk_state_t<2>(a, lds, grid, block, stream);
    case 4: return launch_chunk_state_t<4>(a, lds, grid, block, stream);
    case 8: return launch_chunk_state_t<8>(a, lds, grid, block, stream);
    case 16: return launch_chunk_state_t<16>(a, lds, grid, block, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int NP>
hipError_t launch_chunk_out_t(const ScanArgs &a, size_t lds, dim3 grid, hipStream_t stream) {
  hipError_t e = allow_lds(chunk_out_kernel<NP>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_out_kernel<NP>, grid, dim3(kOutThreads), lds, stream, a);
  return hipGetLastError();
}

// p-tiles of a head: head_dim / 16 in 1 .. 8
hipError_t launch_chunk_out(int np, const ScanArgs &a, size_t lds, dim3 grid, hipStream_t stream) {
  switch (np) {
    case 1: return launch_chunk_out_t<1>(a, lds, grid, stream);
    case 2: return launch_chunk_out_t<2>(a, lds, grid, stream);
    case 3: return launch_chunk_out_t<3>(a, lds, grid, stream);
    case 4: return launch_chunk_out_t<4>(a, lds, grid, stream);
    case 5: return launch_chunk_out_t<5>(a, lds, grid, stream);
    case 6: return launch_chunk_out_t<6>(a, lds, grid, stream);
    case 7: return launch_chunk_out_t<7>(a, lds, grid, stream);
    case 8: return launch_chunk_out_t<8>(a, lds, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_gemm(const m2_layer_s &L, bool in_proj, const float *A, int lda, float *C, int ldc,
                    const float *R, int ldr, const float *rs, int M, hipStream_t stream) {
  const m2_config &c = L.cfg;
  const int N = in_proj ? L.d_in_proj : c.d_model;
  const int K = in_proj ? c.d_model : L.d_inner;
  // the MFMA GEMM reads whole 16-wide groups of K (K % 16 == 0 for every layer) and one
  // scale per group of 16 (the norm group a multiple of 16)
  if (c.wtype == M2_W_BF16 && K % 16 == 0 && (!rs || L.ng % 16 == 0)) {
    GemmArgs g{};
    g.A = A;
    g.lda = lda;
    const void *panels = in_proj ? L.w.w_in_panels : L.w.w_out_panels;
    g.W = static_cast<const unsigned short *>(panels ? panels : in_proj ? L.w.w_in : L.w.w_out);
    g.S = (K + 31) / 32;
    g.C = C;
    g.ldc = ldc;
    g.R = R;
    g.ldr = ldr;
    g.rs = rs;
    g.n_rs = L.n_norm;
    g.ng = L.ng;
    g.M = M;
    g.N = N;
    g.K = K;
    auto *k = panels ? gemm_bf16_kernel<true> : gemm_bf16_kernel<false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kGemmLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(((N + GBN - 1) / GBN) * ((M + GBM - 1) / GBM)), dim3(256), kGemmLds, stream, g);
    return hipGetLastError();
  }
  GemmValuArgs g{};
  g.A = A;
  g.lda = lda;
  g.W = in_proj ? L.w.w_in : L.w.w_out;
  g.S = static_cast<const __half *>(in_proj ? L.w.s_in : L.w.s_out);
  g.wtype = c.wtype;
  const bool quantized = c.wtype == M2_W_INT8G || c.wtype == M2_W_INT4G || c.wtype == M2_W_INT3G;
  g.q_group = quantized ? c.q_group : K;
  g.gamma = quantized ? (in_proj ? c.q_gamma_in : c.q_gamma_out) : 1.0f;
  g.C = C;
  g.ldc = ldc;
  g.R = R;
  g.ldr = ldr;
  g.rs = rs;
  g.n_rs = L.n_norm;
  g.ng = L.ng;
  g.M = M;
  g.N = N;
  g.K = K;
  hipLaunchKernelGGL(gemm_valu_kernel, dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

size_t prefill_ws_bytes(const m2_layer_s &L, int batch, int seqlen, int chunk) {
  if (!prefill_supported(L)) return 0;
  // the scan kernels hold a chunk's operands in LDS: refuse chunk lengths whose tiles do
  // not fit, before anything is launched
  if (scan_lds_out(L, chunk) > kLdsBytes || scan_lds_state(L, chunk) > kLdsBytes) return 0;
  return prefill_layout(L, batch, seqlen, chunk, nullptr).bytes;
}

hipError_t launch_prefill(const m2_layer_s &L, const m2_state_s &S, const float *x, float *y, int batch,
                          int seqlen, int chunk, const int32_t *slots, int flags, void *ws_base,
                          hipStream_t stream) {
  const m2_config &c = L.cfg;
  const int B = batch, T = seqlen, Q = chunk;
  const int M = B * T;
  PrefillWs ws = prefill_layout(L, B, T, Q, ws_base);
  ScanArgs a{};
  a.B = B;
  a.T = T;
  a.Q = Q;
  a.nch = (T + Q - 1) / Q;
  a.H = c.n_heads;
  a.P = c.head_dim;
  a.N = c.d_state;
  a.G = c.n_groups;
  a.hpg = L.hpg;
  a.d_inner = L.d_inner;
  a.conv_dim = L.conv_dim;
  a.d_conv = c.d_conv;
  a.zx_stride = L.zx_stride;
  a.zx = ws.zx;
  a.xc = ws.xc;
  a.dt = ws.dt;
  a.cs = ws.cs;
  a.cse = ws.cse;
  a.sc = ws.sc;
  a.cbt = ws.cbt;
  a.vw = ws.vw;
  a.ssh = ws.ssh;
  a.rn = ws.rn;
  a.n_norm = L.n_norm;
  a.ng = L.ng;
  a.eps = c.norm_eps;
  a.conv_w = L.w.conv_w;
  a.conv_b = L.w.conv_b;
  a.dt_bias = L.w.dt_bias;
  a.A_log = L.w.A_log;
  a.D = L.w.D;
  a.norm_w = L.w.norm_w;
  a.ssm = S.ssm;
  a.conv = S.conv;
  a.slots = slots;
  a.n_slots = S.n_slots;

  // 1. in_proj
  hipError_t e = run_gemm(L, true, x, c.d_model, ws.zx, L.zx_stride, nullptr, 0, nullptr, M, stream);
  if (e != hipSuccess) return e;
  // 2. conv + dt
  {
    const dim3 grid((L.conv_dim + c.n_heads + 255) / 256, batch, (seqlen + kConvSeg - 1) / kConvSeg);
    hipLaunchKernelGGL(conv_dt_kernel, grid, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 3. C B^T tiles
  hipLaunchKernelGGL(cb_kernel, dim3(Q / 16, a.nch, c.n_groups * B), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 4. chunk states
  {
    // per group when its B chunk and the weights of its heads fit in LDS, else per head
    const size_t lds_g = sizeof(float) * ((size_t)Q * (c.d_state + 4) + (size_t)L.hpg * Q);
    if (lds_g <= kLdsBytes) {
      if ((e = launch_chunk_state_group(c.d_state / 16, a, lds_g, dim3(a.nch, c.n_groups, B), stream)) != hipSuccess)
        return e;
    } else {
      const size_t lds = scan_lds_state(L, Q);
      if ((e = launch_chunk_state(c.d_state / 16, a, lds, dim3(a.nch, c.n_heads, B), dim3(64 * (c.head_dim / 16)),
                                  stream)) != hipSuccess)
        return e;
    }
  }
  // 5. inter-chunk pass (reads the slots' states, writes the final ones)
  {
    const size_t n = (size_t)B * c.n_heads * c.head_dim * c.d_state;
    hipLaunchKernelGGL(state_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 6. chunk outputs, gate, sums of squares
  {
    const size_t lds = scan_lds_out(L, Q);
    if ((e = launch_chunk_out(c.head_dim / 16, a, lds, dim3(a.nch, c.n_heads, B), stream)) != hipSuccess) return e;
  }
  // 7. RMS factors
  {
    const size_t n = (size_t)M * L.n_norm;
    hipLaunchKernelGGL(rms_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 8. out_proj (+ residual)
  e = run_gemm(L, false, ws.vw, L.d_inner, y, c.d_model, (flags & M2_RESIDUAL) ? x : nullptr, c.d_model, ws.rn, M,
               stream);
  if (e != hipSuccess) return e;
  // 9. conv cache
  {
    const int n = B * L.conv_dim;
    hipLaunchKernelGGL(cache_update_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace m2d
