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
#include "decode_common.h"
#include <algorithm>

namespace m2d {
namespace {

// ---------------------------------------------------------------------------
// gemv_wave: one wave per row, whole-K activations of BT (= batch) sessions in LDS.
// LDS: act [BT][K] | rn [BT][n_norm]
template <int WT, int BT, int TPB, int U, int NT, int PRO, int EPI>
__global__ __launch_bounds__(TPB) void gemv_wave_kernel(GemvArgs a) {
  extern __shared__ float lds[];
  constexpr int WPB = TPB / 64;
  constexpr int EPC = WTraits<WT>::EPC;
  constexpr int CB = WTraits<WT>::CB;
  using chunk_t = typename WTraits<WT>::chunk_t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x * WPB + __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool row_ok = row < a.rows;
  const int nb = min(BT, a.B);
  const int K = a.K;
  const int NC = K / EPC;
  const char *wr = static_cast<const char *>(a.W) + (size_t)(row_ok ? row : 0) * NC * CB;
  const void *srow = scale_row<WT>(a.S, (size_t)(row_ok ? row : 0), NC >> a.q_shift);
  // 16-byte chunks are read through a buffer resource over the wave's row (none for a row
  // past the matrix): a chunk past the row takes an offset past the resource and reads zeros
  // without a memory access, so no weight load is conditional and each register can be
  // refilled as soon as its chunk has been used (the compiler's wait counts stay exact)
  constexpr bool BUF = CB == 16;
  const __amdgpu_buffer_rsrc_t rr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(wr), (short)0, row_ok ? NC * CB : 0, 0x00020000);
  auto ldw = [&](int c) -> chunk_t {
    if constexpr (BUF) {
      return __builtin_amdgcn_raw_buffer_load_b128(rr, c < NC ? c * 16 : kBufOutOfRange, 0, NT ? 2 : 0);   // 2: nt
    } else {
      return (row_ok && c < NC) ? load_chunk<WT, NT>(wr, c) : chunk_t{};
    }
  };

  // weights do not depend on the activations: put the first U loads in flight first
  chunk_t w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) w[u] = ldw(lane + 64 * u);
  EpiIn epi{};
  if (row_ok && lane < nb) epi = epilogue_prefetch<EPI>(a, row, lane);
  if (EPI == EPI_INPROJ && a.bar_clear && blockIdx.x == 0 && tid < kBarWords) a.bar_clear[tid * kBarStride] = 0u;

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
  // lane l adds its chunks l, l + 64, l + 128, ... in order (trip t holds chunks
  // l + 64 (U t + u), u < U); with buffer loads each register takes the same chunk of the
  // next trip right after its use, so U loads stay in flight through the whole row
  if (row_ok) {
    const int trips = (NC + 64 * U - 1) / (64 * U);
    for (int t = 0; t < trips; ++t) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = lane + 64 * (U * t + u);
        if (c < NC) {
          const QScale qs = load_qscale<WT>(srow, c, a.q_shift);
#pragma unroll
          for (int bb = 0; bb < BT; ++bb) acc[bb] = chunk_acc<WT>(w[u], act_s + bb * K + c * EPC, qs, acc[bb]);
        }
        if constexpr (BUF) w[u] = ldw(c + 64 * U);
      }
      if constexpr (!BUF) {
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = ldw(lane + 64 * (U * (t + 1) + u));
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
// LDS: act [BT][K] | xsum [BT][K/32] (| rn [BT][n_norm], out_proj)
constexpr int kLbThreads = 512;

template <int WT, int BT, int PRO>
__device__ __forceinline__ void lb_stage(const GemvArgs &a, float *lds, int tid) {
  constexpr int TPB = kLbThreads;
  constexpr int MAXF = kNormF4PerThread;
  const int K = a.K, nf = K / 4, nb = min(BT, a.B);
  f32x4 v[BT][MAXF];
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    const int sb = min(bb, nb - 1);
    const f32x4 *src = reinterpret_cast<const f32x4 *>(a.act + (size_t)sb * K);
#pragma unroll
    for (int i = 0; i < MAXF; ++i) v[bb][i] = src[min(tid + TPB * i, nf - 1)];   // clamped index
  }
  const int KP = lds_padded(K);
  float *acts = lds;
  if (PRO == PRO_NORM) {
    // the RMS factors: wave w reduces norm groups w, w + 8, ... (each lane a strided part of
    // the group's partials, then a cross-lane tree: a fixed order)
    float *rn = lds + BT * (KP + K / 32);
    const int per = a.n_partials / a.n_norm, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) {
      const float *ssb = a.ss + (size_t)min(bb, nb - 1) * a.n_partials;
      for (int g = wave; g < a.n_norm; g += TPB / 64) {
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


// NW waves per item, up to MAXI state slices per wave (NW * MAXI >= the item's
// wave instructions).
template <int NW, int MAXI>
__global__ __launch_bounds__(NW * 64) void ssd_step_kernel(SsdArgs a) {
  __shared__ float wsum[NW];
  __shared__ float cx[2 * 256 + 64];   // conv outputs: B [N] | C [N] | x rows [prange <= 64]
  const int h = blockIdx.x / a.psplit, ps = blockIdx.x - h * a.psplit;
  ssd_item<NW, MAXI>(a, h, ps, blockIdx.y, threadIdx.x >> 6, threadIdx.x & 63, wsum, cx);
}


// ---------------------------------------------------------------------------
// gemv_mfma: batch 3..32 with bf16 weights, or int8 weights with q_group 128 or
// 256. Work is cut stream-K fashion: a unit is one 128-row block x one 256-wide k tile,
// units are numbered row block by row block, and workgroup g of G takes units
// [g U / G, (g + 1) U / G). G is about one workgroup per CU but at least the number of
// row blocks, so every workgroup gets the same work to within one
// unit and its run spans at most two row blocks; it writes one partial sum per row block
// it touches (its first at partial g, a second one, which begins inside its run, at
// partial G + row block), and gemv_mfma_reduce adds a row block's partials in workgroup
// order, so results do not depend on scheduling. Within a workgroup, 8 waves
// own 16 rows each. Per 32-wide k-step: A = 16 weight rows x 32 k straight from HBM
// (one 16- or 8-byte load per lane and step), B = 32 k x 16 sessions from LDS as bf16
// hi + lo (an fp32 value is hi + lo to 2^-16 relative; bf16 and int8 weights are exact
// in bf16), two 16x16x32 bf16 MFMAs per product. The units are software-pipelined:
// each k-step's weight registers are refilled with the same k-step of the next unit as
// soon as its MFMAs are issued (8 loads per lane in flight: more only queue behind the
// HBM's capacity and slow the stream), the next unit's activations are loaded into
// registers meanwhile and converted into the second LDS buffer; one barrier per unit.
// Weights come either row-major or as 16-row panels (m2_pack_panels), in which one
// k-step of a 16-row panel is the 1 KB (bf16; 512 B int8) of the lanes' A fragments in
// lane order: a load instruction then reads whole cache lines instead of 64 (32) bytes
// of each of 16 rows, and goes out nontemporal. Every global load goes through a buffer
// resource: a row past the matrix, a session past the batch or a k past K takes an
// out-of-range offset and reads zeros, so the unit loop has no branch around a load and
// each wait is for exactly the load whose value comes next. With RMS (out_proj) the
// workgroup first forms the RMS factors of the norm groups its units cover from the
// sums of squares (fixed order) and scales the activations by them while staging.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMRows = 128;        // rows per workgroup (8 waves x 16)
// k tile of a unit, and LDS rows of a tile's activations (KT + 8 bf16). A 512-wide tile
// for int8 (the same 8 KB per wave in flight as bf16) measured no faster (27-layer int8
// stack at 8 sessions: 548 against 553 stack steps/s).
template <int WT> constexpr int mfma_kt() { return 256; }
template <int WT> constexpr int mfma_ldw() { return mfma_kt<WT>() + 8; }
constexpr int kMaxScaleGroups = 2; // int8 scale groups in one k tile (q_group >= 128)
constexpr int kRmsLoads = 16;      // out_proj RMS prologue: partial sums a lane requests at once

struct MfmaArgs {
  const void *W;                   // row-major [rows][K], or 16-row panels
  const __half *S;                 // int8: fp16 scales [rows][K / q_group]
  int rows, K, q_group;
  int T;                           // k tiles per row block: ceil(K / 256)
  int U;                           // units: row blocks x T
  int nks;                         // panels: 32-wide k-steps per panel, ceil(K / 32)
  const float *act;                // [B][K]
  int B;
  // RMS prologue (out_proj): act[b][k] *= 1/sqrt(sum_j ss[b][g*per + j] / ng + eps), g = k / ng
  const float *ss;
  int n_partials, n_norm, ng;
  float eps;
  int ngt;                         // RMS factors held per session in LDS
  float *part;                     // [G + row blocks][B][128]
};

// Raw weights of one unit for one lane: KT / 32 k-steps of 8 values.
template <int WT> struct MRaw;
template <> struct MRaw<M2_W_BF16> { bf16x8 v[mfma_kt<M2_W_BF16>() / 32]; };
template <> struct MRaw<M2_W_INT8G> { uint2 v[mfma_kt<M2_W_INT8G>() / 32]; };

template <int WT> constexpr int mfma_esz() { return WT == M2_W_BF16 ? 2 : 1; }
template <int WT> constexpr int mfma_frag() { return 8 * mfma_esz<WT>(); }   // bytes per lane and k-step

// Weight resource of row block rb. Offsets stay below 2^31 (checked on the host).
template <int WT, bool PANEL>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mfma_wres(const MfmaArgs &a, int rb) {
  char *base = const_cast<char *>(static_cast<const char *>(a.W));
  if constexpr (PANEL) {
    const int npan = (a.rows + 15) / 16;
    const int np = min(kMRows / 16, npan - rb * (kMRows / 16));
    const int pbytes = a.nks * 64 * mfma_frag<WT>();
    return __builtin_amdgcn_make_buffer_rsrc(base + (size_t)rb * (kMRows / 16) * pbytes, (short)0, np * pbytes,
                                             0x00020000);
  } else {
    const int nr = min(kMRows, a.rows - rb * kMRows);
    return __builtin_amdgcn_make_buffer_rsrc(base + (size_t)rb * kMRows * a.K * mfma_esz<WT>(), (short)0,
                                             nr * a.K * mfma_esz<WT>(), 0x00020000);
  }
}

// This lane's byte offset of k-step 0 within its row block's resource.
template <int WT, bool PANEL>
__device__ __forceinline__ int mfma_lbase(const MfmaArgs &a, int wave, int lane) {
  if constexpr (PANEL) return (wave * a.nks * 64 + lane) * mfma_frag<WT>();
  else return (wave * 16 + (lane & 15)) * a.K * mfma_esz<WT>();
}

// One k-step of weights for this lane at k (its 8 values start there); zeros at k >= K
// or past the block's rows.
template <int WT, bool PANEL>
__device__ __forceinline__ void mfma_ld(__amdgpu_buffer_rsrc_t wr, int lb, int k, int K, MRaw<WT> &w, int st) {
  const int off = k < K ? lb + (PANEL ? (k >> 5) * 64 * mfma_frag<WT>() : k * mfma_esz<WT>()) : kBufOutOfRange;
  constexpr int aux = PANEL ? 2 : 0;     // panels: nontemporal
  if constexpr (WT == M2_W_BF16) {
    w.v[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, aux));
  } else {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, off, 0, aux);
    w.v[st] = make_uint2(v.x, v.y);
  }
}

// int8 scales of a unit's q_group groups (at most kMaxScaleGroups) for this lane's 4 C
// rows (rows r4 .. r4 + 3 of the matrix); zero for a group that starts at or past K. Kept
// as fp16 bits until the tile applies them: converted here, the conversion would wait for
// the loads at once.
template <int KT>
__device__ __forceinline__ void mfma_load_s(const MfmaArgs &a, __amdgpu_buffer_rsrc_t sr, int r4, int kt,
                                            unsigned short (&sc)[kMaxScaleGroups][4]) {
  const int ngrp = a.K / a.q_group;
#pragma unroll
  for (int q = 0; q < kMaxScaleGroups; ++q) {
    const int k0 = kt + q * a.q_group;
    const bool ok = q * a.q_group < KT && k0 < a.K;
    const int g = k0 / a.q_group;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int off = ok ? ((r4 + i) * ngrp + g) * 2 : kBufOutOfRange;
      sc[q][i] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
    }
  }
}

template <int WT> __device__ __forceinline__ bf16x8 mfma_a(const MRaw<WT> &w, int st);
template <> __device__ __forceinline__ bf16x8 mfma_a<M2_W_BF16>(const MRaw<M2_W_BF16> &w, int st) { return w.v[st]; }
// int8 -> bf16 is exact; the conversions vectorise to byte-select converts and packed
// bf16 converts (1.5 instructions per value).
template <> __device__ __forceinline__ bf16x8 mfma_a<M2_W_INT8G>(const MRaw<M2_W_INT8G> &w, int st) {
  // the empty asm keeps each k-step's conversion at its k-step: without it the
  // instruction scheduler converts all eight at the top of the tile, which waits there for
  // the last of the tile's weight loads
  uint2 v = w.v[st];
  asm volatile("" : "+v"(v.x), "+v"(v.y));
  f32x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const unsigned wd = e < 4 ? v.x : v.y;
    f[e] = (float)((int32_t)(wd << (24 - 8 * (e & 3))) >> 24);
  }
  return __builtin_convertvector(f, bf16x8);
}

// Activations of one k tile (NBT*16 sessions x KT k; zeros past the batch and past K)
// into registers.
template <int NBT, int KT>
__device__ __forceinline__ void mfma_load_x(const MfmaArgs &a, __amdgpu_buffer_rsrc_t xr, int kt, int tid,
                                            float4 (&xv)[NBT * KT / 128]) {
#pragma unroll
  for (int q = 0; q < NBT * KT / 128; ++q) {
    const int i = tid + 512 * q;
    const int b = i / (KT / 4), k4 = (i - b * (KT / 4)) * 4;
    const int off = kt + k4 < a.K ? (b * a.K + kt + k4) * 4 : kBufOutOfRange;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
    xv[q] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  }
}

// The RMS factors a workgroup holds: groups [g0, g1] of its first row block's k range,
// then [0, h1] of the second's (if its units reach into a second row block).
struct RmsMap {
  int g0, g1, h1, nA;
};

// ... scaled by the RMS factors (RMS; `first`: the unit is in the workgroup's first row
// block) and stored as bf16 hi / lo.
template <int NBT, int KT, bool RMS>
__device__ __forceinline__ void mfma_store_x(const MfmaArgs &a, int kt, int tid, const float4 (&xv)[NBT * KT / 128],
                                             unsigned short *xh, unsigned short *xl, const float *rn_s,
                                             const RmsMap &m, bool first) {
  constexpr int LD = KT + 8;
#pragma unroll
  for (int q = 0; q < NBT * KT / 128; ++q) {
    const int i = tid + 512 * q;
    const int b = i / (KT / 4), k4 = (i - b * (KT / 4)) * 4;
    f32x4 vv = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
    if (RMS) {
      // Past the end of K (a ragged last tile) the activation is 0 and the group index
      // would leave the range of held factors; clamped, the factor is this session's own
      // last one, so 0 * r is 0 unless this very session's factors are NaN (an
      // out-of-range slot).
      const int g = (kt + k4) / a.ng;
      const int gi = first ? min(g, m.g1) - m.g0 : m.nA + min(g, m.h1);
      const float r = b < a.B ? rn_s[b * a.ngt + gi] : 0.0f;
      vv *= r;
    }
    // hi = bf16(v) and lo = bf16(v - hi), both rounded to nearest even
    const bf16x4 h = __builtin_convertvector(vv, bf16x4);
    const bf16x4 l = __builtin_convertvector(vv - __builtin_convertvector(h, f32x4), bf16x4);
    *reinterpret_cast<bf16x4 *>(&xh[b * LD + k4]) = h;
    *reinterpret_cast<bf16x4 *>(&xl[b * LD + k4]) = l;
  }
}

// The MFMAs of one unit; with REFILL each k-step's weight registers are refilled with
// the same k-step of the next unit (resource wn, k tile kn) as soon as its MFMAs are
// issued. int8: SPG k-steps form one scale group (q_group / 32), whose products are
// gathered and then scaled.
template <int WT, bool PANEL, int NBT, int SPG, bool REFILL>
__device__ __forceinline__ void mfma_tile(MRaw<WT> &w, const unsigned short (&sc)[kMaxScaleGroups][4], int lane, int kq,
                                          const unsigned short *xh, const unsigned short *xl, f32x4 (&acc)[NBT],
                                          __amdgpu_buffer_rsrc_t wn, int lb, int kn, int K) {
  constexpr int KT = mfma_kt<WT>(), LD = KT + 8;
  f32x4 gacc[NBT];
#pragma unroll
  for (int st = 0; st < KT / 32; ++st) {
    if (WT == M2_W_INT8G && st % SPG == 0) {
#pragma unroll
      for (int j = 0; j < NBT; ++j) gacc[j] = f32x4{};
    }
    const bf16x8 av = mfma_a<WT>(w, st);
#pragma unroll
    for (int j = 0; j < NBT; ++j) {
      const int b = 16 * j + (lane & 15);
      const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&xh[b * LD + 32 * st + kq]);
      const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&xl[b * LD + 32 * st + kq]);
      f32x4 &d = WT == M2_W_BF16 ? acc[j] : gacc[j];
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, d, 0, 0, 0);
    }
    if (WT == M2_W_INT8G && st % SPG == SPG - 1) {
      const int q = st / SPG;
#pragma unroll
      for (int j = 0; j < NBT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(__half2float(__ushort_as_half(sc[q][i])), gacc[j][i], acc[j][i]);
    }
    if (REFILL) {
      // issued here, not clustered at the unit's end by the scheduler: each load then has
      // a whole unit's time to arrive
      mfma_ld<WT, PANEL>(wn, lb, kn + 32 * st + kq, K, w, st);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// This lane's accumulators to partial `pi`: lane l, register i -> block row
// wave*16 + (l/16)*4 + i, session 16 j + l % 16.
template <int NBT>
__device__ __forceinline__ void mfma_flush(const MfmaArgs &a, int pi, int lr4, int lane, f32x4 (&acc)[NBT]) {
  float *part = a.part + (size_t)pi * a.B * kMRows;
#pragma unroll
  for (int j = 0; j < NBT; ++j) {
    const int b = 16 * j + (lane & 15);
    if (b < a.B) {
#pragma unroll
      for (int i = 0; i < 4; ++i) part[(size_t)b * kMRows + lr4 + i] = acc[j][i];
    }
    acc[j] = f32x4{};
  }
}

// A workgroup that owns a whole row block (EPI >= 0): its sums are final, so each lane
// applies the row epilogue to its own 4 rows x NBT sessions. The epilogue inputs are
// loaded before the last tile (unconditional loads, so that the tile's weights need no
// wait for them) and the results stored after it.
template <int EPI, int NBT>
struct MfmaEpi {
  EpiIn e[NBT][4];
};

template <int EPI, int NBT>
__device__ __forceinline__ void mfma_epi_load(const GemvArgs &g, int row0, int lane, MfmaEpi<EPI, NBT> &m) {
#pragma unroll
  for (int j = 0; j < NBT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m.e[j][i] = epilogue_load_all<EPI>(g, min(row0 + i, g.rows - 1), min(16 * j + (lane & 15), g.B - 1));
}

template <int EPI, int NBT>
__device__ __forceinline__ void mfma_epi_store(const GemvArgs &g, int row0, int lane, const f32x4 (&acc)[NBT],
                                               const MfmaEpi<EPI, NBT> &m) {
#pragma unroll
  for (int j = 0; j < NBT; ++j) {
    const int b = 16 * j + (lane & 15);
    if (b < g.B) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (row0 + i < g.rows) gemv_epilogue<EPI>(g, row0 + i, b, acc[j][i], m.e[j][i]);
    }
  }
}

constexpr int kEpiPartials = -1;

// One workgroup of 8 waves per CU (2 waves per SIMD): up to 256 VGPRs a wave. EPI:
// kEpiPartials (partial sums per workgroup, reduced by gemv_mfma_reduce_kernel) or the
// row epilogue of g (every workgroup owns exactly one row block: G = U / T).
template <int WT, bool PANEL, int NBT, bool RMS, int SPG, int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemv_mfma_kernel(MfmaArgs a,
                                                                                                    GemvArgs g) {
  extern __shared__ unsigned short xs[];            // [2 buffers][hi, lo][NBT*16][KT + 8], then rn
  constexpr int KT = mfma_kt<WT>();
  constexpr int XB = NBT * 16 * mfma_ldw<WT>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x;
  const int u0 = (int)((long)blockIdx.x * a.U / G), u1 = (int)((long)(blockIdx.x + 1) * a.U / G);
  if (u0 >= u1) return;
  const int lr4 = wave * 16 + (lane >> 4) * 4;       // block row of this lane's first result
  const int kq = (lane >> 4) * 8;                    // this lane's 8 k within a 32-wide step
  const int lb = mfma_lbase<WT, PANEL>(a, wave, lane);
  float *rn_s = reinterpret_cast<float *>(xs + 4 * XB);
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.act), (short)0, a.B * a.K * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__half *>(a.S), (short)0, WT == M2_W_INT8G ? a.rows * (a.K / a.q_group) * 2 : 0, 0x00020000);

  int rb = u0 / a.T, t = u0 - rb * a.T;
  const int rbA = rb;
  __amdgpu_buffer_rsrc_t wr = mfma_wres<WT, PANEL>(a, rb);
  MRaw<WT> w;
  unsigned short s0[kMaxScaleGroups][4] = {}, s1[kMaxScaleGroups][4] = {};
  float4 xv[NBT * KT / 128];
  // activations first, so that staging them waits for them alone
  mfma_load_x<NBT, KT>(a, xr, t * KT, tid, xv);
  if (WT == M2_W_INT8G) mfma_load_s<KT>(a, sr, rb * kMRows + lr4, t * KT, s0);
#pragma unroll
  for (int st = 0; st < KT / 32; ++st) mfma_ld<WT, PANEL>(wr, lb, t * KT + 32 * st + kq, a.K, w, st);

  RmsMap m{};
  if (RMS) {
    // the groups of the first row block's k range [t * 256, end) and of the second's
    // [0, end); their RMS factors: 8 lanes per (session, group), strided sums combined in
    // a fixed order
    const int ul = u1 - 1, rbl = ul / a.T, tl = ul - rbl * a.T;
    const int kA1 = min(a.K, (rbl == rbA ? tl + 1 : a.T) * KT);
    m.g0 = t * KT / a.ng;
    m.g1 = (kA1 - 1) / a.ng;
    m.nA = m.g1 - m.g0 + 1;
    m.h1 = rbl > rbA ? (min(a.K, (tl + 1) * KT) - 1) / a.ng : -1;
    const int nh = m.nA + m.h1 + 1;
    const int per = a.n_partials / a.n_norm;
    for (int base = 0; base < a.B * nh * 8; base += 512) {
      const int i = base + tid, pair = i >> 3, j = i & 7;
      const bool ok = pair < a.B * nh;
      const int pc = ok ? pair : 0;
      const int b = pc / max(nh, 1), slot = pc - b * nh;
      const int g = slot < m.nA ? m.g0 + slot : slot - m.nA;
      const float *sp = a.ss + (size_t)b * a.n_partials + g * per;
      float sum = 0.0f;
      // this lane's partials j, j + 8, ... requested together (indices clamped, values
      // selected after: a load behind a branch or in a loop waits for everything before it),
      // added in that order
      for (int q0 = j; q0 < per; q0 += 8 * kRmsLoads) {
        float pv[kRmsLoads];
#pragma unroll
        for (int k = 0; k < kRmsLoads; ++k) pv[k] = sp[min(q0 + 8 * k, per - 1)];
#pragma unroll
        for (int k = 0; k < kRmsLoads; ++k) sum += q0 + 8 * k < per ? pv[k] : 0.0f;
      }
      sum = group_reduce<8>(sum);
      if (ok && j == 0) rn_s[b * a.ngt + slot] = 1.0f / sqrtf(sum / (float)a.ng + a.eps);
    }
    lds_barrier();
  }
  mfma_store_x<NBT, KT, RMS>(a, t * KT, tid, xv, xs, xs + XB, rn_s, m, true);
  lds_barrier();

  f32x4 acc[NBT];
#pragma unroll
  for (int j = 0; j < NBT; ++j) acc[j] = f32x4{};
  int buf = 0;
  // Every unit but the last: the next unit's activations and scales, this unit's MFMAs
  // with the next unit's weight loads, the next activations staged; the last unit runs
  // after the loop (with an exit test between loads and their use the compiler sinks the
  // loads past it).
  for (int u = u0; u < u1 - 1; ++u) {
    const int rbn = (u + 1) / a.T, tn = u + 1 - rbn * a.T;
    const __amdgpu_buffer_rsrc_t wn = rbn == rb ? wr : mfma_wres<WT, PANEL>(a, rbn);
    mfma_load_x<NBT, KT>(a, xr, tn * KT, tid, xv);
    if (WT == M2_W_INT8G) mfma_load_s<KT>(a, sr, rbn * kMRows + lr4, tn * KT, s1);
    __builtin_amdgcn_sched_barrier(0);
    unsigned short *const xc = xs + 2 * buf * XB, *const xn = xs + 2 * (buf ^ 1) * XB;
    mfma_tile<WT, PANEL, NBT, SPG, true>(w, s0, lane, kq, xc, xc + XB, acc, wn, lb, tn * KT, a.K);
    mfma_store_x<NBT, KT, RMS>(a, tn * KT, tid, xv, xn, xn + XB, rn_s, m, rbn == rbA);
    if (EPI == kEpiPartials && rbn != rb) mfma_flush<NBT>(a, rb == rbA ? (int)blockIdx.x : G + rb, lr4, lane, acc);
    if (WT == M2_W_INT8G) {
#pragma unroll
      for (int q = 0; q < kMaxScaleGroups; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) s0[q][i] = s1[q][i];
    }
    lds_barrier();
    buf ^= 1;
    rb = rbn;
    wr = wn;
  }
  if constexpr (EPI == kEpiPartials) {
    mfma_tile<WT, PANEL, NBT, SPG, false>(w, s0, lane, kq, xs + 2 * buf * XB, xs + (2 * buf + 1) * XB, acc, wr, lb, 0,
                                          a.K);
    mfma_flush<NBT>(a, rb == rbA ? (int)blockIdx.x : G + rb, lr4, lane, acc);
  } else {
    MfmaEpi<EPI, NBT> me;
    mfma_epi_load<EPI, NBT>(g, rb * kMRows + lr4, lane, me);
    mfma_tile<WT, PANEL, NBT, SPG, false>(w, s0, lane, kq, xs + 2 * buf * XB, xs + (2 * buf + 1) * XB, acc, wr, lb, 0,
                                          a.K);
    mfma_epi_store<EPI, NBT>(g, rb * kMRows + lr4, lane, acc, me);
  }
}

// Sum of a row block's partials in workgroup order, then the row epilogue. The
// workgroups of row block rb are those holding its first and its last unit and all
// between; rb is the first row block of each but (possibly) the first of them, whose
// partial of rb is then G + rb. The partials are loaded MAXW at a time (past the last
// workgroup the offset is out of range and the load gives 0, which adds exactly), then
// added in order. out_proj: the grid also covers the conv-cache shift.
template <int EPI, int MAXW>
__global__ void gemv_mfma_reduce_kernel(GemvArgs a, const float *part, int T, int G, int part_bytes) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (EPI == EPI_OUT && a.conv_cache) conv_cache_shift(a, idx, (size_t)gridDim.x * blockDim.x);
  if (idx >= a.rows * a.B) return;
  const int b = idx / a.rows, row = idx - b * a.rows;
  const EpiIn e = epilogue_prefetch<EPI>(a, row, b);
  const int rb = row / kMRows, lr = row - rb * kMRows;
  const int U = (a.rows + kMRows - 1) / kMRows * T;   // U G < 2^31 (checked on the host)
  // the workgroup holding unit u is the last g with g U / G <= u: ((u + 1) G - 1) / U
  const int gf = ((rb * T + 1) * G - 1) / U, gl = ((rb * T + T) * G - 1) / U;
  const __amdgpu_buffer_rsrc_t pr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(part), (short)0, part_bytes, 0x00020000);
  float v = 0.0f;
  for (int g0 = gf; g0 <= gl; g0 += MAXW) {
    float pv[MAXW];
#pragma unroll
    for (int i = 0; i < MAXW; ++i) {
      const int g = g0 + i, gg = min(g, G - 1);        // past gl the offset is out of range
      const int pi = gg * U / G / T == rb ? gg : G + rb;
      const int off = g <= gl ? ((pi * a.B + b) * kMRows + lr) * 4 : kBufOutOfRange;
      pv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < MAXW; ++i) v += pv[i];
  }
  gemv_epilogue<EPI>(a, row, b, v, e);
}

// 16-row panels of a row-major [rows][K] matrix of ESZ-byte elements: fragment (p, s, l)
// (E = 8 ESZ bytes at ((p S + s) 64 + l) E, S = ceil(K / 32)) holds row 16 p + l % 16,
// k = 32 s + 8 (l / 16) .. + 8; rows past the matrix and k past K are zeros. One thread per
// fragment; element by element, so any K and alignment of a row work.
template <int ESZ>
__global__ void pack_panels_kernel(const unsigned char *w, int rows, int K, unsigned char *out, long nfrag) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nfrag) return;
  const int S = (K + 31) / 32;
  const int l = (int)(i & 63);
  const long ps = i >> 6;
  const int s = (int)(ps % S), p = (int)(ps / S);
  const int row = 16 * p + (l & 15), k0 = 32 * s + 8 * (l >> 4);
  unsigned char *o = out + i * 8 * ESZ;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = k0 + e;
    const bool ok = row < rows && k < K;
#pragma unroll
    for (int b = 0; b < ESZ; ++b) o[e * ESZ + b] = ok ? w[((size_t)row * K + k) * ESZ + b] : 0;
  }
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
  return sizeof(float) * ((size_t)BT * a.K + (PRO == PRO_NORM ? (size_t)BT * a.n_norm : 0));
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
  return sizeof(float) * ((size_t)BT * (lds_padded(a.K) + a.K / 32) + (PRO == PRO_NORM ? (size_t)BT * a.n_norm : 0));
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
      if (a.B == 1) return u3 ? launch_lowbit<WT, 1, 1, 3, 1, PRO, EPI>(a, stream) : launch_lowbit<WT, 1, 1, 5, 1, PRO, EPI>(a, stream);
      return u3 ? launch_lowbit<WT, 2, 1, 3, 1, PRO, EPI>(a, stream) : launch_lowbit<WT, 2, 1, 5, 1, PRO, EPI>(a, stream);
    }
  }
  constexpr int KS = EPI == EPI_INPROJ ? 1 : 4;
  const bool regs_ok = PRO != PRO_NORM || (a.K / 4 <= 512 * kNormF4PerThread && a.n_partials <= 512 && a.n_norm <= 512);
  // Both projections stream their weights with nontemporal loads: such loads do not allocate
  // in the last-level cache, and in a stack of layers no weight line is read again before it
  // would be evicted anyway (measured on 8 distinct 9B layers: out_proj 19.8 us with 5
  // nontemporal loads in flight per lane, 20.6 / 20.8 / 21.3 / 20.7 with 4 / 3 / 6 / 8, 21.9
  // with 8 cache-allocating ones, which only win when two layers' W_out fit the cache).
  // out_proj at one session runs 6 rows per workgroup (384 threads): its 40 KB of staged
  // activations allow 3 workgroups per CU, and 4480 rows then make one even round of 747
  // workgroups on 256 CUs (8 rows per workgroup leave 48 CUs with 3 and the rest with 2);
  // with 7 loads in flight per lane: 17.2 us against 19.5 (8 / 5 / 10 in flight: 17.5 /
  // 18.2 / 21.2; 256, 320 and 448 threads: 23.0, 21.8 and 18.5). in_proj at one session keeps
  // 3 loads per lane in flight (33.3 us against 33.55 with 5, 33.8 with 4, 34.7 with 6).
  if (a.B <= 2 && regs_ok && wave_lds_bytes(a, a.B, PRO) <= kWaveLdsMax) {
    if (EPI == EPI_OUT && PRO == PRO_NORM && a.B == 1) return launch_wave<WT, 1, 384, 7, 1, PRO, EPI>(a, stream);
    if (EPI == EPI_INPROJ && a.B == 1) return launch_wave<WT, 1, 512, 3, 1, PRO, EPI>(a, stream);
    if (a.B == 1) return launch_wave<WT, 1, 512, 5, 1, PRO, EPI>(a, stream);
    return launch_wave<WT, 2, 512, 5, 1, PRO, EPI>(a, stream);
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
  int G, T, U, nbt, ngt;
  bool whole;          // one workgroup per row block, the row epilogue in the GEMV kernel
  size_t lds;
};

// Stream-K plan: U units of one 128-row block x one 256-wide k tile over G workgroups:
// as few as give every workgroup the same number of units (to within one) with about one
// per CU of the 256-CU gfx950 parts, at least one per row block (so that a workgroup's run
// of units spans at most two row blocks) and at most one per unit. One workgroup per CU
// streamed fastest on MI355X (73 / 146 / 75 us per step at 4 and 32 bf16 sessions and 8
// int8 sessions, against 77 / 158 / 78 with two per CU and 82 / 161 / 83 with 320 in all);
// more loads in flight only queue behind the HBM's capacity. The plan needs no HIP call,
// so workspace sizes can be computed on the host alone.
constexpr int kMfmaGrid = 256;

// With bf16 weights and at least this many row blocks, a workgroup per row block keeps
// the HBM about as busy as the balanced stream-K grid, and its sums need no second
// kernel: the in_proj of the 9B-shaped layer (177 row blocks of 4480) ran 1.3 / 2.8 us
// longer at 4 / 32 sessions than over 246 workgroups, against 4.7 / 6.9 us for the
// reduction it drops. int8 weights lost 2 us net (their tiles cost more ALU per byte).
constexpr int kMfmaWholeMinBlocks = 160;

// `whole_ok`: the caller can take the row epilogue in the GEMV kernel (no RMS prologue, no
// conv-cache shift).
MfmaPlan mfma_plan(int wtype, int rows, int K, int B, int ng, bool whole_ok) {
  MfmaPlan p;
  p.nbt = B <= 16 ? 1 : 2;
  const int kt = wtype == M2_W_INT8G ? mfma_kt<M2_W_INT8G>() : mfma_kt<M2_W_BF16>();
  const int rbn = (rows + kMRows - 1) / kMRows;
  p.T = (K + kt - 1) / kt;
  p.U = rbn * p.T;
  const int per = (p.U + kMfmaGrid - 1) / kMfmaGrid;
  p.whole = whole_ok && ng == 0 && wtype == M2_W_BF16 && rbn >= kMfmaWholeMinBlocks;
  p.G = p.whole ? rbn : std::max((p.U + per - 1) / per, std::min(p.U, rbn));
  const int upw = (p.U + p.G - 1) / p.G;               // units per workgroup, at most
  p.ngt = ng > 0 ? upw * kt / ng + 4 : 0;              // norm groups its two k ranges can touch
  p.lds = 4 * sizeof(unsigned short) * (size_t)p.nbt * 16 * (kt + 8) + sizeof(float) * (size_t)B * p.ngt;
  return p;
}

size_t mfma_part_floats(const MfmaPlan &p, int B) { return p.whole ? 0 : (size_t)(p.G + p.U / p.T) * B * kMRows; }

// The reduction of a plan's partials (and, out_proj, the conv-cache shift): one thread per
// output, or per conv element if those are more.
template <int EPI>
hipError_t launch_mfma_reduce(const GemvArgs &g, const MfmaPlan &p, float *part, hipStream_t stream) {
  const long pbytes = (long)mfma_part_floats(p, g.B) * 4;
  if ((long)p.U * p.G >= (1L << 31) || pbytes >= kBufOutOfRange) return hipErrorInvalidValue;
  // workgroups of a row block: its T units over runs of at least U / G units each (more
  // than 32 are summed in batches of 32)
  const int minrun = std::max(1, p.U / p.G);
  const int maxw = (p.T + minrun - 1) / minrun + 1;
  long n = (long)g.rows * g.B;
  if (EPI == EPI_OUT && g.conv_cache) n = std::max(n, (long)g.B * g.conv_dim);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (maxw <= 4)
    hipLaunchKernelGGL((gemv_mfma_reduce_kernel<EPI, 4>), grid, block, 0, stream, g, part, p.T, p.G, (int)pbytes);
  else if (maxw <= 8)
    hipLaunchKernelGGL((gemv_mfma_reduce_kernel<EPI, 8>), grid, block, 0, stream, g, part, p.T, p.G, (int)pbytes);
  else if (maxw <= 16)
    hipLaunchKernelGGL((gemv_mfma_reduce_kernel<EPI, 16>), grid, block, 0, stream, g, part, p.T, p.G, (int)pbytes);
  else
    hipLaunchKernelGGL((gemv_mfma_reduce_kernel<EPI, 32>), grid, block, 0, stream, g, part, p.T, p.G, (int)pbytes);
  return hipGetLastError();
}

template <int WT, bool PANEL, int NBT, bool RMS, int SPG, int EPI>
hipError_t launch_mfma_k(const MfmaArgs &m, const GemvArgs &g, const MfmaPlan &p, hipStream_t stream) {
  auto *k = gemv_mfma_kernel<WT, PANEL, NBT, RMS, SPG, EPI>;
  hipError_t e = allow_lds(k, p.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(p.G), dim3(512), p.lds, stream, m, g);
  return hipGetLastError();
}

// The in-kernel epilogue exists for bf16 weights and the in_proj epilogue only (the plans
// that choose it).
template <int WT, bool PANEL, bool RMS, int SPG>
hipError_t launch_mfma_nbt(const MfmaArgs &m, const GemvArgs &g, int epi, const MfmaPlan &p, hipStream_t stream) {
  if constexpr (WT == M2_W_BF16 && !RMS) {
    if (p.whole) {
      if (epi != EPI_INPROJ) return hipErrorInvalidValue;
      return p.nbt == 1 ? launch_mfma_k<WT, PANEL, 1, RMS, SPG, EPI_INPROJ>(m, g, p, stream)
                        : launch_mfma_k<WT, PANEL, 2, RMS, SPG, EPI_INPROJ>(m, g, p, stream);
    }
  }
  if (p.whole) return hipErrorInvalidValue;
  return p.nbt == 1 ? launch_mfma_k<WT, PANEL, 1, RMS, SPG, kEpiPartials>(m, g, p, stream)
                    : launch_mfma_k<WT, PANEL, 2, RMS, SPG, kEpiPartials>(m, g, p, stream);
}

// The kernels' buffer offsets (a row block of W or of its panels, the activations [B][K],
// the scales, with the out-of-range marker above all) and U G must stay below 2^31.
template <int WT, bool PANEL, bool RMS>
hipError_t launch_mfma(const MfmaArgs &m, const GemvArgs &g, int epi, const MfmaPlan &p, hipStream_t stream) {
  const long esz = WT == M2_W_BF16 ? 2 : 1;
  const long kpad = PANEL ? (long)(m.K + 31) / 32 * 32 : m.K;
  if ((long)kMRows * kpad * esz >= kBufOutOfRange || (long)m.B * m.K * 4 >= kBufOutOfRange ||
      (long)m.rows * (m.K / m.q_group) * 2 >= kBufOutOfRange || (long)p.U * p.G >= (1L << 31))
    return hipErrorInvalidValue;
  if constexpr (WT == M2_W_BF16) {
    return launch_mfma_nbt<WT, PANEL, RMS, 8>(m, g, epi, p, stream);
  } else {
    if (m.q_group == 128) return launch_mfma_nbt<WT, PANEL, RMS, 4>(m, g, epi, p, stream);
    if (m.q_group == 256) return launch_mfma_nbt<WT, PANEL, RMS, 8>(m, g, epi, p, stream);
    return hipErrorInvalidValue;
  }
}

// `g`, `epi`: the row epilogue of a whole-row-block plan (unused otherwise).
template <bool RMS>
hipError_t launch_mfma_wt(int wtype, bool panel, const MfmaArgs &m, const GemvArgs &g, int epi, const MfmaPlan &p,
                          hipStream_t stream) {
  if (wtype == M2_W_BF16)
    return panel ? launch_mfma<M2_W_BF16, true, RMS>(m, g, epi, p, stream)
                 : launch_mfma<M2_W_BF16, false, RMS>(m, g, epi, p, stream);
  return panel ? launch_mfma<M2_W_INT8G, true, RMS>(m, g, epi, p, stream)
               : launch_mfma<M2_W_INT8G, false, RMS>(m, g, epi, p, stream);
}

// One MFMA GEMV + reduce for the arguments of a gemv_* launch, from the 16-row panels of
// the weights when given; out_proj (EPI_OUT) also forms the RMS factors from g.ss. An
// in_proj plan of whole row blocks applies the epilogue in the GEMV kernel and needs no
// reduction.
template <int EPI>
hipError_t run_mfma_gemv(const m2_config &c, const GemvArgs &g, const void *panels, float *part,
                         hipStream_t stream) {
  constexpr bool RMS = EPI == EPI_OUT;
  const MfmaPlan p = mfma_plan(c.wtype, g.rows, g.K, g.B, RMS ? g.ng : 0, EPI == EPI_INPROJ);
  MfmaArgs m{};
  m.W = panels ? panels : g.W;
  m.S = static_cast<const __half *>(g.S);
  m.rows = g.rows;
  m.K = g.K;
  m.q_group = c.wtype == M2_W_INT8G ? c.q_group : g.K;
  m.T = p.T;
  m.U = p.U;
  m.nks = (g.K + 31) / 32;
  m.act = g.act;
  m.B = g.B;
  m.ss = g.ss;
  m.n_partials = g.n_partials;
  m.n_norm = g.n_norm;
  m.ng = g.ng;
  m.eps = g.eps;
  m.ngt = p.ngt;
  m.part = part;
  hipError_t e = launch_mfma_wt<RMS>(c.wtype, panels != nullptr, m, g, EPI, p, stream);
  if (e != hipSuccess || p.whole) return e;
  return launch_mfma_reduce<EPI>(g, p, part, stream);
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
  w.bar = p ? reinterpret_cast<unsigned *>(p + off) : nullptr;
  off += align256(kBarBytes);
  if (step_uses_mfma(L, batch)) {
    const MfmaPlan pi = mfma_plan(L.cfg.wtype, L.d_in_proj, L.cfg.d_model, batch, 0, true);
    const MfmaPlan po = mfma_plan(L.cfg.wtype, L.cfg.d_model, L.d_inner, batch, L.ng, false);
    const size_t n_in = mfma_part_floats(pi, batch), n_out = mfma_part_floats(po, batch);
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
  // one or two sessions: items of 10 waves x 2 slices for 17-20 slice instructions (the 9B
  // layer's 40-row items: step 18,440 against 18,389 steps/s with 8 x 3, 18,429 with 12 x 2,
  // 18,226 with 5 x 4, same box, two repeats each)
  // 3 or more sessions, 17-20 slice instructions (the 9B layer's 40-row items): 4 waves x 5
  // slices up to 4 sessions, 2 x 10 beyond (4 sessions: 15,340 / 15,006 steps/s with 4 x 5 /
  // 2 x 10; 8 int8 sessions: 564 / 572 stack steps/s)
  if (batch > 2 && batch <= 4 && n_inst > 16 && n_inst <= 20) {
    hipLaunchKernelGGL((ssd_step_kernel<4, 5>), grid, dim3(256), 0, stream, sa);
    return hipGetLastError();
  }
  if (batch > 4 && n_inst > 16 && n_inst <= 20) {
    hipLaunchKernelGGL((ssd_step_kernel<2, 10>), grid, dim3(128), 0, stream, sa);
    return hipGetLastError();
  }
  if (batch <= 2 && n_inst <= 16)
    hipLaunchKernelGGL((ssd_step_kernel<8, 2>), grid, dim3(512), 0, stream, sa);
  else if (batch <= 2 && n_inst <= 20)
    hipLaunchKernelGGL((ssd_step_kernel<10, 2>), grid, dim3(640), 0, stream, sa);
  else if (batch <= 2 && n_inst <= 24)
    hipLaunchKernelGGL((ssd_step_kernel<8, 3>), grid, dim3(512), 0, stream, sa);
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
  const int plan = step_plan(L, batch, flags);
  if (plan == kPlanFused) {
    // in_proj as in plan 0 (it also zeroes the next kernel's barrier counter), then the
    // SSD and out_proj in one persistent kernel
    gi.bar_clear = ws.bar;
    e = launch_wave<M2_W_BF16, 1, 512, 3, 1, PRO_PLAIN, EPI_INPROJ>(gi, stream);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = launch_fused_step(L, S, x, y, slots, flags, ws, fused_grid(L), stream);
    for (int i = 2; i < 4 && e == hipSuccess; ++i) e = mark(i);
    return e;
  }
  const bool mfma = plan == kPlanMfma;
  e = mfma ? run_mfma_gemv<EPI_INPROJ>(c, gi, L.w.w_in_panels, ws.part, stream)
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
  // SSD items of twice the layer's row range where it still divides the head and the RMS
  // group and fits the items below (measured on the 9B layer, 40 rows instead of 20: at one
  // session the SSD 6.9 against 7.1 us, and out_proj sums half the partials, step +0.43 % on
  // one box, three repeats each, where two 20-row ranges per item with a partial each gave
  // +0.08 %; 4 sessions +0.6 %, the 8-session int8 stack 558 -> 572 stack steps/s, 32 sessions
  // 7,470 -> 7,563 steps/s). The partials then number half of the workspace's n_partials.
  {
    const int pr2 = 2 * L.prange, rpi = 64 / (c.d_state / 4);
    if (L.psplit % 2 == 0 && L.ng % pr2 == 0 && pr2 <= 64 && (pr2 + rpi - 1) / rpi <= 24) {
      sa.prange = pr2;
      sa.psplit = L.psplit / 2;
      sa.n_partials = L.n_partials / 2;
    }
  }

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
  go.n_partials = sa.n_partials;
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
  e = launch_ssd(sa, c.n_heads * sa.psplit, batch, stream);
  if (e == hipSuccess) e = mark(2);
  if (e != hipSuccess) return e;
  if (mfma) {
    e = run_mfma_gemv<EPI_OUT>(c, go, L.w.w_out_panels, ws.part, stream);
  } else {
    e = dispatch_wt<PRO_NORM, EPI_OUT>(c.wtype, go, stream);
  }
  if (e == hipSuccess) e = mark(3);
  return e;
}

// Batches of 3..32 sessions with bf16 weights, or int8 weights in groups of 128 or
// 256, run the projections as MFMA GEMVs; the rest as VALU GEMVs.
int step_plan(const m2_layer_s &L, int batch, int flags) {
  const m2_config &c = L.cfg;
  if ((flags & M2_PERSISTENT) && batch == 1 && c.wtype == M2_W_BF16 && fused_fits(L, fused_grid(L)))
    return kPlanFused;
  if (batch < 3 || batch > 32) return kPlanValu;
  if (c.wtype == M2_W_BF16) return kPlanMfma;
  return c.wtype == M2_W_INT8G && (c.q_group == 128 || c.q_group == 256) ? kPlanMfma : kPlanValu;
}

bool step_uses_mfma(const m2_layer_s &L, int batch) { return step_plan(L, batch) == kPlanMfma; }


size_t panels_bytes(int wtype, int rows, int K) {
  if ((wtype != M2_W_BF16 && wtype != M2_W_INT8G) || rows <= 0 || K <= 0) return 0;
  const size_t esz = wtype == M2_W_BF16 ? 2 : 1;
  return (size_t)((rows + 15) / 16) * ((K + 31) / 32) * 64 * 8 * esz;
}

hipError_t launch_pack_panels(int wtype, const void *w, int rows, int K, void *out, hipStream_t stream) {
  const long nfrag = (long)((rows + 15) / 16) * ((K + 31) / 32) * 64;
  const dim3 grid((unsigned)((nfrag + 255) / 256));
  if (wtype == M2_W_BF16)
    hipLaunchKernelGGL(pack_panels_kernel<2>, grid, dim3(256), 0, stream, static_cast<const unsigned char *>(w), rows,
                       K, static_cast<unsigned char *>(out), nfrag);
  else
    hipLaunchKernelGGL(pack_panels_kernel<1>, grid, dim3(256), 0, stream, static_cast<const unsigned char *>(w), rows,
                       K, static_cast<unsigned char *>(out), nfrag);
  return hipGetLastError();
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

bool gemv_plain_uses_mfma(int wtype, int q_group, int batch) {
  if (batch < 3 || batch > 32) return false;
  return wtype == M2_W_BF16 || (wtype == M2_W_INT8G && (q_group == 128 || q_group == 256));
}

size_t gemv_plain_part_bytes(int wtype, int q_group, int rows, int K, int batch) {
  if (!gemv_plain_uses_mfma(wtype, q_group, batch)) return 0;
  const MfmaPlan p = mfma_plan(wtype, rows, K, batch, 0, false);
  return sizeof(float) * mfma_part_floats(p, batch);
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
    const MfmaPlan p = mfma_plan(wtype, rows, K, batch, 0, false);
    MfmaArgs m{};
    m.W = W;
    m.S = static_cast<const __half *>(S);
    m.rows = rows;
    m.K = K;
    m.q_group = wtype == M2_W_INT8G ? q_group : K;
    m.T = p.T;
    m.U = p.U;
    m.nks = (K + 31) / 32;
    m.act = act;
    m.B = batch;
    m.part = part;
    hipError_t e = launch_mfma_wt<false>(wtype, false, m, a, EPI_OUT, p, stream);
    if (e != hipSuccess) return e;
    return launch_mfma_reduce<EPI_OUT>(a, p, part, stream);
  }
  // 1-2 sessions, 2- and 4-byte weights: one wave per row, 5 nontemporal loads in flight;
  // bf16 at one session with 6 rows per workgroup (384 threads): measured on the attention
  // layer's projections (7168 x 4480 and 4480 x 5120, 23 rotating copies), 13.2 and 10.2 us
  // against 13.9 and 11.0 with 8 rows (256 / 768 threads: 13.8 / 15.0 and 10.7 / 10.6; 3, 7
  // or 8 loads in flight slower); otherwise the decode step's choice for out_proj.
  if (batch <= 2 && (wtype == M2_W_BF16 || wtype == M2_W_F32) && wave_lds_bytes(a, batch, PRO_PLAIN) <= kWaveLdsMax) {
    if (wtype == M2_W_BF16)
      return batch == 1 ? launch_wave<M2_W_BF16, 1, 384, 5, 1, PRO_PLAIN, EPI_OUT>(a, stream)
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
