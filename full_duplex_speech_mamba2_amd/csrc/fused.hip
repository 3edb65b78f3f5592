// SSD and out_proj of the decode step in one persistent launch, on gfx950 (one session,
// bf16 weights): the step's plan 2, after the in_proj GEMV of decode.hip.
//
// The step is bound by streaming the two projection matrices from HBM (page
// "NemotronLabs VoiceChat 11B: GPTQ 3-bit LLM, MLX", introduction: the LLM step is limited
// by memory bandwidth). With one kernel for the SSD update and one for out_proj, the HBM
// stream stops between in_proj and out_proj for the whole SSD kernel, a short kernel bound
// by the latency of its state loads, and again while out_proj's first loads are in flight.
// Here the workgroups of one kernel, all resident at once (two per CU), issue the loads of
// their SSD item (state tile, gate and conv inputs), then the first third of their out_proj
// weights, which stream in while the item is computed; they arrive at one grid-wide barrier
// (the SSD's output v and its sums of squares complete), issue the second third while they
// wait, and finish out_proj. (Loads complete in issue order as far as a wave's wait counts
// go, so weights requested before the item's own inputs would delay the item.)
//
//   SSD      workgroup w takes item w (head, range of head rows) as the three-kernel step's
//            SSD kernel does; its barriers order LDS only, so the weight loads stay in
//            flight; v and the sums of squares are stored past the per-XCD caches; the
//            updated state tile is written after the workgroup has arrived at the barrier
//            (nothing in the launch reads it again).
//   out_proj workgroup w owns a contiguous block of at most 9 rows and wave j of it the j-th
//            eighth of every row's chunks, so every wave moves the same bytes; v is staged
//            with coalesced loads past the caches, scaled by its RMS factor, into LDS; the 8
//            waves' row sums meet in LDS and are added in a fixed order; the conv-cache
//            shift runs here too (the SSD, its last reader, has finished).
//
// Grid barrier: each wave waits for its stores to complete and counts itself in LDS; wave 0
// then counts the workgroup in its group's counter (8 groups, so that no address takes the
// atomics of the whole grid, which serialise at the memory), the group's last workgroup
// counts the group, the last group raises every group's flag; wave 0 polls its group's flag
// (words zeroed by the in_proj kernel before this launch) and releases the other waves
// through an LDS flag, so only wave 0 waits on memory. (With one counter for all 512
// workgroups the barrier took ~20 us.) The data crossing the barrier bypasses the per-XCD caches (loads and
// stores with the sc1 policy), so no cache write-back or invalidation is needed. Every wait
// is bounded: were the grid not all resident the kernel would still finish (and raise a
// flag) instead of hanging. Measured forms, not kept: the in_proj GEMV in the same kernel
// (a third phase, a second barrier) ran at 5 TB/s against 6.3 for its own kernel, since a
// persistent grid's fixed row assignment leaves slow waves no one takes work from; and
// barriers that wrote back and invalidated the L2 (plain accesses to the shared data).
#include "decode_common.h"

#include <algorithm>
#include <cstring>

namespace m2d {
namespace {

constexpr int kFThreads = 512;
constexpr int kFWaves = kFThreads / 64;
constexpr int kFJC = 3;        // out_proj: chunks per lane of a wave's eighth of a row (<= 192 chunks)
constexpr int kFRMax = 9;      // out_proj: rows per workgroup
constexpr int kFDepth = 4;     // out_proj: rows of a wave in flight while one is multiplied
constexpr int kFMaxI = 2;      // SSD: state slices per wave (items of up to 16 wave instructions)
constexpr int kFGroups = 4;    // out_proj: RMS groups an eighth of a row may touch
// Bounds of the barrier waits, in polls: LDS polls take ~0.1 us, global ones about a memory
// latency (~1 us); a wave waiting on LDS outlasts wave 0's two waits together.
constexpr unsigned kLdsSpin = 1u << 22;
constexpr unsigned kGlobalSpin = 1u << 18;

typedef float f32x4b __attribute__((ext_vector_type(4)));

struct FusedArgs {
  GemvArgs go;
  SsdArgs sa;
  unsigned *bar;       // the grid-barrier words (kBar*, zeroed before the launch)
  int items;           // SSD items: H * psplit (one session)
};

struct BarCtl {
  unsigned arrived;    // waves 1..7 arrived, counted over the launch
  unsigned go;         // number of the last barrier wave 0 has passed
};

// LDS words polled by the waves of one workgroup (relaxed atomics, so that they stay LDS
// instructions and a poll never waits for the wave's global loads in flight)
__device__ __forceinline__ unsigned lds_load(unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Grid-wide barrier number `gen` of the launch: every global store a wave made before it is
// complete before any wave passes it. `after_arrival()` is called once by every wave after
// its workgroup's arrival is counted, before the wave waits -- except wave 0, which polls
// memory (each poll waits for all of the wave's earlier memory operations): it calls it
// once the barrier is passed.
template <typename F>
__device__ __forceinline__ void grid_barrier(unsigned *bar, BarCtl *ctl, unsigned gen, int wave, int lane,
                                             F &&after_arrival) {
  // this wave's stores complete: a workgroup-scope release does not wait for them (waves of
  // a workgroup share the L1), and an agent-scope one would also write back the L2, which
  // data stored past the caches does not need; so an explicit wait for every counter
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (wave != 0) {
    if (lane == 0) __hip_atomic_fetch_add(&ctl->arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    after_arrival();
    for (unsigned n = 0; lds_load(&ctl->go) < gen && n < 4 * kLdsSpin; ++n) __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return;
  }
  for (unsigned n = 0; lds_load(&ctl->arrived) < gen * (kFWaves - 1) && n < kLdsSpin; ++n)
    __builtin_amdgcn_s_sleep(1);
  // two levels, so that no address takes more than a group's worth of atomics: the last
  // workgroup of a group counts the group complete, the last group releases every group
  if (lane == 0) {
    const int grp = blockIdx.x % kBarGroups;
    const unsigned members = (gridDim.x - grp + kBarGroups - 1) / kBarGroups;
    const unsigned groups = gridDim.x < kBarGroups ? gridDim.x : kBarGroups;
    unsigned *flag = bar + (kBarFlag + grp) * kBarStride;
    unsigned *err = bar + kBarError * kBarStride;
    if (__hip_atomic_fetch_add(bar + (kBarCount + grp) * kBarStride, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == gen * members - 1) {
      if (__hip_atomic_fetch_add(bar + kBarTop * kBarStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          gen * groups - 1) {
        for (unsigned q = 0; q < groups; ++q)
          __hip_atomic_store(bar + (kBarFlag + q) * kBarStride, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // once any wait has run out (the error word raised), no later barrier waits at all, so
    // a launch with many barriers still ends after one bound's time
    unsigned n = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < gen &&
           __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      if (++n > kGlobalSpin) {
        __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane == 0) __hip_atomic_store(&ctl->go, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  after_arrival();
}

// ---------------------------------------------------------------------------
// out_proj rows [r0, r0 + nr) of this workgroup, this wave's chunks [s0, s1) of them. The
// weights are read through a buffer resource over W_out: a row past the block or a chunk
// past the eighth takes an offset past the resource, which returns zeros without a memory
// access, so every load is unconditional and the compiler's wait counts stay exact.
struct OutRow {
  u32x4 w[kFJC];
};

__device__ __forceinline__ void out_row_load(__amdgpu_buffer_rsrc_t wr, int NC, int r0, int nr, int rl, int s0,
                                             int s1, int lane, OutRow &o) {
#pragma unroll
  for (int j = 0; j < kFJC; ++j) {
    const int c = s0 + lane + 64 * j;
    const int off = (rl < nr && c < s1) ? ((r0 + rl) * NC + c) * 16 : kBufOutOfRange;
    const f32x4b v = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
    o.w[j] = u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  }
}

// act: the RMS-scaled activations in LDS, [K]
__device__ __forceinline__ float out_row_dot(int s0, int s1, int lane, const OutRow &o, const float *act) {
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kFJC; ++j) {
    const int c = s0 + lane + 64 * j;
    if (c < s1) s += chunk_dot<M2_W_BF16>(o.w[j], act + 8 * c);
  }
  return s;
}

// ---------------------------------------------------------------------------
// The SSD item of this workgroup, one grid barrier (number `gen` of the launch), then its
// out_proj rows (+ residual) and its share of the conv-cache shift. Called by every thread.
// STACK: inside the persistent stack kernel, where zx, the residual input and y are
// written and read by other workgroups of the same launch: all of them go past the per-XCD
// caches (zx and the residual input read, y stored). LDS: fused_lds_bytes; ctl initialised.
// The workgroup's SSD item: which it is (without one of its own, a copy of the last, never
// written), and its state tile's loads.
struct FItem {
  bool has;
  int h, ps;
};

__device__ __forceinline__ FItem fused_item(const SsdArgs &sa, int items) {
  FItem it;
  it.has = (int)blockIdx.x < items;
  const int item = it.has ? (int)blockIdx.x : items - 1;
  it.h = item / sa.psplit;
  it.ps = item - it.h * sa.psplit;
  return it;
}

__device__ __forceinline__ void fused_tile_load(const SsdArgs &sa, const FItem &it, int wave, int lane,
                                                SsdTile<kFMaxI> &tile) {
  const int slot = sa.slots ? sa.slots[0] : 0;
  ssd_load<kFWaves, kFMaxI>(sa, it.h, it.ps, slot, wave, lane, tile);
}

template <bool STACK>
__device__ __forceinline__ void ssd_out_phase(const GemvArgs &go, const SsdArgs &sa, unsigned *bar, const FItem &it,
                                              SsdTile<kFMaxI> &tile, BarCtl *ctl, unsigned gen, float *lds, int tid,
                                              int lane, int wave) {
  const int nwg = gridDim.x;
  const int slot = go.slots ? go.slots[0] : 0;          // the session's slot, read once
  const bool sok = slot >= 0 && slot < go.n_slots;
  const bool has_item = it.has;
  const int h = it.h, ps = it.ps;
  const int r0 = (int)(((long)blockIdx.x * go.rows) / nwg);
  const int nr = (int)(((long)(blockIdx.x + 1) * go.rows) / nwg) - r0;
  const int NC = go.K / 8, per_w = (NC + kFWaves - 1) / kFWaves;
  const int s0 = min(wave * per_w, NC), s1 = min(s0 + per_w, NC);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(go.W), (short)0,
                                                                      go.rows * NC * 16, 0x00020000);
  OutRow rows[kFDepth + 1];                          // a ring: row k in rows[k % (kFDepth + 1)]

  // ---- SSD item (the workgroup barriers inside order LDS only); once its own loads are
  // all issued, the first out_proj row (more would only queue behind the HBM's capacity and
  // hold up the issue of the item's work)
  float *wsum = lds;
  float *cx = lds + 16;
  ssd_finish<kFWaves, kFMaxI, false, true, STACK>(sa, h, ps, 0, slot, wave, lane, tile, wsum, cx, has_item, [&] {
    // every slice register of the tile counts as used here, also on paths where the item
    // leaves it untouched, so that the compiler waits for the tile's loads now (not for
    // the weight loads issued next), and not again at the tile's store
#pragma unroll
    for (int k = 0; k < kFMaxI; ++k)
      asm volatile("" : "+v"(tile.st[k].x), "+v"(tile.st[k].y), "+v"(tile.st[k].z), "+v"(tile.st[k].w));
    out_row_load(wr, NC, r0, nr, 0, s0, s1, lane, rows[0]);
  });

  // ---- grid barrier: v and the sums of squares complete; after arriving, the state tile
  grid_barrier(bar, ctl, gen, wave, lane, [&] { ssd_store<kFMaxI>(sa, h, has_item ? slot : -1, lane, tile); });

  // ---- out_proj (+ residual), conv-cache shift
  conv_cache_shift<STACK>(go, (size_t)blockIdx.x * kFThreads + tid, (size_t)nwg * kFThreads);
  if (nr <= 0) return;                               // uniform over the workgroup
  float *act = lds;                                  // [K]: this wave's eighth, scaled
  float *red = lds + go.K;                           // [kFWaves][kFRMax]
  float acc[kFRMax];
#pragma unroll
  for (int i = 0; i < kFRMax; ++i) acc[i] = 0.0f;
  const float rv = (tid < nr && go.resid) ? ldc<STACK>(go.resid + r0 + tid) : 0.0f;
  if (s1 > s0) {
    // first the loads the staging of v needs (the partial sums of squares of the groups this
    // wave's chunks touch, v of its eighth, coalesced, both past the caches), then the next
    // out_proj rows: waiting for the former then never waits for the latter
    const int g_lo = (8 * s0) / go.ng, g_hi = (8 * s1 - 1) / go.ng;
    const int per = go.n_partials / go.n_norm;
    float sq[kFGroups];
#pragma unroll
    for (int gq = 0; gq < kFGroups; ++gq) {
      const int g = min(g_lo + gq, g_hi);
      float sum = 0.0f;
      for (int p = lane; p < per; p += 64) sum += ldc<true>(go.ss + g * per + p);
      sq[gq] = sum;
    }
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(go.act), (short)0,
                                                                        go.K * 4, 0x00020000);
    constexpr int kV = 2 * 64 * kFJC / 64;           // float4s of v per lane (an eighth of <= 192 chunks)
    f32x4b vv[kV];
#pragma unroll
    for (int k = 0; k < kV; ++k) {
      const int i4 = 2 * s0 + lane + 64 * k;
      vv[k] = __builtin_amdgcn_raw_buffer_load_b128(vr, i4 < 2 * s1 ? i4 * 16 : kBufOutOfRange, 0, 16);   // sc1
    }
#pragma unroll
    for (int k = 1; k <= kFDepth; ++k) out_row_load(wr, NC, r0, nr, k, s0, s1, lane, rows[k]);
    float rf[kFGroups];
#pragma unroll
    for (int gq = 0; gq < kFGroups; ++gq) rf[gq] = 1.0f / sqrtf(group_reduce<64>(sq[gq]) / (float)go.ng + go.eps);
#pragma unroll
    for (int k = 0; k < kV; ++k) {
      const int i4 = 2 * s0 + lane + 64 * k;
      if (i4 < 2 * s1) {
        const int q = (4 * i4) / go.ng - g_lo;
        float fq = rf[0];
#pragma unroll
        for (int gq = 1; gq < kFGroups; ++gq) fq = q == gq ? rf[gq] : fq;
        *reinterpret_cast<float4 *>(act + 4 * i4) = make_float4(vv[k].x * fq, vv[k].y * fq, vv[k].z * fq, vv[k].w * fq);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);         // LDS writes of this wave before its reads
    // rows in order, kFDepth of them in flight
#pragma unroll
    for (int k = 0; k < kFRMax; ++k) {
      acc[k] = out_row_dot(s0, s1, lane, rows[k % (kFDepth + 1)], act);
      if (k + kFDepth + 1 < kFRMax)
        out_row_load(wr, NC, r0, nr, k + kFDepth + 1, s0, s1, lane, rows[(k + kFDepth + 1) % (kFDepth + 1)]);
    }
#pragma unroll
    for (int i = 0; i < kFRMax; ++i) acc[i] = group_reduce<64>(acc[i]);
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < kFRMax; ++i) red[wave * kFRMax + i] = acc[i];
  }
  __syncthreads();
  if (tid < nr) {
    const int row = r0 + tid;
    float s = 0.0f;
    for (int w = 0; w < kFWaves; ++w) s += red[w * kFRMax + tid];
    s *= go.gamma;
    stc<STACK>(go.y + row, sok ? s + rv : __builtin_nanf(""));
  }
}

// 16 waves per CU (two workgroups): at most 128 VGPRs
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void fused_ssd_out_kernel(FusedArgs f) {
  extern __shared__ float lds[];
  __shared__ BarCtl ctl;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    ctl.arrived = 0;
    ctl.go = 0;
  }
  // the SSD item's state tile first
  const FItem it = fused_item(f.sa, f.items);
  SsdTile<kFMaxI> tile;
  fused_tile_load(f.sa, it, wave, lane, tile);
  ssd_out_phase<false>(f.go, f.sa, f.bar, it, tile, &ctl, 1, lds, tid, lane, wave);
}

// ---------------------------------------------------------------------------
// The persistent stack step: every Mamba-2 mixer of a run of consecutive layers (one
// session, bf16) in one launch, three phases per layer with a grid barrier after each:
// in_proj | SSD (+ the barrier inside ssd_out_phase) | out_proj + residual. Between layers the
// residual stream u_{l+1} = u_l + mixer_l(u_l) goes through a buffer of its own per layer,
// as do zx, v and the sums of squares, so that nothing a phase reads was read or written
// earlier in the launch at another address's behest: each is written once (past the per-XCD
// caches) and read after a barrier (past them too).

// in_proj of one session, as the three-kernel step's wave GEMV computes it: one wave per
// row, lane l summing the row's 8-element chunks l, l + 64, ... in order, then the same
// cross-lane tree and epilogue, so the results are bitwise that kernel's. Wave gw of the
// grid's nw takes rows gw, gw + nw, ... A row is at most kIJ chunks per lane (d_model <=
// 4608), all requested at once; each register is refilled with the same chunk of the wave's
// next row as soon as it has been used, so the wave keeps a row's loads in flight across its
// reductions and epilogues, and the first row's loads are requested before the barrier the
// phase starts after (weights do not depend on the data). Loads go through a buffer resource:
// a chunk past the row or a row past the matrix reads zeros without a memory access, so no
// load is conditional. x is staged into LDS and zx stored past the per-XCD caches.
constexpr int kIJ = 9;          // chunks per lane of one row

struct InRow {
  u32x4 w[kIJ];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t inproj_rsrc(const GemvArgs &gi) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(gi.W), (short)0, gi.rows * (gi.K / 8) * 16, 0x00020000);
}

__device__ __forceinline__ u32x4 inproj_chunk(__amdgpu_buffer_rsrc_t wr, const GemvArgs &gi, int row, int j, int lane) {
  const int NC = gi.K / 8, c = lane + 64 * j;
  const int off = (row < gi.rows && c < NC) ? (row * NC + c) * 16 : kBufOutOfRange;
  const f32x4b v = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2);     // nt
  return u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
}

// the first row of this wave, before the phase's barrier
__device__ __forceinline__ void inproj_first(const GemvArgs &gi, int wave, int lane, InRow &r) {
  const __amdgpu_buffer_rsrc_t wr = inproj_rsrc(gi);
  const int row = blockIdx.x * kFWaves + wave;
#pragma unroll
  for (int j = 0; j < kIJ; ++j) r.w[j] = inproj_chunk(wr, gi, row, j, lane);
}

__device__ __forceinline__ void inproj_phase(const GemvArgs &gi, InRow &r, float *lds, int tid, int lane, int wave) {
  const int nw = gridDim.x * kFWaves;
  const int K = gi.K, NC = K / 8;
  const int slot = gi.slots ? gi.slots[0] : 0;
  const bool sok = slot >= 0 && slot < gi.n_slots;
  const __amdgpu_buffer_rsrc_t wr = inproj_rsrc(gi);
  for (int i = tid; i < K; i += kFThreads) lds[i] = ldc<true>(gi.act + i);
  __syncthreads();
  const int dt0 = gi.d_inner + gi.conv_dim;
  for (int row = blockIdx.x * kFWaves + wave; row < gi.rows; row += nw) {   // uniform over the wave
    const int next = row + nw;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kIJ; ++j) {
      const int c = lane + 64 * j;
      if (c < NC) acc = chunk_acc<M2_W_BF16>(r.w[j], lds + c * 8, QScale{1.0f, 0.0f}, acc);
      r.w[j] = inproj_chunk(wr, gi, next, j, lane);
    }
    acc = group_reduce<64>(acc);
    if (lane == 0) {
      float val = acc * gi.gamma;
      if (row >= dt0) val = softplus(val + gi.dt_bias[row - dt0]);
      stc<true>(gi.zx + row, sok ? val : __builtin_nanf(""));
    }
  }
}

// One mixer layer of the table: the three phases' arguments with every pointer of the call
// left out, and the byte offsets of the layer's buffers in the persistent area.
struct StackRec {
  GemvArgs gi, go;
  SsdArgs sa;
  int items;
  long long zx_off, v_off, ss_off, u_off;
};

struct StackArgs {
  const StackRec *tab;    // device table, one record per layer of the stack
  int l0, l1;             // the run: layers [l0, l1), all mixers
  char *area;             // the barrier words, then each layer's buffers
  float *y;               // the residual stream: the run's input and its output
  const int32_t *slots;
  int n_slots;
};

__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void stack_persistent_kernel(StackArgs a) {
  extern __shared__ float lds[];
  __shared__ BarCtl ctl;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    ctl.arrived = 0;
    ctl.go = 0;
  }
  __syncthreads();
  unsigned *bar = reinterpret_cast<unsigned *>(a.area);
  unsigned gen = 0;
  const float *u = a.y;
  InRow w;
  inproj_first(a.tab[a.l0].gi, wave, lane, w);
  for (int l = a.l0; l < a.l1; ++l) {
    const StackRec &r = a.tab[l];
    float *zx = reinterpret_cast<float *>(a.area + r.zx_off);
    float *v = reinterpret_cast<float *>(a.area + r.v_off);
    float *ss = reinterpret_cast<float *>(a.area + r.ss_off);
    float *uo = l + 1 == a.l1 ? a.y : reinterpret_cast<float *>(a.area + r.u_off);
    GemvArgs gi = r.gi;
    gi.act = u;
    gi.zx = zx;
    gi.slots = a.slots;
    gi.n_slots = a.n_slots;
    inproj_phase(gi, w, lds, tid, lane, wave);
    // the SSD item's state tile (no phase of this launch writes it before) while waiting
    SsdArgs sa = r.sa;
    sa.zx = zx;
    sa.vw = v;
    sa.ss = ss;
    sa.slots = a.slots;
    sa.n_slots = a.n_slots;
    const FItem it = fused_item(sa, r.items);
    SsdTile<kFMaxI> tile;
    fused_tile_load(sa, it, wave, lane, tile);
    grid_barrier(bar, &ctl, ++gen, wave, lane, NoOp());
    GemvArgs go = r.go;
    go.act = v;
    go.ss = ss;
    go.y = uo;
    go.resid = u;
    go.zx = zx;
    go.slots = a.slots;
    go.n_slots = a.n_slots;
    ssd_out_phase<true>(go, sa, bar, it, tile, &ctl, ++gen, lds, tid, lane, wave);
    if (l + 1 < a.l1) {
      inproj_first(a.tab[l + 1].gi, wave, lane, w);   // the next layer's first row, while waiting
      grid_barrier(bar, &ctl, ++gen, wave, lane, NoOp());
    }
    u = uo;
  }
  // A barrier wait that ran out (the grid was not all resident) left the results undefined;
  // every workgroup then sees the error word (it was raised before any workgroup passed that
  // barrier) and writes NaN over its rows of the output, so the failure cannot pass unseen.
  if (__hip_atomic_load(bar + kBarError * kBarStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
    const int rows = a.tab[a.l1 - 1].go.rows;
    const int r0 = (int)(((long)blockIdx.x * rows) / gridDim.x);
    const int r1 = (int)(((long)(blockIdx.x + 1) * rows) / gridDim.x);
    if (r0 + tid < r1) stc<true>(a.y + r0 + tid, __builtin_nanf(""));
  }
}

__global__ void bar_zero_kernel(unsigned *bar) {
  if ((int)threadIdx.x < kBarWords) bar[threadIdx.x * kBarStride] = 0u;
}

size_t fused_lds_bytes(const m2_layer_s &L) {
  const size_t b = 16 + 2 * (size_t)L.cfg.d_state + L.prange;         // wsum | conv outputs
  const size_t c = (size_t)L.d_inner + kFWaves * kFRMax;              // scaled activations | row sums
  return sizeof(float) * std::max(b, c);
}

}  // namespace

// The grid of the persistent kernel on the current device: two workgroups per CU, if the
// kernel's occupancy allows two (0: it cannot run here). Cached per device and LDS size.
int fused_grid(const m2_layer_s &L) {
  static int cus[64] = {0}, occ[64][2] = {{0}};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cus[dev] = n;
  }
  const size_t lds = fused_lds_bytes(L);
  if (occ[dev][1] != (int)lds) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fused_ssd_out_kernel, kFThreads, lds) != hipSuccess)
      return 0;
    occ[dev][0] = nb;
    occ[dev][1] = (int)lds;
  }
  return occ[dev][0] >= 2 ? 2 * cus[dev] : 0;
}

// Whether the layer's shapes fit plan 2 at this grid size (one session, bf16).
bool fused_fits(const m2_layer_s &L, int grid) {
  const m2_config &c = L.cfg;
  if (c.wtype != M2_W_BF16 || grid <= 0) return false;
  if (c.d_model % 8 || L.d_inner % 8 || c.d_model > 24576) return false;   // in_proj x in LDS
  const long nco = L.d_inner / 8, per_w = (nco + kFWaves - 1) / kFWaves;
  if (per_w > 64 * kFJC) return false;                                // out_proj eighth of a row
  if ((c.d_model + grid - 1) / grid > kFRMax) return false;           // out_proj rows per workgroup
  if ((long)c.d_model * nco * 16 >= kBufOutOfRange) return false;     // W_out within one buffer resource
  if (c.n_heads * L.psplit > grid) return false;                      // one SSD item per workgroup
  const int rpi = 64 / (c.d_state / 4);
  if ((L.prange + rpi - 1) / rpi > kFWaves * kFMaxI) return false;    // slices per wave
  for (int w = 0; w < kFWaves; ++w) {                                 // RMS groups per eighth
    const long s0 = std::min(w * per_w, nco), s1 = std::min(s0 + per_w, nco);
    if (s1 > s0 && (8 * s1 - 1) / L.ng - (8 * s0) / L.ng + 1 > kFGroups) return false;
  }
  return true;
}

hipError_t launch_fused_step(const m2_layer_s &L, const m2_state_s &S, const float *x, float *y,
                             const int32_t *slots, int flags, const StepWs &ws, int grid, hipStream_t stream) {
  const m2_config &c = L.cfg;
  FusedArgs f{};
  SsdArgs &sa = f.sa;
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
  GemvArgs &go = f.go;
  go.W = L.w.w_out;
  go.rows = c.d_model;
  go.K = L.d_inner;
  go.gamma = 1.0f;
  go.act = ws.v;
  go.B = 1;
  go.ss = ws.ss;
  go.ng = L.ng;
  go.n_partials = L.n_partials;
  go.n_norm = L.n_norm;
  go.eps = c.norm_eps;
  go.y = y;
  go.resid = (flags & M2_RESIDUAL) ? x : nullptr;
  go.slots = slots;
  go.n_slots = S.n_slots;
  go.zx = ws.zx;
  go.zx_stride = L.zx_stride;
  go.d_inner = L.d_inner;
  go.conv_dim = L.conv_dim;
  go.d_conv = c.d_conv;
  go.conv_cache = S.conv;
  f.bar = ws.bar;
  f.items = c.n_heads * L.psplit;
  hipLaunchKernelGGL(fused_ssd_out_kernel, dim3(grid), dim3(kFThreads), fused_lds_bytes(L), stream, f);
  return hipGetLastError();
}


// ---- the persistent stack step (host side)
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t stack_area_head() { return al256(kBarBytes); }

size_t stack_area_layer_bytes(const m2_layer_s &L) {
  return al256(sizeof(float) * (size_t)L.zx_stride) + al256(sizeof(float) * (size_t)L.d_inner) +
         al256(sizeof(float) * (size_t)L.n_partials) + al256(sizeof(float) * (size_t)L.cfg.d_model);
}

size_t stack_rec_bytes() { return sizeof(StackRec); }

void stack_rec_fill(const m2_layer_s &L, const m2_state_s &S, size_t off, void *out) {
  const m2_config &c = L.cfg;
  StackRec r{};
  GemvArgs &gi = r.gi;
  gi.W = L.w.w_in;
  gi.rows = L.d_in_proj;
  gi.K = c.d_model;
  gi.gamma = 1.0f;
  gi.B = 1;
  gi.zx_stride = L.zx_stride;
  gi.d_inner = L.d_inner;
  gi.conv_dim = L.conv_dim;
  gi.d_conv = c.d_conv;
  gi.dt_bias = L.w.dt_bias;
  SsdArgs &sa = r.sa;
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
  sa.prange = L.prange;
  sa.psplit = L.psplit;
  sa.n_partials = L.n_partials;
  GemvArgs &go = r.go;
  go.W = L.w.w_out;
  go.rows = c.d_model;
  go.K = L.d_inner;
  go.gamma = 1.0f;
  go.B = 1;
  go.ng = L.ng;
  go.n_partials = L.n_partials;
  go.n_norm = L.n_norm;
  go.eps = c.norm_eps;
  go.zx_stride = L.zx_stride;
  go.d_inner = L.d_inner;
  go.conv_dim = L.conv_dim;
  go.d_conv = c.d_conv;
  go.conv_cache = S.conv;
  r.items = c.n_heads * L.psplit;
  r.zx_off = (long long)off;
  r.v_off = r.zx_off + (long long)al256(sizeof(float) * (size_t)L.zx_stride);
  r.ss_off = r.v_off + (long long)al256(sizeof(float) * (size_t)L.d_inner);
  r.u_off = r.ss_off + (long long)al256(sizeof(float) * (size_t)L.n_partials);
  std::memcpy(out, &r, sizeof r);
}

size_t stack_lds_bytes(const m2_layer_s &L) {
  return std::max(fused_lds_bytes(L), sizeof(float) * (size_t)L.cfg.d_model);
}

// Two workgroups per CU if the kernel's occupancy at this LDS size allows two (else 0).
int stack_grid(size_t lds) {
  static int cus[64] = {0}, occ[64][2] = {{0}};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cus[dev] = n;
  }
  if (occ[dev][1] != (int)lds) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, stack_persistent_kernel, kFThreads, lds) != hipSuccess)
      return 0;
    occ[dev][0] = nb;
    occ[dev][1] = (int)lds;
  }
  return occ[dev][0] >= 2 ? 2 * cus[dev] : 0;
}

bool stack_fits(const m2_layer_s &L, int grid) {
  return fused_fits(L, grid) && L.cfg.d_model <= 8 * 64 * kIJ &&                // in_proj: one row per trip
         (long)L.d_in_proj * (L.cfg.d_model / 8) * 16 < kBufOutOfRange;       // W_in within one resource
}

hipError_t launch_stack_run(const void *tab, int l0, int l1, size_t lds, void *area, float *y,
                            const int32_t *slots, int n_slots, int grid, hipStream_t stream) {
  StackArgs a{};
  a.tab = static_cast<const StackRec *>(tab);
  a.l0 = l0;
  a.l1 = l1;
  a.area = static_cast<char *>(area);
  a.y = y;
  a.slots = slots;
  a.n_slots = n_slots;
  hipLaunchKernelGGL(bar_zero_kernel, dim3(1), dim3(64), 0, stream, reinterpret_cast<unsigned *>(area));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stack_persistent_kernel, dim3(grid), dim3(kFThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace m2d
