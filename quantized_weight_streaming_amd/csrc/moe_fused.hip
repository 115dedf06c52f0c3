// Fused MoE layer(s) on gfx950: router GEMV, top-K, softmax, expert union, MXFP4 gate_up + SwiGLU,
// MXFP4 down + gate-weighted combine with the shared expert -- one persistent launch for one or
// more layers (each layer routes eight of E routed experts plus one shared expert:
// runbyai.xyz/posts/593 paragraph 2; a window of M <= 4 tokens reads each activated expert once:
// paragraph 5).
//
// Why one launch: a kernel boundary costs ~1.7 us on MI355X even inside a HIP graph, about a third
// of a layer's streaming time at M = 1. The grid is one 512-thread workgroup per compute unit, all
// resident at once.
//
// Work decomposition. A "task" is (slot u, block j): the 32 gate rows and 32 up rows of activation
// block j of expert id(u), plus the 32-column block j of that expert's down projection for all H
// output rows. One workgroup issues all of a task's loads in one burst (2 x 32 x H/2 gate/up bytes
// + H x 16 down bytes: 120 KB of codes at H = 2560), computes the block's 32 activations itself --
// activations never cross workgroups -- and writes H partial sums per token, already multiplied by
// the token's gate weight. The down projection is stored block-major (moe_pack_mxfp4) so that
// block j of an expert is one contiguous stream. Weights are read with non-temporal loads: each
// byte is used once per step, and on MI355X a burst of such loads streams ~2x faster than cached
// loads when the caches hold dirty lines.
//
// Hand-offs between workgroups carry their own validity: a 64-bit word holds a 32-bit value and a
// 32-bit tag unique to (launch, layer, kind), written with one device-coherent store and polled
// with device-coherent loads (64-bit accesses are single-copy atomic), so a reader needs no
// separate signal, fence or counter; a poll reloads only the words that are not yet valid. Per
// layer:
//   1  x into LDS: layer 0 from the caller's buffer; in a chained sequence (x of layer l+1 is y of
//      layer l) from the tagged copy of y the previous layer published.
//   2  router dots of this workgroup's rows (prefetched into LDS during the previous layer) ->
//      tagged logits; workgroups G-J .. G-1 then run the shared expert's J tasks (they need no
//      routing).
//   3  every workgroup selects top-K itself from the tagged logits, in parallel: a threshold from
//      the per-wave maxima leaves a few candidates, each of which counts the candidates that beat
//      it (logit descending, index ascending) to find its rank; softmax over the selected; union of
//      the window's selections (first-occurrence order).
//   4  routed tasks, round-robin over workgroups (at M = 1 one task per workgroup).
//   5  workgroup b owns output rows [b*R, b*R + R): it polls their tagged partial sums, sums them in
//      a fixed order (deterministic), writes y and, in a chained sequence, a tagged copy.
// Layers that are not chained are separated by a counter barrier instead.
#include "qws_common.hpp"

namespace {

using namespace qws;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxM = 4;
constexpr int kMaxK = 8;
constexpr int kMaxSlots = kMaxM * kMaxK + 1;    // routed union + shared
constexpr int kMaxPairs = kMaxM * (kMaxK + 1);  // (slot, token) pairs
constexpr int kMaxE = 1024;
constexpr int kEpt = kMaxE / kThreads;          // experts per thread in the selection
constexpr int kHMax = 2560;
constexpr int kIMax = 1024;
constexpr int kBlk = 32;        // activations per task: one MX block of the down projection
constexpr int kGuCpl = 5;       // 16-byte chunks per lane of a gate/up row: H <= 16 * 5 * 32
constexpr int kRtCpl = 5;       // 16-byte chunks per lane of a router row: H <= 64 * 5 * 8
constexpr int kDnRpl = 5;       // down rows per thread in a task: H <= 512 * 5
constexpr int kMaxRows = 16;    // output rows owned by one workgroup
constexpr int kMaxGrid = 512;
constexpr int kRowsPad = 2 * kMaxGrid;   // partial buffer rows allowed beyond H (G * R >= H)
constexpr int kPollBatch = 12;  // tagged words per thread in flight while reading partials
constexpr int kSumLanes = 8;    // lanes that share the sum of one (token, row) in the combine
constexpr int kSyncCounters = 16;
constexpr int kSyncStride = 16;             // 64-bit words: 128 bytes apart
constexpr unsigned kSpinLimit = 1u << 20;   // polls before a wait gives up (~1 s)
constexpr int kTracePoints = 16;            // timestamps per (layer, workgroup) when tracing
constexpr int kTagsPerLaunch = 4096;        // tag space of one launch: 4 per layer
constexpr int kMaxLayers = kTagsPerLaunch / 4;
constexpr int kDescWords = sizeof(qws_moe_layer) / 8;
static_assert(sizeof(qws_moe_layer) % 8 == 0 && kDescWords <= kWave, "descriptor copy");

struct Layer {
  const uint16_t* x;
  const uint16_t* wr;
  const float* bias;
  long long bias_stride;
  const uint8_t* gq;
  const uint8_t* gs;
  const uint8_t* dq;   // block-major [n][I/32][H][16]
  const uint8_t* ds;   // block-major [n][I/32][H]
  int* topk_idx;
  float* topk_w;
  float* logits_out;
  uint16_t* y16;
  float* y32;
};

__host__ __device__ Layer to_layer(const qws_moe_layer& d) {
  return Layer{static_cast<const uint16_t*>(d.x_bf16), static_cast<const uint16_t*>(d.w_router_bf16), d.bias,
               d.bias_row_stride, d.experts.gate_up_q, d.experts.gate_up_s, d.experts.down_q, d.experts.down_s,
               d.topk_idx, d.topk_w, d.logits_out, static_cast<uint16_t*>(d.y_bf16), d.y_f32};
}

struct Shape {
  int E, K, H, I, has_shared;
  int R;        // output rows per workgroup (even)
  int P;        // (slot, token) pairs the partial buffer holds per block: M * (K + 1)
  int chained;  // x of layer l+1 is y (bf16) of layer l, for every l
  int rows_total;  // G * R: rows of the partial buffer, H and padding
  int nrw;      // router rows per workgroup (one wave each)
};

struct Work {
  unsigned long long* trace;     // NULL, or [n_layers][G][kTracePoints] wall-clock stamps (100 MHz)
  unsigned long long* sync;      // kSyncCounters monotonic counters, kSyncStride apart
  unsigned long long* launches;  // launch counter (each workgroup adds 1 per launch)
  unsigned* errors;              // count of bounded waits that timed out (sticky)
  unsigned long long* logits;    // [M][E] tagged logits
  unsigned long long* ytag;      // [M][H/2] tagged bf16 pairs of y (chained sequences)
  unsigned long long* done;      // [G] tagged "layer finished" words (layers that are not chained)
  unsigned long long* partial;   // [G][P][J][R] tagged, gate-weighted partial sums of the down projection
};

// Routing of the current layer, shared by the workgroup (LDS).
struct Union {
  int n;                         // slots: 0 = shared (if any), then routed ids in first-occurrence order
  int id[kMaxSlots];
  unsigned mask[kMaxSlots];      // tokens using the slot
  int pair0[kMaxSlots];          // first (slot, token) pair index of the slot
  float w[kMaxSlots][kMaxM];     // gate weight of (slot, token)
  int n_pairs;
  int tok_n[kMaxM];              // pairs of each token, in slot order
  int tok_pair[kMaxM][kMaxSlots];
};

__device__ __forceinline__ void stamp(const Work& w, int l, int k) {
  if (w.trace && threadIdx.x == 0)
    w.trace[((size_t)l * gridDim.x + blockIdx.x) * kTracePoints + k] = wall_clock64();
}

__device__ __forceinline__ unsigned long long tagged(uint32_t tag, uint32_t v) {
  return ((unsigned long long)tag << 32) | (unsigned long long)v;
}
__device__ __forceinline__ uint32_t tag_of(unsigned long long v) { return (uint32_t)(v >> 32); }

__device__ __forceinline__ bool gave_up(const Work& w) { return ld_coherent(w.errors) != 0u; }

// Poll count, error check and back-off of a bounded wait; returns true when the wait must end.
// Once any wait has timed out (the error count is sticky) every other wait ends at its next check.
__device__ __forceinline__ bool wait_expired(const Work& w, unsigned& spins) {
  if ((++spins & 255u) == 0) {
    const bool other = gave_up(w);
    if (other || spins > kSpinLimit) {
      if (!other && (threadIdx.x % kWave) == 0) atomicAdd(w.errors, 1u);
      return true;
    }
  }
  __builtin_amdgcn_s_sleep(1);
  return false;
}

// Reloads the words Q .. N-1 of a poll that do not carry `tag` yet (compile-time recursion rather
// than a loop: a loop inside the wait loop was not unrolled, which put v in scratch memory).
template <int Q, int N>
__device__ __forceinline__ void reload_missing(const unsigned long long* src, const int (&idx)[N], uint32_t tag,
                                               unsigned long long (&v)[N]) {
  if constexpr (Q < N) {
    if (tag_of(v[Q]) != tag) v[Q] = ld_coherent(src + idx[Q]);
    reload_missing<Q + 1, N>(src, idx, tag, v);
  }
}
template <int Q, int N>
__device__ __forceinline__ bool all_tagged(const unsigned long long (&v)[N], uint32_t tag) {
  if constexpr (Q < N) return tag_of(v[Q]) == tag && all_tagged<Q + 1, N>(v, tag);
  else return true;
}

// Loads src[idx[q]] for q < N (idx < 0: no load, the word counts as valid) and waits until each
// carries `tag`, reloading only the words that do not yet. Every lane of the wave must call it
// (the wait is wave-wide).
template <int N>
__device__ __forceinline__ void poll_tagged(const Work& w, const unsigned long long* src, const int (&idx)[N],
                                            uint32_t tag, unsigned long long (&v)[N]) {
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = idx[q] >= 0 ? ld_coherent(src + idx[q]) : tagged(tag, 0u);
  unsigned spins = 0;
  while (!__all(all_tagged<0, N>(v, tag))) {
    if (wait_expired(w, spins)) break;
    reload_missing<0, N>(src, idx, tag, v);
  }
}

// ------------------------------------------------------------------------------ grid barrier
// Between layers that are not chained. Every workgroup arrives once on counter blockIdx % 16; the
// counters only ever increase. The first barrier of a launch learns its epoch from the value its
// atomic saw; later ones count epochs in registers. Completion is every counter c reaching
// (epoch + 1) * arrivals(c). Returning atomics: measured on MI355X, their increment is visible to
// pollers within ~1 us, a posted (non-returning) one took ~3 us.
struct SyncState {
  unsigned long long epoch;  // valid in wave 0 once `known`
  bool known;
};

__device__ void grid_sync(const Work& w, SyncState& st) {
  wait_mem();
  __syncthreads();
  const unsigned G = gridDim.x;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const unsigned ncnt = G < (unsigned)kSyncCounters ? G : (unsigned)kSyncCounters;
    const unsigned c = blockIdx.x % ncnt;
    unsigned long long prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(w.sync + c * kSyncStride, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, kWave);
    if (!st.known) {
      st.epoch = prev / ((G - c + ncnt - 1) / ncnt);
      st.known = true;
    }
    bool done = lane >= (int)ncnt;
    const unsigned long long target = done ? 0ull : (st.epoch + 1) * (unsigned long long)((G - lane + ncnt - 1) / ncnt);
    unsigned spins = 0;
    while (true) {
      if (!done) done = ld_coherent(w.sync + lane * kSyncStride) >= target;
      if (__all(done)) break;
      if (wait_expired(w, spins)) break;
    }
    st.epoch += 1;
  }
  __syncthreads();
}

// Between layers that are not chained: every workgroup publishes a tagged word once all of its
// stores have been acknowledged, then waits for every workgroup's word. No atomics, so no
// round trip to a counter before the wait starts.
__device__ void tagged_barrier(const Work& w, uint32_t tag, int tid, int l) {
  wait_mem();
  __syncthreads();
  stamp(w, l, 14);
  if (tid == 0) st_coherent(w.done + blockIdx.x, tagged(tag, 0u));
  if (tid < kWave) {
    constexpr int kPer = kMaxGrid / kWave;
    int idx[kPer];
    unsigned long long v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) idx[q] = tid + q * kWave < (int)gridDim.x ? tid + q * kWave : -1;
    poll_tagged<kPer>(w, w.done, idx, tag, v);
  }
  __syncthreads();
}

// Selection key: order-preserving float -> uint32 (larger float, larger key; -0 == +0; NaN ranks
// as -inf). Every logit maps to >= 0x007fffff; 0 marks an absent entry.
__device__ __forceinline__ uint32_t sel_key(float f) {
  if (f != f) f = -__builtin_inff();
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Total order of the selection: larger key first, then lower expert index.
__device__ __forceinline__ unsigned long long rank_key(uint32_t key, int e) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - (uint32_t)e);
}

// Non-temporal 16-byte load of weights that are read once per step.
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const QWS_GLOBAL u32x4_t*)p);
}
__device__ __forceinline__ uint32_t ldb_stream(const uint8_t* p) {
  return __builtin_nontemporal_load((const QWS_GLOBAL uint8_t*)p);
}

// ------------------------------------------------------------------------------ tasks
struct TaskRegs {
  u32x4_t g[kGuCpl], u[kGuCpl], d[kDnRpl];
  uint32_t gs[kGuCpl], us[kGuCpl], ds[kDnRpl];
};

// Issues the loads of task (expert e, block j). 16-lane group g of the workgroup takes gate row
// 32j+g and up row I+32j+g (lane j16: chunks j16, j16+16, ...); thread t takes down rows t, t+512, ...
__device__ __forceinline__ void task_load(const Layer& L, const Shape& sh, int e, int j, unsigned tid, TaskRegs& r) {
  const unsigned g = tid >> 4, j16 = tid & 15;
  const int H = sh.H, I = sh.I, J = I / kBlk;
  const unsigned nch = (unsigned)(H >> 5), rb = (unsigned)(H >> 1);
  const size_t row_g = (size_t)e * 2 * I + (size_t)kBlk * j;   // first gate row of the block
  const uint8_t* gq = L.gq + row_g * rb;
  const uint8_t* uq = gq + (size_t)I * rb;
  const uint8_t* gs = L.gs + row_g * nch;
  const uint8_t* us = gs + (size_t)I * nch;
  // unconditional loads from clamped (in-bounds) addresses: no branch around a load, so a task's
  // loads issue back to back. A chunk past the row end is loaded from the last chunk and skipped
  // by the compute; a down row past H is loaded from row H-1 and its partial sum is not stored.
#pragma unroll
  for (int t = 0; t < kGuCpl; ++t) {
    const unsigned c = min(j16 + 16u * t, nch - 1);
    r.g[t] = ld16_stream(gq + g * rb + c * 16u);
    r.u[t] = ld16_stream(uq + g * rb + c * 16u);
    r.gs[t] = ldb_stream(gs + g * nch + c);
    r.us[t] = ldb_stream(us + g * nch + c);
  }
  const size_t blk = ((size_t)e * J + j) * (size_t)H;
  const uint8_t* dq = L.dq + blk * 16;
  const uint8_t* ds = L.ds + blk;
#pragma unroll
  for (int t = 0; t < kDnRpl; ++t) {
    const unsigned row = min(tid + (unsigned)(kThreads * t), (unsigned)H - 1);
    r.d[t] = ld16_stream(dq + row * 16u);
    r.ds[t] = ldb_stream(ds + row);
  }
}

// Computes task (slot u: tokens in un.mask[u], pairs un.pair0[u] + rank, gate weights un.w[u][m],
// block j) from its loaded registers: the block's activations silu(gate) * up into LDS, then
// partial[p][j][row] = w * sum_k W_down[row][32j+k] * a[k] for every row, stored tagged at this
// thread's row offsets in the owners' regions.
template <int M>
__device__ __forceinline__ void task_compute(const Shape& sh, const Work& w, const TaskRegs& r, const Union& un,
                                             int u, int j, const uint16_t* xs, float* a_s, unsigned tid,
                                             uint32_t tag) {
  const int g = tid >> 4, j16 = tid & 15;
  const int H = sh.H, nch = H >> 5, J = sh.I / kBlk, R = sh.R;
  const unsigned mask = un.mask[u];
  const int p0 = un.pair0[u];
  float ag[M], au[M];
#pragma unroll
  for (int m = 0; m < M; ++m) ag[m] = au[m] = 0.0f;
#pragma unroll
  for (int t = 0; t < kGuCpl; ++t) {
    const int c = j16 + 16 * t;
    if (c < nch) {
      const float scg = e8m0_to_f32(r.gs[t]), scu = e8m0_to_f32(r.us[t]);
      bf16x2_t pg[16], pu[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        pg[4 * d + 0] = fp4x2_to_bf16x2<0>(r.g[t][d], scg);
        pg[4 * d + 1] = fp4x2_to_bf16x2<1>(r.g[t][d], scg);
        pg[4 * d + 2] = fp4x2_to_bf16x2<2>(r.g[t][d], scg);
        pg[4 * d + 3] = fp4x2_to_bf16x2<3>(r.g[t][d], scg);
        pu[4 * d + 0] = fp4x2_to_bf16x2<0>(r.u[t][d], scu);
        pu[4 * d + 1] = fp4x2_to_bf16x2<1>(r.u[t][d], scu);
        pu[4 * d + 2] = fp4x2_to_bf16x2<2>(r.u[t][d], scu);
        pu[4 * d + 3] = fp4x2_to_bf16x2<3>(r.u[t][d], scu);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if ((mask >> m) & 1u) {
          const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xs + m * H + c * 32);
          float a = ag[m], b = au[m];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4_t xv = xp[q];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              a = dot2(pg[4 * q + k], as_bf16x2(xv[k]), a);
              b = dot2(pu[4 * q + k], as_bf16x2(xv[k]), b);
            }
          }
          ag[m] = a;
          au[m] = b;
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float hg = row16_sum(ag[m]);
    const float hu = row16_sum(au[m]);
    if (j16 == 0) a_s[m * kBlk + g] = silu(hg) * hu;
  }
  __syncthreads();
  float wt[M];
  int pm[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    wt[m] = un.w[u][m];
    pm[m] = p0 + __popc(mask & ((1u << m) - 1u));
  }
#pragma unroll
  for (int t = 0; t < kDnRpl; ++t) {
    const int row = tid + kThreads * t;
    // this row's word in its owner's region [owner][P][J][R]
    const int rc = min(row, sh.rows_total - 1), owner = rc / R;
    const unsigned rowoff = (unsigned)(owner * sh.P * J * R + (rc - owner * R));
    const float sc = e8m0_to_f32(r.ds[t]);
    float wf[kBlk];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const f32x2_t v0 = fp4x2_to_f32x2<0>(r.d[t][d], sc), v1 = fp4x2_to_f32x2<1>(r.d[t][d], sc);
      const f32x2_t v2 = fp4x2_to_f32x2<2>(r.d[t][d], sc), v3 = fp4x2_to_f32x2<3>(r.d[t][d], sc);
      wf[8 * d + 0] = v0.x; wf[8 * d + 1] = v0.y; wf[8 * d + 2] = v1.x; wf[8 * d + 3] = v1.y;
      wf[8 * d + 4] = v2.x; wf[8 * d + 5] = v2.y; wf[8 * d + 6] = v3.x; wf[8 * d + 7] = v3.y;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if ((mask >> m) & 1u) {
        const float4* ap = reinterpret_cast<const float4*>(a_s + m * kBlk);
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < kBlk / 4; ++q) {
          const float4 a4 = ap[q];
          s = fmaf(wf[4 * q + 0], a4.x, s);
          s = fmaf(wf[4 * q + 1], a4.y, s);
          s = fmaf(wf[4 * q + 2], a4.z, s);
          s = fmaf(wf[4 * q + 3], a4.w, s);
        }
        // rows H .. G*R-1 (zero weights) pad the last owner's region so that it is written whole
        s = row < H ? wt[m] * s : 0.0f;
        if (row < sh.rows_total)
          st_coherent(w.partial + (size_t)(pm[m] * J + j) * R + rowoff, tagged(tag, __float_as_uint(s)));
      }
    }
  }
  __syncthreads();  // a_s is rewritten by the next task
}

// ------------------------------------------------------------------------------ top-K + union
// Every workgroup selects the top-K of each token from the tagged logits (same result in every
// workgroup). Thread t holds experts t + 512 i. A candidate must reach T = the smallest of the
// per-wave maxima when at least K waves hold experts (then >= K logits reach T, so every one of
// the top K does); otherwise T admits every expert. Each candidate's rank is the number of
// candidates that beat it; ranks < K are the selection, in order.
template <int M>
__device__ __forceinline__ void select_topk(const Shape& sh, const Work& w, uint32_t tag, int tid, int wave, int lane,
                                            unsigned long long* cand, Union& un, int (*s_idx)[kMaxK],
                                            float (*s_w)[kMaxK], uint32_t (*s_wmax)[kWaves],
                                            int (*s_cnt)[kEpt][kWaves], uint32_t (*s_sel)[kMaxK], int l) {
  const int E = sh.E, K = sh.K;
  uint32_t key[M][kEpt];
  {
    int idx[M * kEpt];
    unsigned long long v[M * kEpt];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < kEpt; ++i) {
        const int e = tid + kThreads * i;
        idx[m * kEpt + i] = e < E ? m * E + e : -1;
      }
    poll_tagged<M * kEpt>(w, w.logits, idx, tag, v);
    stamp(w, l, 4);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < kEpt; ++i)
        key[m][i] = idx[m * kEpt + i] >= 0 ? sel_key(__uint_as_float((uint32_t)v[m * kEpt + i])) : 0u;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint32_t k = key[m][0];
#pragma unroll
    for (int i = 1; i < kEpt; ++i) k = max(k, key[m][i]);
    const uint32_t wm = wave_max_u32(k);
    if (lane == 0) s_wmax[m][wave] = wm;
  }
  __syncthreads();
  stamp(w, l, 10);
  // waves holding at least one expert: wave v holds experts v*64 .. v*64+63 (+ 512 i)
  const int nvw = min(kWaves, (E + kWave - 1) / kWave);
  bool cf[M][kEpt];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint32_t T = 0u;
    if (nvw >= K) {
      T = 0xffffffffu;
      for (int v = 0; v < nvw; ++v) T = min(T, s_wmax[m][v]);
    }
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      cf[m][i] = key[m][i] != 0u && key[m][i] >= T;
      const unsigned long long b = __ballot(cf[m][i]);
      if (lane == 0) s_cnt[m][i][wave] = __popcll(b);
    }
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  int ncand[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    // candidate order in the buffer: (i, wave, lane); any order would do, ranks are counted
    int pos[kEpt], total = 0;
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      pos[i] = total;
      for (int v = 0; v < kWaves; ++v) {
        const int c = s_cnt[m][i][v];
        pos[i] += v < wave ? c : 0;
        total += c;
      }
    }
    ncand[m] = total;
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      const unsigned long long bl = __ballot(cf[m][i]);
      if (cf[m][i]) cand[m * E + pos[i] + __popcll(bl & lt)] = rank_key(key[m][i], tid + kThreads * i);
    }
  }
  __syncthreads();
  stamp(w, l, 11);
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      if (cf[m][i]) {
        const unsigned long long mine = rank_key(key[m][i], tid + kThreads * i);
        const unsigned long long* cm = cand + m * E;
        int rank = 0;
        for (int q = 0; q < ncand[m] && rank < K; ++q) rank += cm[q] > mine ? 1 : 0;
        if (rank < K) {
          s_idx[m][rank] = tid + kThreads * i;
          s_sel[m][rank] = key[m][i];
        }
      }
    }
  }
  __syncthreads();
  stamp(w, l, 12);
  if (wave == 0) {
    // softmax over the selected logits of each token: lane l is selection (l / K, l % K); every
    // lane of a token sums the same terms in the same order
    const int n = M * K;
    const int mj = lane < n ? lane / K : 0, rj = lane - mj * K;
    const float z = lane < n ? expf(key_to_float(s_sel[mj][rj]) - key_to_float(s_sel[mj][0])) : 0.0f;
    float s = 0.0f;   // sum of the token's K terms in rank order, the same in each of its lanes
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float sm = 0.0f;
      for (int r = 0; r < K; ++r) sm += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), m * K + r));
      s = m == mj ? sm : s;
    }
    float wj = 0.0f;
    int e = -1;
    if (lane < n) {
      wj = z / s;
      e = s_idx[mj][rj];
      s_w[mj][rj] = wj;
    }
    // union in first-occurrence order over (token, rank); slot 0 is the shared expert (if any)
    const int ns = sh.has_shared ? 1 : 0;
    bool first = lane < n;
    unsigned mask = 0;
    float wsum[M];
#pragma unroll
    for (int m = 0; m < M; ++m) wsum[m] = 0.0f;
    for (int i = 0; i < n; ++i) {
      const int ei = __builtin_amdgcn_readlane(e, i);
      const int mi = i / K;
      const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), i));
      if (ei == e) {
        if (i < lane) first = false;
        mask |= 1u << mi;
#pragma unroll
        for (int m = 0; m < M; ++m)
          if (m == mi) wsum[m] += wi;
      }
    }
    const unsigned long long firsts = __ballot(first);
    const int cnt = first ? __popc(mask) : 0;
    int pair0 = ns * M;
    for (int i = 0; i < n; ++i) {
      const int ci = __builtin_amdgcn_readlane(cnt, i);
      pair0 += i < lane ? ci : 0;
    }
    const int slot = ns + __popcll(firsts & lt);
    if (first) {
      un.id[slot] = e;
      un.mask[slot] = mask;
      un.pair0[slot] = pair0;
#pragma unroll
      for (int m = 0; m < M; ++m) un.w[slot][m] = wsum[m];
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const unsigned long long bm = __ballot(first && ((mask >> m) & 1u));
      if (first && ((mask >> m) & 1u)) un.tok_pair[m][ns + __popcll(bm & lt)] = pair0 + __popc(mask & ((1u << m) - 1u));
      if (lane == 0) {
        un.tok_n[m] = ns + __popcll(bm);
        if (ns) un.tok_pair[m][0] = m;
      }
    }
    if (lane == 0) {
      if (ns) {
        un.id[0] = E;
        un.mask[0] = (1u << M) - 1u;
        un.pair0[0] = 0;
#pragma unroll
        for (int m = 0; m < M; ++m) un.w[0][m] = 1.0f;
      }
      int total = ns * M;
      for (int i = 0; i < n; ++i) total += __builtin_amdgcn_readlane(cnt, i);
      un.n = __popcll(firsts) + ns;
      un.n_pairs = total;
    }
  }
}

// ------------------------------------------------------------------------------ the kernel
__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
// A layer descriptor copied into LDS (raw words of a qws_moe_layer), read as wave-uniform values.
__device__ __forceinline__ Layer desc_from_lds(const unsigned long long* raw) {
  unsigned long long v[kDescWords];
#pragma unroll
  for (int i = 0; i < kDescWords; ++i) v[i] = uniform_u64(raw[i]);
  qws_moe_layer d;
  __builtin_memcpy(&d, v, sizeof(d));
  return to_layer(d);
}

template <int M>
__global__ __launch_bounds__(kThreads) void moe_layers_kernel(Layer first, const qws_moe_layer* __restrict__ rest,
                                                              int n_layers, Shape sh, Work w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ Union un;
  __shared__ int s_idx[kMaxM][kMaxK];
  __shared__ float s_w[kMaxM][kMaxK];
  __shared__ uint32_t s_sel[kMaxM][kMaxK];
  __shared__ uint32_t s_wmax[kMaxM][kWaves];
  __shared__ int s_cnt[kMaxM][kEpt][kWaves];
  __shared__ __attribute__((aligned(16))) float a_s[kMaxM * kBlk];
  __shared__ float s_y[kMaxM][kMaxRows];
  __shared__ __attribute__((aligned(16))) unsigned long long s_desc[2][kDescWords];
  __shared__ unsigned long long s_launch;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int G = gridDim.x, b = blockIdx.x;
  const int E = sh.E, H = sh.H, I = sh.I, R = sh.R;
  const int J = I / kBlk;
  const int ns = sh.has_shared ? 1 : 0;

  // dynamic LDS: x [M][H] bf16 | router rows [nrw][H] bf16 | scratch: selection candidates
  // [M][E] u64, later this workgroup's partial sums [pairs][J][R] fp32
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  uint16_t* wr_s = reinterpret_cast<uint16_t*>(lds + (size_t)M * H * 2);
  unsigned char* scratch = lds + (size_t)M * H * 2 + (size_t)sh.nrw * H * 2;
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(scratch);
  float* red = reinterpret_cast<float*>(scratch);

  const int row0 = b * R;
  const int my_rows = max(0, min(R, H - row0));
  const bool shared_task = sh.has_shared && b >= G - J;
  const int r_row = b + G * wave;                       // this wave's router row
  const bool is_router = wave < sh.nrw && r_row < E;
  SyncState sync{0ull, false};

  // launch number -> this launch's tag base (every workgroup adds 1 per launch)
  if (tid == 0)
    s_launch = __hip_atomic_fetch_add(w.launches, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) / (unsigned)G;
  __syncthreads();
  const uint32_t tag_base = (uint32_t)(s_launch * kTagsPerLaunch);
  if (s_launch > 0 && tag_base == 0) {
    // tags repeat from here on: clear every tagged word (tag 0 is never valid) before any use
    const size_t own = (size_t)sh.P * J * R;
    for (size_t i = tid; i < own; i += kThreads) st_coherent(w.partial + (size_t)b * own + i, 0ull);
    for (int i = b * kThreads + tid; i < M * E; i += G * kThreads) st_coherent(w.logits + i, 0ull);
    for (int i = b * kThreads + tid; i < M * H / 2; i += G * kThreads) st_coherent(w.ytag + i, 0ull);
    if (tid == 0) st_coherent(w.done + b, 0ull);
    grid_sync(w, sync);
  }

  // router rows of layer 0 -> LDS (asynchronous; this wave waits for them before its dots)
  if (is_router) {
    const uint16_t* row = first.wr + (size_t)r_row * H;
    for (int c0 = 0; c0 < (H >> 3); c0 += kWave)
      if (c0 + lane < (H >> 3))
        __builtin_amdgcn_global_load_lds((const QWS_GLOBAL void*)(row + (c0 + lane) * 8),
                                         (__attribute__((address_space(3))) void*)(wr_s + (size_t)wave * H + c0 * 8),
                                         16, 0, 0);
  }

  for (int l = 0; l < n_layers; ++l) {
    // an opaque copy of the thread index per layer: addresses derived from it are recomputed where
    // they are used instead of being hoisted out of the layer loop and kept live (spilled) across it
    unsigned tid_l = threadIdx.x;
    asm volatile("" : "+v"(tid_l));
    const int tid = (int)tid_l, lane = tid % kWave;   // shadow the kernel-level indices in this layer
    // descriptor of layer l: layer 0 from the kernel arguments, later ones from the LDS copy made
    // during the previous layer
    Layer L = first;
    if (l > 0) L = desc_from_lds(s_desc[l & 1]);
    // tags never 0: a zero-filled workspace holds tag 0
    const uint32_t tag_lg = tag_base + 4u * (uint32_t)l + 1u, tag_pt = tag_lg + 1u, tag_y = tag_lg + 2u;
    // the next layer's descriptor -> registers now, LDS after the router (its load has landed by then)
    unsigned long long next_desc = 0;
    const bool has_next = l + 1 < n_layers;
    if (has_next && wave == kWaves - 1 && lane < kDescWords)
      next_desc = ldg(reinterpret_cast<const unsigned long long*>(rest + (l + 1)) + lane);
    stamp(w, l, 0);

    // ------------------------------------------------------------------ 1: x
    if (l == 0) {
      for (int v = tid; v < M * H / 8; v += kThreads)
        *reinterpret_cast<u32x4_t*>(xs + v * 8) = ld16(L.x + (size_t)v * 8);
    } else if (sh.chained) {
      // y of the previous layer, as its owners published it
      const int n = M * H / 2;
      constexpr int kXw = (M * kHMax / 2 + kThreads - 1) / kThreads;
      int idx[kXw];
      unsigned long long v[kXw];
#pragma unroll
      for (int q = 0; q < kXw; ++q) idx[q] = tid + q * kThreads < n ? tid + q * kThreads : -1;
      poll_tagged<kXw>(w, w.ytag, idx, tag_y - 4u, v);
#pragma unroll
      for (int q = 0; q < kXw; ++q)
        if (idx[q] >= 0) reinterpret_cast<uint32_t*>(xs)[idx[q]] = (uint32_t)v[q];
    } else {
      // x may have been written earlier in this launch: device-coherent loads
      const unsigned long long* src = reinterpret_cast<const unsigned long long*>(L.x);
      for (int v = tid; v < M * H / 4; v += kThreads) reinterpret_cast<unsigned long long*>(xs)[v] = ld_coherent(src + v);
    }
    __syncthreads();
    stamp(w, l, 1);

    // ------------------------------------------------------------------ 2: router, shared task
    if (is_router) {
      wait_mem();   // this wave's router-row copy into LDS has landed
      const uint16_t* wrow = wr_s + (size_t)wave * H;
      float acc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
      for (int t = 0; t < kRtCpl; ++t) {
        const int c = lane + t * kWave;
        if (c < (H >> 3)) {
          const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(wrow + c * 8);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + m * H + c * 8);
#pragma unroll
            for (int d = 0; d < 4; ++d) acc[m] = dot2(as_bf16x2(rv[d]), as_bf16x2(xv[d]), acc[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float s = wave_sum(acc[m]);
        if (lane == 0) {
          const float v = s + (L.bias ? ldg(L.bias + (size_t)m * L.bias_stride + r_row) : 0.0f);
          st_coherent(w.logits + (size_t)m * E + r_row, tagged(tag_lg, __float_as_uint(v)));
          if (L.logits_out) stg(L.logits_out + (size_t)m * E + r_row, v);
        }
      }
    }
    if (has_next && wave == kWaves - 1 && lane < kDescWords) s_desc[(l + 1) & 1][lane] = next_desc;
    stamp(w, l, 2);
    if (shared_task) {
      // the shared expert needs no routing: its tasks run while the logits are exchanged
      if (tid == 0) {
        un.mask[0] = (1u << M) - 1u;
        un.pair0[0] = 0;
#pragma unroll
        for (int m = 0; m < M; ++m) un.w[0][m] = 1.0f;
      }
      __syncthreads();
      TaskRegs sreg;
      task_load(L, sh, E, b - (G - J), tid, sreg);
      task_compute<M>(sh, w, sreg, un, 0, b - (G - J), xs, a_s, tid, tag_pt);
    }
    stamp(w, l, 3);

    // ------------------------------------------------------------------ 3: top-K and union
    select_topk<M>(sh, w, tag_lg, tid, wave, lane, cand, un, s_idx, s_w, s_wmax, s_cnt, s_sel, l);
    if (b == 0 && tid < M * sh.K) {
      const int m = tid / sh.K, r = tid - m * sh.K;
      if (L.topk_idx) stg(L.topk_idx + tid, s_idx[m][r]);
      if (L.topk_w) stg(L.topk_w + tid, s_w[m][r]);
    }
    __syncthreads();
    stamp(w, l, 5);

    // the next layer's router rows -> LDS, behind this layer's task loads
    if (has_next && is_router) {
      const uint16_t* nwr = reinterpret_cast<const uint16_t*>(
          uniform_u64(s_desc[(l + 1) & 1][offsetof(qws_moe_layer, w_router_bf16) / 8]));
      const uint16_t* row = nwr + (size_t)r_row * H;
      for (int c0 = 0; c0 < (H >> 3); c0 += kWave)
        if (c0 + lane < (H >> 3))
          __builtin_amdgcn_global_load_lds((const QWS_GLOBAL void*)(row + (c0 + lane) * 8),
                                           (__attribute__((address_space(3))) void*)(wr_s + (size_t)wave * H + c0 * 8),
                                           16, 0, 0);
    }

    // ------------------------------------------------------------------ 4: routed tasks
    {
      const int n_rt = (un.n - ns) * J;
      for (int q = b; q < n_rt; q += G) {
        TaskRegs cur;
        const int u = ns + q / J;
        task_load(L, sh, un.id[u], q % J, tid, cur);
        task_compute<M>(sh, w, cur, un, u, q % J, xs, a_s, tid, tag_pt);
      }
    }
    stamp(w, l, 6);

    // ------------------------------------------------------------------ 5: combine owned rows
    if (my_rows > 0) {
      const int np = un.n_pairs;
      const int n_words = np * J * R;
      const unsigned long long* src = w.partial + (size_t)b * sh.P * J * R;
      for (int base = 0; base < n_words; base += kPollBatch * kThreads) {
        int idx[kPollBatch];
        unsigned long long v[kPollBatch];
#pragma unroll
        for (int q = 0; q < kPollBatch; ++q) {
          const int i = base + tid + q * kThreads;
          idx[q] = i < n_words ? i : -1;
        }
        poll_tagged<kPollBatch>(w, src, idx, tag_pt, v);
#pragma unroll
        for (int q = 0; q < kPollBatch; ++q)
          if (idx[q] >= 0) red[idx[q]] = __uint_as_float((uint32_t)v[q]);
      }
      __syncthreads();
      stamp(w, l, 7);
      // y[m][row] = sum over token m's pairs (slot order) and blocks; kSumLanes lanes per (m, row)
      {
        const int grp = tid / kSumLanes, s = tid % kSumLanes;
        const int m = grp / kMaxRows, rl = grp % kMaxRows;
        float acc = 0.0f;
        if (m < M && rl < my_rows) {
          const int npm = un.tok_n[m];
          for (int i = 0; i < npm; ++i) {
            const float* rp = red + (size_t)un.tok_pair[m][i] * J * R + rl;
            for (int j = s; j < J; j += kSumLanes) acc += rp[j * R];
          }
        }
        acc = row8_sum(acc);
        if (s == 0 && m < M && rl < my_rows) s_y[m][rl] = acc;
      }
      __syncthreads();
      stamp(w, l, 13);
      // outputs: a thread takes two adjacent rows of one token (the tagged copy holds a bf16 pair)
      for (int t = tid; t < (my_rows / 2) * M; t += kThreads) {
        const int rp = t / M, m = t - rp * M;
        const float y0 = s_y[m][2 * rp], y1 = s_y[m][2 * rp + 1];
        const size_t o = (size_t)m * H + row0 + 2 * rp;
        const uint16_t h0 = f32_to_bf16_rne(y0), h1 = f32_to_bf16_rne(y1);
        if (L.y32) {
          st_coherent(L.y32 + o, y0);
          st_coherent(L.y32 + o + 1, y1);
        }
        if (L.y16) {
          st_coherent(L.y16 + o, h0);
          st_coherent(L.y16 + o + 1, h1);
        }
        if (sh.chained && l + 1 < n_layers)
          st_coherent(w.ytag + o / 2, tagged(tag_y, (uint32_t)h0 | ((uint32_t)h1 << 16)));
      }
    }
    stamp(w, l, 8);
    if (!sh.chained && l + 1 < n_layers) {
      tagged_barrier(w, tag_y, tid, l);   // layer l's output is written before layer l+1 starts
      stamp(w, l, 9);
    } else {
      __syncthreads();      // LDS (union, s_y, red) is rewritten by the next layer
    }
  }
}

// ------------------------------------------------------------------------------ block-major down
// down_q [n][H][I/2] -> [n][I/32][H][16] and down_s [n][H][I/32] -> [n][I/32][H]; one thread per
// (expert, row, block) chunk, reading in canonical order.
__global__ void pack_down_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, long long n_chunks,
                                 int H, int J, uint8_t* __restrict__ qp, uint8_t* __restrict__ sp) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n_chunks;
       i += (long long)gridDim.x * blockDim.x) {
    const long long per_e = (long long)H * J;
    const long long e = i / per_e, rem = i - e * per_e;
    const long long row = rem / J, j = rem - row * J;
    const long long dst = (e * J + j) * H + row;
    *reinterpret_cast<u32x4_t*>(qp + dst * 16) = ld16(q + i * 16);
    sp[dst] = s[i];
  }
}

// ------------------------------------------------------------------------------ host side
int g_grid[64];       // workgroups per launch, per device (one per CU)
unsigned long long* g_trace[64];  // per device: trace buffer registered by qws_debug_trace_buffer
size_t g_trace_bytes[64];
constexpr size_t kMaxDynLds = 160 * 1024 - 16 * 1024;

size_t lds_bytes(int M, int E, int H, int P, int J, int R, int nrw) {
  const size_t sel = (size_t)M * E * 8, comb = (size_t)P * J * R * 4;
  return (size_t)M * H * 2 + (size_t)nrw * H * 2 + (sel > comb ? sel : comb);
}

size_t ws_layout(int M, int K, int E, int H, int I, char* base, Work* w) {
  const size_t sync = qws_host::align256(kSyncCounters * kSyncStride * 8);
  const size_t misc = 256;   // launch counter, error count
  const size_t lg = qws_host::align256((size_t)M * E * 8);
  const size_t yt = qws_host::align256((size_t)M * H * 4);
  const size_t dn = qws_host::align256((size_t)kMaxGrid * 8);
  const size_t part = qws_host::align256((size_t)M * (K + 1) * (I / kBlk) * (H + kRowsPad) * 8);
  if (w) {
    w->trace = nullptr;
    w->sync = reinterpret_cast<unsigned long long*>(base);
    w->launches = reinterpret_cast<unsigned long long*>(base + sync);
    w->errors = reinterpret_cast<unsigned*>(base + sync + 128);
    w->logits = reinterpret_cast<unsigned long long*>(base + sync + misc);
    w->ytag = reinterpret_cast<unsigned long long*>(base + sync + misc + lg);
    w->done = reinterpret_cast<unsigned long long*>(base + sync + misc + lg + yt);
    w->partial = reinterpret_cast<unsigned long long*>(base + sync + misc + lg + yt + dn);
  }
  return sync + misc + lg + yt + dn + part;
}

int grid_for_device(int* G) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return qws_host::set_device_error(e);
  if (dev < 0 || dev >= 64) return QWS_ERR_DEVICE;
  if (g_grid[dev] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return qws_host::set_device_error(e);
    g_grid[dev] = cus;
  }
  *G = g_grid[dev];
  return QWS_OK;
}

int check_layer(const qws_moe_layer& d, int E, int H, int I, int has_shared) {
  if (!d.x_bf16 || !d.w_router_bf16 || (!d.y_bf16 && !d.y_f32)) return QWS_ERR_ARG;
  const qws_mxfp4_experts& x = d.experts;
  if (x.format != QWS_FMT_MXFP4_E2M1_E8M0_B32_DOWN_BLOCKMAJOR) return QWS_ERR_FORMAT;
  if (!x.gate_up_q || !x.gate_up_s || !x.down_q || !x.down_s) return QWS_ERR_ARG;
  if (x.n_routed != E || x.hidden != H || x.inter != I || x.has_shared != has_shared) return QWS_ERR_SHAPE;
  if (d.bias && !(d.bias_row_stride == 0 || d.bias_row_stride == E)) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(d.x_bf16) || !qws_host::aligned16(d.w_router_bf16) || !qws_host::aligned16(x.gate_up_q) ||
      !qws_host::aligned16(x.down_q))
    return QWS_ERR_ALIGN;
  return QWS_OK;
}

template <int M>
int launch(const Layer& first, const qws_moe_layer* rest, int n, const Shape& sh, const Work& w, int G, size_t lds,
           hipStream_t s) {
  static bool configured[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (!configured[dev]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_layers_kernel<M>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxDynLds);
    if (e != hipSuccess) return qws_host::set_device_error(e);
    configured[dev] = true;
  }
  // the in-kernel hand-offs need every workgroup resident at once: one per compute unit
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_layers_kernel<M>, kThreads, lds);
  if (e != hipSuccess) return qws_host::set_device_error(e);
  if (per_cu < 1) return QWS_ERR_SHAPE;
  hipLaunchKernelGGL(moe_layers_kernel<M>, dim3(G), dim3(kThreads), lds, s, first, rest, n, sh, w);
  return qws_host::check_launch();
}

int run_layers(const qws_moe_layer* host, const qws_moe_layer* dev_copy, int n_layers, int M, int K,
               void* workspace, size_t workspace_bytes, qws_stream_t stream) {
  if (!host || n_layers < 1) return QWS_ERR_ARG;
  if (n_layers > 1 && !dev_copy) return QWS_ERR_ARG;
  if (n_layers > kMaxLayers) return QWS_ERR_SHAPE;
  const qws_mxfp4_experts& x0 = host[0].experts;
  const int E = x0.n_routed, H = x0.hidden, I = x0.inter, hs = x0.has_shared;
  if (M < 1 || M > kMaxM || K < 1 || K > kMaxK || E < K || E > kMaxE) return QWS_ERR_SHAPE;
  if (H < 32 || H > kHMax || H % 32 || I < 32 || I > kIMax || I % 32 || (hs != 0 && hs != 1)) return QWS_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    const int st = check_layer(host[l], E, H, I, hs);
    if (st != QWS_OK) return st;
  }
  if (!workspace || workspace_bytes < ws_layout(M, K, E, H, I, nullptr, nullptr)) return QWS_ERR_WORKSPACE;
  if (!qws_host::aligned16(workspace)) return QWS_ERR_ALIGN;
  if (dev_copy && (reinterpret_cast<uintptr_t>(dev_copy) & 7u)) return QWS_ERR_ALIGN;
  int G = 0;
  int st = grid_for_device(&G);
  if (st != QWS_OK) return st;
  const int J = I / kBlk;
  const int nrw = (E + G - 1) / G;
  const int R = ((H + G - 1) / G + 1) & ~1;   // even, so a thread writes a bf16 pair of one token
  if (G > kMaxGrid || G < J || nrw > kWaves || R > kMaxRows || (size_t)G * R > (size_t)H + kRowsPad ||
      G * R > kThreads * kDnRpl || M * kMaxRows * kSumLanes > kThreads)
    return QWS_ERR_SHAPE;
  const int P = M * (K + 1);
  const size_t lds = lds_bytes(M, E, H, P, J, R, nrw);
  if (lds > kMaxDynLds) return QWS_ERR_SHAPE;
  // Chained: layer l+1 reads y of layer l. Then the layers need no barrier, provided every
  // workgroup computes router rows and owns output rows, so that no workgroup can fall a layer
  // behind the others (each layer waits for every workgroup's logits and every owner's y).
  bool chained = n_layers > 1 && E >= G && (size_t)(G - 1) * R < (size_t)H;
  for (int l = 0; chained && l + 1 < n_layers; ++l)
    chained = host[l].y_bf16 != nullptr && host[l + 1].x_bf16 == host[l].y_bf16;
  Work w;
  ws_layout(M, K, E, H, I, static_cast<char*>(workspace), &w);
  {
    int dev = 0;
    (void)hipGetDevice(&dev);
    const size_t need = (size_t)n_layers * G * kTracePoints * 8;
    w.trace = (dev >= 0 && dev < 64 && g_trace[dev] && g_trace_bytes[dev] >= need) ? g_trace[dev] : nullptr;
  }
  const Shape sh{E, K, H, I, hs, R, P, chained ? 1 : 0, G * R, nrw};
  const Layer first = to_layer(host[0]);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (M) {
    case 1: return launch<1>(first, dev_copy, n_layers, sh, w, G, lds, s);
    case 2: return launch<2>(first, dev_copy, n_layers, sh, w, G, lds, s);
    case 3: return launch<3>(first, dev_copy, n_layers, sh, w, G, lds, s);
    default: return launch<4>(first, dev_copy, n_layers, sh, w, G, lds, s);
  }
}

}  // namespace

extern "C" size_t moe_layer_workspace_bytes(int M, int K, int E, int hidden, int inter) {
  if (M < 1 || M > kMaxM || K < 1 || K > kMaxK || E < 1 || E > kMaxE || hidden < 32 || hidden > kHMax || inter < 32 ||
      inter > kIMax)
    return 0;
  return ws_layout(M, K, E, hidden, inter, nullptr, nullptr);
}

extern "C" int moe_layer_mxfp4(const qws_moe_layer* layer, int M, int K, void* workspace, size_t workspace_bytes,
                               qws_stream_t stream) {
  return run_layers(layer, nullptr, 1, M, K, workspace, workspace_bytes, stream);
}

extern "C" int moe_layers_mxfp4(const qws_moe_layer* layers_host, const qws_moe_layer* layers_device, int n_layers,
                                int M, int K, void* workspace, size_t workspace_bytes, qws_stream_t stream) {
  return run_layers(layers_host, layers_device, n_layers, M, K, workspace, workspace_bytes, stream);
}

extern "C" int moe_workspace_errors(const void* workspace, int M, int K, int E, int inter, unsigned* errors_out,
                                    qws_stream_t stream) {
  if (!workspace || !errors_out) return QWS_ERR_ARG;
  (void)M;
  (void)K;
  (void)E;
  (void)inter;
  Work w;
  ws_layout(1, 1, 1, 32, 32, static_cast<char*>(const_cast<void*>(workspace)), &w);  // fixed offset
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(errors_out, w.errors, sizeof(unsigned), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? QWS_OK : qws_host::set_device_error(e);
}

extern "C" int moe_pack_mxfp4(const qws_mxfp4_experts* src, unsigned char* down_q_out, unsigned char* down_s_out,
                              qws_mxfp4_experts* desc_out, qws_stream_t stream) {
  if (!src || !down_q_out || !down_s_out || !desc_out) return QWS_ERR_ARG;
  if (src->format != QWS_FMT_MXFP4_E2M1_E8M0_B32) return QWS_ERR_FORMAT;
  if (!src->gate_up_q || !src->gate_up_s || !src->down_q || !src->down_s) return QWS_ERR_ARG;
  if (src->has_shared != 0 && src->has_shared != 1) return QWS_ERR_ARG;
  if (src->n_routed < 1 || src->n_routed > kMaxE) return QWS_ERR_SHAPE;
  if (src->hidden < 32 || src->hidden > kHMax || src->hidden % 32) return QWS_ERR_SHAPE;
  if (src->inter < 32 || src->inter > kIMax || src->inter % 32) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(src->down_q) || !qws_host::aligned16(down_q_out)) return QWS_ERR_ALIGN;
  const int H = src->hidden, J = src->inter / kBlk;
  const long long n = (long long)(src->n_routed + src->has_shared) * H * J;
  const long long want = (n + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_down_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), src->down_q,
                     src->down_s, n, H, J, down_q_out, down_s_out);
  const int st = qws_host::check_launch();
  if (st == QWS_OK) {
    *desc_out = *src;
    desc_out->format = QWS_FMT_MXFP4_E2M1_E8M0_B32_DOWN_BLOCKMAJOR;
    desc_out->down_q = down_q_out;
    desc_out->down_s = down_s_out;
  }
  return st;
}

extern "C" int qws_debug_trace_buffer(void* buf, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return qws_host::set_device_error(e);
  if (dev < 0 || dev >= 64) return QWS_ERR_DEVICE;
  if (buf && !qws_host::aligned16(buf)) return QWS_ERR_ALIGN;
  g_trace[dev] = static_cast<unsigned long long*>(buf);
  g_trace_bytes[dev] = buf ? bytes : 0;
  return QWS_OK;
}
