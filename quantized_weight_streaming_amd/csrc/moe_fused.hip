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
// activations never cross workgroups -- and writes H partial sums per token. The down projection
// is stored block-major (moe_pack_mxfp4) so that block j of an expert is one contiguous stream.
//
// Hand-offs between workgroups carry their own validity: a 64-bit word holds a 32-bit value and a
// 32-bit tag unique to (launch, layer, kind), written with one device-coherent store and polled
// with device-coherent loads (64-bit accesses are single-copy atomic), so a reader needs no
// separate signal, fence or counter. Per layer:
//   1  this workgroup's router rows are loaded (they need no x), then x into LDS: layer 0 from the
//      caller's buffer; in a chained sequence (x of layer l+1 is y of layer l) from the tagged copy
//      of y the previous layer published.
//   2  router dots -> tagged logits; workgroups G-J .. G-1 run the shared expert's J tasks (they
//      need no routing) -> tagged partials.
//   3  every workgroup selects top-K itself from the tagged logits: 8 waves take 64-expert chunks
//      (one logit per lane, K rounds of DPP max + lowest lane), one wave per token merges the chunk
//      candidates; softmax; union of the window's selections in LDS.
//   4  routed tasks, round-robin over workgroups (at M = 1 one task per workgroup).
//   5  workgroup b owns output rows [b*R, b*R + R): it polls their tagged partials, adds blocks then
//      slots in a fixed order (deterministic), writes y and, in a chained sequence, a tagged copy.
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
constexpr int kMaxChunks = kMaxE / kWave;
constexpr int kHMax = 2560;
constexpr int kIMax = 1024;
constexpr int kBlk = 32;        // activations per task: one MX block of the down projection
constexpr int kGuCpl = 5;       // 16-byte chunks per lane of a gate/up row: H <= 16 * 5 * 32
constexpr int kRtCpl = 5;       // router row: H <= 64 * 5 * 8
constexpr int kDnRpl = 5;       // down rows per thread in a task: H <= 512 * 5
constexpr int kMaxRows = 16;    // output rows owned by one workgroup
constexpr int kMaxGrid = 512;
constexpr int kRowsPad = 2 * kMaxGrid;   // partial buffer rows allowed beyond H (G * R >= H)
constexpr int kPollBatch = 12;  // tagged words per thread in flight while polling partials
constexpr int kSyncCounters = 16;
constexpr int kSyncStride = 16;             // 64-bit words: 128 bytes apart
constexpr unsigned kSpinLimit = 1u << 20;   // polls before a wait gives up (~1 s)
constexpr int kTracePoints = 16;            // timestamps per (layer, workgroup) when tracing
constexpr int kTagsPerLaunch = 4096;        // tag space of one launch: 4 per layer
constexpr int kMaxLayers = kTagsPerLaunch / 4;

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
};

struct Work {
  unsigned long long* trace;     // NULL, or [n_layers][G][kTracePoints] wall-clock stamps (100 MHz)
  unsigned long long* sync;      // kSyncCounters monotonic counters, kSyncStride apart
  unsigned long long* launches;  // launch counter (each workgroup adds 1 per launch)
  unsigned* errors;              // count of bounded waits that timed out (sticky)
  unsigned long long* logits;    // [M][E] tagged logits
  unsigned long long* ytag;      // [M][H/2] tagged bf16 pairs of y (chained sequences)
  unsigned long long* partial;   // [G][P][J][R] tagged partial sums of the down projection
};

struct Union {
  int n;                       // slots: 0 = shared (if any), then routed ids ascending
  int id[kMaxSlots];
  unsigned mask[kMaxSlots];    // tokens using the slot
  int pair0[kMaxSlots];        // first (slot, token) pair index of the slot
  float w[kMaxSlots][kMaxM];   // gate weight of (slot, token)
  int n_pairs;
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

// Reloads word Q .. N-1 of a poll, keeping those that already carry `tag` (compile-time recursion
// rather than a loop: the loop form was not unrolled inside the wait loop, which put v in scratch).
template <int Q, int N>
__device__ __forceinline__ void reload_tagged(const unsigned long long* src, int i0, int stride, int n, uint32_t tag,
                                              unsigned long long (&v)[N]) {
  if constexpr (Q < N) {
    const unsigned long long nv = ld_coherent(src + min(i0 + Q * stride, n - 1));
    v[Q] = tag_of(v[Q]) == tag ? v[Q] : nv;
    reload_tagged<Q + 1, N>(src, i0, stride, n, tag, v);
  }
}

// Loads src[i0 + q * stride] (clamped to n - 1) for q < N and waits until each carries `tag`.
// Every lane of the wave must call it (the wait is wave-wide).
template <int N>
__device__ __forceinline__ void poll_tagged(const Work& w, const unsigned long long* src, int i0, int stride, int n,
                                            uint32_t tag, unsigned long long (&v)[N]) {
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = ld_coherent(src + min(i0 + q * stride, n - 1));
  unsigned spins = 0;
  while (true) {
    bool ok = true;
#pragma unroll
    for (int q = 0; q < N; ++q) ok = ok && tag_of(v[q]) == tag;
    if (__all(ok)) break;
    if (wait_expired(w, spins)) break;
    reload_tagged<0, N>(src, i0, stride, n, tag, v);
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

// ------------------------------------------------------------------------------ DPP reductions
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
// Wave-uniform max / min of a uint32 across 64 lanes: quad xor-1, xor-2, half-row and row mirrors
// leave each 16-lane row with its extreme in every lane; four readlanes finish it.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<0xB1>(v));
  v = max(v, dpp<0x4E>(v));
  v = max(v, dpp<0x141>(v));
  v = max(v, dpp<0x140>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp<0xB1>(v));
  v = min(v, dpp<0x4E>(v));
  v = min(v, dpp<0x141>(v));
  v = min(v, dpp<0x140>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// Selection key: order-preserving float -> uint32 (larger float, larger key; -0 == +0; NaN ranks
// as -inf). Every logit maps to >= 0x007fffff; 0 marks a taken or absent entry.
__device__ __forceinline__ uint32_t sel_key(float f) {
  if (f != f) f = -__builtin_inff();
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ------------------------------------------------------------------------------ tasks
struct TaskRegs {
  u32x4_t g[kGuCpl], u[kGuCpl], d[kDnRpl];
  uint32_t gs[kGuCpl], us[kGuCpl], ds[kDnRpl];
};

// Issues the loads of task (expert e, block j). 16-lane group g of the workgroup takes gate row
// 32j+g and up row I+32j+g (lane j16: chunks j16, j16+16, ...); thread t takes down rows t, t+512, ...
// Addresses are a wave-uniform 64-bit base plus a 32-bit per-thread offset, so that the per-thread
// part stays one register across the layer loop.
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
  // by the compute; a down row past H is loaded from row H-1 and its partial sum is zeroed.
#pragma unroll
  for (int t = 0; t < kGuCpl; ++t) {
    const unsigned c = min(j16 + 16u * t, nch - 1);
    r.g[t] = ld16(gq + g * rb + c * 16u);
    r.u[t] = ld16(uq + g * rb + c * 16u);
    r.gs[t] = ldg(gs + g * nch + c);
    r.us[t] = ldg(us + g * nch + c);
  }
  const size_t blk = ((size_t)e * J + j) * (size_t)H;
  const uint8_t* dq = L.dq + blk * 16;
  const uint8_t* ds = L.ds + blk;
#pragma unroll
  for (int t = 0; t < kDnRpl; ++t) {
    const unsigned row = min(tid + (unsigned)(kThreads * t), (unsigned)H - 1);
    r.d[t] = ld16(dq + row * 16u);
    r.ds[t] = ldg(ds + row);
  }
}

// Computes task (block j, tokens in `mask`, pairs p0 + rank) from its loaded registers: the block's
// activations silu(gate) * up into LDS, then partial[p][j][row] = sum_k W_down[row][32j+k] * a[k]
// for every row, stored tagged at this thread's row offsets.
template <int M>
__device__ __forceinline__ void task_compute(const Shape& sh, const Work& w, const TaskRegs& r, unsigned mask,
                                             int p0, int j, const uint16_t* xs, float* a_s, unsigned tid,
                                             uint32_t tag) {
  const int g = tid >> 4, j16 = tid & 15;
  const int H = sh.H, nch = H >> 5, J = sh.I / kBlk, R = sh.R;
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
    const float hg = group_sum<16>(ag[m]);
    const float hu = group_sum<16>(au[m]);
    if (j16 == 0) a_s[m * kBlk + g] = silu(hg) * hu;
  }
  __syncthreads();
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
        const int p = p0 + __popc(mask & ((1u << m) - 1u));
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
        if (row >= H) s = 0.0f;
        if (row < sh.rows_total) st_coherent(w.partial + (size_t)(p * J + j) * R + rowoff, tagged(tag, __float_as_uint(s)));
      }
    }
  }
  __syncthreads();  // a_s is rewritten by the next task
}

// ------------------------------------------------------------------------------ the kernel
template <int M>
__global__ __launch_bounds__(kThreads) void moe_layers_kernel(Layer first, const qws_moe_layer* __restrict__ rest,
                                                              int n_layers, Shape sh, Work w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ Union un;
  __shared__ int s_idx[kMaxM][kMaxK];
  __shared__ float s_w[kMaxM][kMaxK];
  __shared__ uint32_t s_ck[kMaxM][kMaxChunks][kMaxK];   // chunk candidates: key
  __shared__ int s_ci[kMaxM][kMaxChunks][kMaxK];        // chunk candidates: expert index
  __shared__ __attribute__((aligned(16))) float a_s[kMaxM * kBlk];
  __shared__ float s_red2[kMaxPairs][kMaxRows];
  __shared__ unsigned long long s_launch;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int G = gridDim.x, b = blockIdx.x;
  const int E = sh.E, K = sh.K, H = sh.H, I = sh.I, R = sh.R, P = sh.P;
  const int J = I / kBlk;
  const int ns = sh.has_shared ? 1 : 0;

  // dynamic LDS: x [M][H] bf16 | partial sums of this workgroup's rows [pairs][J][R] fp32
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  float* red = reinterpret_cast<float*>(lds + (size_t)M * H * 2);

  const int nrw = (E + G - 1) / G;   // router rows (waves) per workgroup
  const int row0 = b * R;
  const int my_rows = max(0, min(R, H - row0));
  const int nchunks = (E + kWave - 1) / kWave;
  const bool shared_task = sh.has_shared && b >= G - J;
  SyncState sync{0ull, false};

  // launch number -> this launch's tag base (every workgroup adds 1 per launch)
  if (tid == 0)
    s_launch = __hip_atomic_fetch_add(w.launches, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) / (unsigned)G;
  __syncthreads();
  const uint32_t tag_base = (uint32_t)(s_launch * kTagsPerLaunch);
  if (s_launch > 0 && tag_base == 0) {
    // tags repeat from here on: clear every tagged word (tag 0 is never valid) before any use
    const size_t own = (size_t)P * J * R;
    for (size_t i = tid; i < own; i += kThreads) st_coherent(w.partial + (size_t)b * own + i, 0ull);
    for (int i = b * kThreads + tid; i < M * E; i += G * kThreads) st_coherent(w.logits + i, 0ull);
    for (int i = b * kThreads + tid; i < M * H / 2; i += G * kThreads) st_coherent(w.ytag + i, 0ull);
    grid_sync(w, sync);
  }

  for (int l = 0; l < n_layers; ++l) {
    const Layer L = l == 0 ? first : to_layer(rest[l]);
    // an opaque copy of the thread index per layer: addresses derived from it are recomputed where
    // they are used instead of being hoisted out of the layer loop and kept live (spilled) across it
    unsigned tid_l = threadIdx.x;
    asm volatile("" : "+v"(tid_l));
    const int tid = (int)tid_l, lane = tid % kWave;   // shadows the kernel-level index in this layer
    // tags never 0: a zero-filled workspace holds tag 0
    const uint32_t tag_lg = tag_base + 4u * (uint32_t)l + 1u, tag_pt = tag_lg + 1u, tag_y = tag_lg + 2u;
    stamp(w, l, 0);
    // ------------------------------------------------------------------ 1: loads without x, then x
    const int r_row = b + G * wave;
    const bool is_router = wave < nrw && r_row < E;
    u32x4_t rw[kRtCpl];
    if (is_router) {
      const uint16_t* row = L.wr + (size_t)r_row * H;
#pragma unroll
      for (int t = 0; t < kRtCpl; ++t) {
        const unsigned c = (unsigned)(lane + t * kWave), nc = (unsigned)(H >> 3);
        rw[t] = ld16(row + min(c, nc - 1) * 8u);   // a chunk past the row end is skipped below
      }
    }
    if (l == 0) {
      for (int v = tid; v < M * H / 8; v += kThreads)
        *reinterpret_cast<u32x4_t*>(xs + v * 8) = ld16(L.x + (size_t)v * 8);
    } else if (sh.chained) {
      // y of the previous layer, as its owners published it
      const int n = M * H / 2;
      constexpr int kXw = (M * kHMax / 2 + kThreads - 1) / kThreads;
      unsigned long long v[kXw];
      poll_tagged<kXw>(w, w.ytag, tid, kThreads, n, tag_y - 4u, v);
#pragma unroll
      for (int q = 0; q < kXw; ++q)
        if (tid + q * kThreads < n) reinterpret_cast<uint32_t*>(xs)[tid + q * kThreads] = (uint32_t)v[q];
    } else {
      // x may have been written earlier in this launch: device-coherent loads
      const unsigned long long* src = reinterpret_cast<const unsigned long long*>(L.x);
      for (int v = tid; v < M * H / 4; v += kThreads) reinterpret_cast<unsigned long long*>(xs)[v] = ld_coherent(src + v);
    }
    __syncthreads();
    stamp(w, l, 1);

    // ------------------------------------------------------------------ 2: router, shared task
    if (is_router) {
      float acc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        acc[m] = 0.0f;
#pragma unroll
        for (int t = 0; t < kRtCpl; ++t) {
          const int c = lane + t * kWave;
          if (c < (H >> 3)) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + m * H + c * 8);
#pragma unroll
            for (int d = 0; d < 4; ++d) acc[m] = dot2(as_bf16x2(rw[t][d]), as_bf16x2(xv[d]), acc[m]);
          }
        }
        acc[m] = group_sum<kWave>(acc[m]);
      }
      if (lane == 0) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float v = acc[m] + (L.bias ? ldg(L.bias + (size_t)m * L.bias_stride + r_row) : 0.0f);
          st_coherent(w.logits + (size_t)m * E + r_row, tagged(tag_lg, __float_as_uint(v)));
          if (L.logits_out) stg(L.logits_out + (size_t)m * E + r_row, v);
        }
      }
    }
    stamp(w, l, 2);
    if (shared_task) {
      // off the critical path (the routed tasks start a selection later), so its loads are not held
      // in registers across the x hand-off
      TaskRegs sreg;
      task_load(L, sh, E, b - (G - J), tid_l, sreg);
      task_compute<M>(sh, w, sreg, (1u << M) - 1u, 0, b - (G - J), xs, a_s, tid_l, tag_pt);
    }
    stamp(w, l, 3);

    // ------------------------------------------------------------------ 3: top-K and union
    // chunk pass: (token m, chunk c) per wave; K rounds of (max key, lowest lane holding it), so
    // equal logits go to the lower expert index
    for (int t = wave; t < M * nchunks; t += kWaves) {
      const int m = t / nchunks, c = t - m * nchunks;
      const int e = c * kWave + lane;
      unsigned long long v[1];
      poll_tagged<1>(w, w.logits + (size_t)m * E, e, 0, E, tag_lg, v);
      uint32_t key = e < E ? sel_key(__uint_as_float((uint32_t)v[0])) : 0u;
#pragma unroll
      for (int r = 0; r < kMaxK; ++r) {
        if (r < K) {
          const uint32_t vmax = wave_max_u32(key);
          const int win = __ffsll((unsigned long long)__ballot(key == vmax)) - 1;
          if (lane == win) key = 0u;
          if (lane == 0) {
            s_ck[m][c][r] = vmax;
            s_ci[m][c][r] = c * kWave + win;
          }
        }
      }
    }
    __syncthreads();
    stamp(w, l, 4);
    if (wave < M) {
      // merge token `wave`'s candidates; candidate c*K + r precedes c*K + r + 1 and chunk c + 1,
      // so among equal keys the lowest candidate position is the lowest expert index
      const int m = wave;
      const int nc = nchunks * K;
      uint32_t key[2];
      int idx[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = lane + h * kWave;
        const int c = i / K, r = i - c * K;
        key[h] = i < nc ? s_ck[m][c][r] : 0u;
        idx[h] = i < nc ? s_ci[m][c][r] : 0;
      }
      uint32_t kv[kMaxK];
      int ki[kMaxK];
#pragma unroll
      for (int r = 0; r < kMaxK; ++r) {
        if (r < K) {
          const uint32_t vmax = wave_max_u32(max(key[0], key[1]));
          uint32_t li = key[1] == vmax ? (uint32_t)(lane + kWave) : 0xffffffffu;
          li = key[0] == vmax ? (uint32_t)lane : li;
          const uint32_t win = wave_min_u32(li);
          const int hw = (int)(win / kWave), lw = (int)(win % kWave);
          ki[r] = __builtin_amdgcn_readlane(hw ? idx[1] : idx[0], lw);
          kv[r] = vmax;
          if (lane == lw) {
            if (hw) key[1] = 0u;
            else key[0] = 0u;
          }
        }
      }
      if (lane == 0) {
        const float vmax = key_to_float(kv[0]);
        float z[kMaxK], s = 0.0f;
#pragma unroll
        for (int r = 0; r < kMaxK; ++r)
          if (r < K) {
            z[r] = expf(key_to_float(kv[r]) - vmax);
            s += z[r];
          }
#pragma unroll
        for (int r = 0; r < kMaxK; ++r)
          if (r < K) {
            s_idx[m][r] = ki[r];
            s_w[m][r] = z[r] / s;
          }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // union of the window's selections: slot 0 = shared expert (if any), then routed ids
      // ascending. Lane j holds selection j (token j / K); loops over a uniform index use readlane.
      const int n = M * K;
      const int mj = lane / K;
      const int e = lane < n ? s_idx[mj][lane - mj * K] : -1;
      const float wj = lane < n ? s_w[mj][lane - mj * K] : 0.0f;
      bool first_occ = lane < n;
      unsigned mask = 0;
      float wsum[M];
#pragma unroll
      for (int m = 0; m < M; ++m) wsum[m] = 0.0f;
      for (int i = 0; i < n; ++i) {
        const int ei = __builtin_amdgcn_readlane(e, i);
        const int mi = __builtin_amdgcn_readlane(mj, i);
        const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), i));
        if (ei == e) {
          if (i < lane) first_occ = false;
          mask |= 1u << mi;
#pragma unroll
          for (int m = 0; m < M; ++m)
            if (m == mi) wsum[m] += wi;
        }
      }
      const unsigned long long firsts = __ballot(first_occ);
      int rank = 0;
      for (int i = 0; i < n; ++i)
        if ((firsts >> i) & 1ull) rank += __builtin_amdgcn_readlane(e, i) < e ? 1 : 0;
      const int cnt = __popc(mask);
      int pair0 = ns * M, total = pair0;
      for (int i = 0; i < n; ++i)
        if ((firsts >> i) & 1ull) {
          const int ci = __builtin_amdgcn_readlane(cnt, i);
          pair0 += __builtin_amdgcn_readlane(rank, i) < rank ? ci : 0;
          total += ci;
        }
      if (first_occ) {
        const int slot = ns + rank;
        un.id[slot] = e;
        un.mask[slot] = mask;
        un.pair0[slot] = pair0;
#pragma unroll
        for (int m = 0; m < M; ++m) un.w[slot][m] = wsum[m];
      }
      if (lane == 0) {
        if (ns) {
          un.id[0] = E;
          un.mask[0] = (1u << M) - 1u;
          un.pair0[0] = 0;
#pragma unroll
          for (int m = 0; m < M; ++m) un.w[0][m] = 1.0f;
        }
        un.n = __popcll(firsts) + ns;
        un.n_pairs = total;
      }
    }
    if (b == 0 && tid < M * K) {
      if (L.topk_idx) stg(L.topk_idx + tid, s_idx[tid / K][tid % K]);
      if (L.topk_w) stg(L.topk_w + tid, s_w[tid / K][tid % K]);
    }
    __syncthreads();
    stamp(w, l, 5);

    // ------------------------------------------------------------------ 4: routed tasks
    {
      const int n_rt = (un.n - ns) * J;
      for (int q = b; q < n_rt; q += G) {
        TaskRegs cur;
        const int u = ns + q / J;
        task_load(L, sh, un.id[u], q % J, tid_l, cur);
        task_compute<M>(sh, w, cur, un.mask[u], un.pair0[u], q % J, xs, a_s, tid_l, tag_pt);
      }
    }
    stamp(w, l, 6);

    // ------------------------------------------------------------------ 5: combine owned rows
    if (my_rows > 0) {
      const int np = un.n_pairs;
      const int n_words = np * J * R;
      const unsigned long long* src = w.partial + (size_t)b * P * J * R;
      for (int base = 0; base < n_words; base += kPollBatch * kThreads) {
        unsigned long long v[kPollBatch];
        poll_tagged<kPollBatch>(w, src, base + tid, kThreads, n_words, tag_pt, v);
#pragma unroll
        for (int q = 0; q < kPollBatch; ++q) {
          const int i = base + tid + q * kThreads;
          if (i < n_words) red[i] = __uint_as_float((uint32_t)v[q]);
        }
      }
      __syncthreads();
      stamp(w, l, 7);
      // blocks first: s_red2[p][row] = sum_j partial[p][j][row], j ascending
      for (int t = tid; t < np * R; t += kThreads) {
        const int p = t / R, rl = t - p * R;
        float s = 0.0f;
        for (int j = 0; j < J; ++j) s += red[(p * J + j) * R + rl];
        s_red2[p][rl] = s;
      }
      __syncthreads();
      // then slots, in slot order: y[m][row] = sum_u w[u][m] * s_red2[pair(u, m)][row]; a thread
      // takes two adjacent rows of one token so that the tagged copy holds a bf16 pair
      const int U = un.n;
      for (int t = tid; t < (my_rows / 2) * M; t += kThreads) {
        const int rp = t / M, m = t - rp * M;
        float y0 = 0.0f, y1 = 0.0f;
        for (int u = 0; u < U; ++u) {
          const unsigned mk = un.mask[u];
          if ((mk >> m) & 1u) {
            const int p = un.pair0[u] + __popc(mk & ((1u << m) - 1u));
            y0 += un.w[u][m] * s_red2[p][2 * rp];
            y1 += un.w[u][m] * s_red2[p][2 * rp + 1];
          }
        }
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
      grid_sync(w, sync);   // layer l's output is written before layer l+1 starts
      stamp(w, l, 9);
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

size_t lds_bytes(int M, int H, int P, int J, int R) { return (size_t)M * H * 2 + (size_t)P * J * R * 4; }

size_t ws_layout(int M, int K, int E, int H, int I, char* base, Work* w) {
  const size_t sync = qws_host::align256(kSyncCounters * kSyncStride * 8);
  const size_t misc = 256;   // launch counter, error count
  const size_t lg = qws_host::align256((size_t)M * E * 8);
  const size_t yt = qws_host::align256((size_t)M * H * 4);
  const size_t part = qws_host::align256((size_t)M * (K + 1) * (I / kBlk) * (H + kRowsPad) * 8);
  if (w) {
    w->trace = nullptr;
    w->sync = reinterpret_cast<unsigned long long*>(base);
    w->launches = reinterpret_cast<unsigned long long*>(base + sync);
    w->errors = reinterpret_cast<unsigned*>(base + sync + 128);
    w->logits = reinterpret_cast<unsigned long long*>(base + sync + misc);
    w->ytag = reinterpret_cast<unsigned long long*>(base + sync + misc + lg);
    w->partial = reinterpret_cast<unsigned long long*>(base + sync + misc + lg + yt);
  }
  return sync + misc + lg + yt + part;
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
  int G = 0;
  int st = grid_for_device(&G);
  if (st != QWS_OK) return st;
  const int J = I / kBlk;
  const int nrw = (E + G - 1) / G;
  const int R = ((H + G - 1) / G + 1) & ~1;   // even, so a thread writes a bf16 pair of one token
  if (G > kMaxGrid || G < J || nrw > kWaves || R > kMaxRows || (size_t)G * R > (size_t)H + kRowsPad ||
      G * R > kThreads * kDnRpl)
    return QWS_ERR_SHAPE;
  const int P = M * (K + 1);
  const size_t lds = lds_bytes(M, H, P, J, R);
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
  const Shape sh{E, K, H, I, hs, R, P, chained ? 1 : 0, G * R};
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
