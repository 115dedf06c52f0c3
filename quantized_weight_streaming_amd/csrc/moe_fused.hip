// Fused MoE layer(s) on gfx950: router GEMV, top-K, softmax, expert union, MXFP4 gate_up + SwiGLU,
// MXFP4 down + gate-weighted combine with the shared expert -- one persistent launch for one or
// more layers (each layer routes eight of E routed experts plus one shared expert:
// runbyai.xyz/posts/593 paragraph 2; a window of M <= 4 tokens reads each activated expert once:
// paragraph 5).
//
// Why one launch: a kernel boundary costs ~1.7 us on MI355X even inside a HIP graph, about a third
// of a whole layer's streaming time at M = 1. So the layer runs as one grid of one workgroup per CU
// (all co-resident), and the three data hand-offs inside it use device-coherent stores/loads plus
// spread monotonic arrival counters (no agent-scope fence, no memset, no reset: graph-replay safe):
//   phase 1  router rows (one wave per row) and the shared expert's gate_up rows: their weight loads
//            do not depend on x and are issued first; x is staged in LDS; logits and the shared
//            expert's activations are written device-coherent.              -> sync
//   phase 2  every workgroup reads the M x E logits and selects top-K per token itself (one wave per
//            token, DPP max/min reductions), so no broadcast round trip is needed; union in LDS.
//   phase 3  routed gate_up (16 lanes per row, gate and up rows in partner groups, SwiGLU in
//            registers); the first batch of this workgroup's down rows is loaded before the gate_up
//            compute so it is in flight across the next sync.                 -> sync
//   phase 4  the workgroup owns ceil(H / G) output rows for every slot: activations staged in LDS,
//            8 lanes per down row, slot contributions reduced in LDS in slot order (deterministic),
//            y written device-coherent.                                        -> sync (next layer)
#include "qws_common.hpp"

namespace {

using namespace qws;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kGroups16 = kThreads / 16;   // 32 gate_up row groups
constexpr int kGroups8 = kThreads / 8;     // 64 down row groups
constexpr int kMaxM = 4;
constexpr int kMaxK = 8;
constexpr int kMaxSlots = kMaxM * kMaxK + 1;  // routed union + shared
constexpr int kMaxE = 1024;
constexpr int kGuCpl = 5;   // H <= 16 * 5 * 32 = 2560
constexpr int kRtCpl = 5;   // H <= 64 * 5 * 8 = 2560
constexpr int kDnCpl = 4;   // I <= 8 * 4 * 32 = 1024
constexpr int kHMax = 2560;
constexpr int kIMax = 1024;
constexpr int kSyncCounters = 16;
constexpr int kSyncStride = 16;             // 64-bit words: 128 bytes apart
constexpr unsigned kSpinLimit = 1u << 20;  // polls before a wait gives up (~1 s)

struct Layer {
  const uint16_t* x;
  const uint16_t* wr;
  const float* bias;
  long long bias_stride;
  const uint8_t* gq;
  const uint8_t* gs;
  const uint8_t* dq;
  const uint8_t* ds;
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
  int rows_per_wg;  // ceil(H / G): output rows each workgroup owns in phase 4
};

constexpr int kTracePoints = 16;  // timestamps per (layer, workgroup) when tracing

struct Work {
  unsigned long long* trace;  // NULL, or [n_layers][G][kTracePoints] wall-clock stamps (100 MHz)
  unsigned long long* sync;  // kSyncCounters monotonic counters, kSyncStride apart
  unsigned* errors;          // count of bounded waits that timed out
  float* logits;             // [M, E]
  float* act;                // [M * (K + 1), I] activation rows, one per (slot, token) pair
};

struct Union {
  int n;                       // slots: 0 = shared (if any), then routed ids ascending
  int id[kMaxSlots];
  unsigned mask[kMaxSlots];    // tokens using the slot
  int pair0[kMaxSlots];        // first activation row of the slot
  float w[kMaxSlots][kMaxM];   // gate weight of (slot, token)
  int cnt[kMaxSlots];          // tokens using the slot
  int n_pairs;
};

__device__ __forceinline__ void stamp(const Work& w, int l, int k) {
  if (w.trace && threadIdx.x == 0)
    w.trace[((size_t)l * gridDim.x + blockIdx.x) * kTracePoints + k] = wall_clock64();
}

// ------------------------------------------------------------------------------ grid sync
// Every workgroup arrives once on counter blockIdx % 16; the counters only ever increase. The first
// hand-off of a launch learns its epoch from the value its atomic saw; later hand-offs of the same
// launch count epochs in registers. Completion is every counter c reaching (epoch + 1) *
// arrivals(c). Polling is bounded; a timeout is counted.
struct SyncState {
  unsigned long long epoch;  // valid in wave 0 once `known`
  bool known;
};

__device__ void grid_sync(const Work& w, SyncState& st, int l = 0, int k = -1) {
  wait_mem();
  __syncthreads();
  if (k >= 0) stamp(w, l, k);
  const unsigned G = gridDim.x;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const unsigned ncnt = G < (unsigned)kSyncCounters ? G : (unsigned)kSyncCounters;
    const unsigned c = blockIdx.x % ncnt;
    unsigned long long* mine = w.sync + c * kSyncStride;
    // a returning atomic: measured on MI355X, its increment is visible to pollers within ~1 us,
    // while a non-returning (posted) one took ~3 us
    unsigned long long prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(mine, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      if ((++spins & 255u) == 0) {
        // give up after kSpinLimit polls, or at once if any workgroup has already given up (the
        // error count is sticky: a workspace that saw a timeout must be zero-filled again)
        const bool other = ld_coherent(w.errors) != 0u;
        if (other || spins > kSpinLimit) {
          if (lane == 0 && !other) atomicAdd(w.errors, 1u);
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
    }
    st.epoch += 1;
  }
  if (k >= 0) stamp(w, l, k + 1);
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
__device__ __forceinline__ float wave_sum(float v) { return group_sum<kWave>(v); }

// Selection key: order-preserving float -> uint32 (larger float, larger key; -0 == +0). Every
// number maps to >= 0x007fffff; NaN maps to 1 (below every number); 0 marks a taken/absent entry.
__device__ __forceinline__ uint32_t sel_key(float f) {
  if (f != f) return 1u;
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Top-K of one token's E <= 64 * NV logits (device-coherent loads) by one wave: K rounds of (max
// key, then the lowest index holding it), so ties go to the lower index; softmax over the selection.
template <int NV>
__device__ __forceinline__ void topk_wave(const float* lg, int E, int K, int* sel_idx, float* sel_w) {
  const int lane = threadIdx.x % kWave;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = ld_coherent(lg + min(lane + i * kWave, E - 1));  // all in flight together
  uint32_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = lane + i * kWave < E ? sel_key(v[i]) : 0u;
  uint32_t kv[kMaxK];
  int ki[kMaxK];
#pragma unroll
  for (int r = 0; r < kMaxK; ++r) {
    if (r < K) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) m = max(m, key[i]);
      const uint32_t vmax = wave_max_u32(m);
      uint32_t li = 0xffffffffu;
#pragma unroll
      for (int i = NV - 1; i >= 0; --i) li = key[i] == vmax ? (uint32_t)(lane + i * kWave) : li;
      const uint32_t imin = wave_min_u32(li);
#pragma unroll
      for (int i = 0; i < NV; ++i) key[i] = (uint32_t)(lane + i * kWave) == imin ? 0u : key[i];
      kv[r] = vmax;
      ki[r] = (int)imin;
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
        sel_idx[r] = ki[r];
        sel_w[r] = z[r] / s;
      }
  }
}

// ------------------------------------------------------------------------------ row helpers
// Lane j of a 16-lane group loads chunks j, j+16, ... of one MXFP4 row (16 B nibbles + 1 scale).
__device__ __forceinline__ void load_fp4_row16(const uint8_t* q, const uint8_t* s, int j, int nch, bool valid,
                                               u32x4_t (&wq)[kGuCpl], uint32_t (&wsc)[kGuCpl]) {
#pragma unroll
  for (int t = 0; t < kGuCpl; ++t) {
    const int c = j + 16 * t;
    if (valid && c < nch) {
      wq[t] = ld16(q + (size_t)c * 16);
      wsc[t] = s[c];
    } else {
      wq[t] = u32x4_t{0, 0, 0, 0};
      wsc[t] = 127;
    }
  }
}

// Partial dot (this lane's chunks) of one MXFP4 row with the tokens in `mask`; x in LDS (bf16).
template <int M>
__device__ __forceinline__ void dot_fp4_row16(const u32x4_t (&wq)[kGuCpl], const uint32_t (&wsc)[kGuCpl], int j,
                                              int nch, const uint16_t* xs, int H, unsigned mask, float (&acc)[M]) {
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int t = 0; t < kGuCpl; ++t) {
    const int c = j + 16 * t;
    if (c < nch) {
      const float sc = e8m0_to_f32(wsc[t]);
      bf16x2_t p[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        p[4 * d + 0] = fp4x2_to_bf16x2<0>(wq[t][d], sc);
        p[4 * d + 1] = fp4x2_to_bf16x2<1>(wq[t][d], sc);
        p[4 * d + 2] = fp4x2_to_bf16x2<2>(wq[t][d], sc);
        p[4 * d + 3] = fp4x2_to_bf16x2<3>(wq[t][d], sc);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if ((mask >> m) & 1u) {
          const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xs + m * H + c * 32);
          float a = acc[m];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4_t xv = xp[q];
            a = dot2(p[4 * q + 0], as_bf16x2(xv[0]), a);
            a = dot2(p[4 * q + 1], as_bf16x2(xv[1]), a);
            a = dot2(p[4 * q + 2], as_bf16x2(xv[2]), a);
            a = dot2(p[4 * q + 3], as_bf16x2(xv[3]), a);
          }
          acc[m] = a;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------ the kernel
template <int M>
__global__ __launch_bounds__(kThreads) void moe_layers_kernel(Layer first, const qws_moe_layer* __restrict__ rest,
                                                              int n_layers, Shape sh, Work w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ Union un;
  __shared__ int s_idx[kMaxM][kMaxK];
  __shared__ float s_w[kMaxM][kMaxK];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int G = gridDim.x, b = blockIdx.x;
  const int E = sh.E, K = sh.K, H = sh.H, I = sh.I;
  const int nch_h = H >> 5;      // 32-element blocks along H
  const int nch_i = I >> 5;      // along I
  const size_t gu_row_bytes = (size_t)(H >> 1), dn_row_bytes = (size_t)(I >> 1);
  const size_t gu_rows = 2 * (size_t)I;
  const int n_shared_slots = sh.has_shared ? 1 : 0;

  // dynamic LDS: x [M][H] bf16 | act [M*(K+1)][I] fp32 | red [kMaxSlots][rows_per_wg][M] fp32
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  float* acts = reinterpret_cast<float*>(lds + (size_t)M * H * 2);
  float* red = acts + (size_t)M * (K + 1) * I;

  const int nrw = (E + G - 1) / G;          // router rows (waves) per workgroup
  const int nsp = (I + G - 1) / G;          // shared-expert act indices per workgroup
  const int R0 = sh.rows_per_wg;
  const int row0 = b * R0;
  const int my_rows = max(0, min(R0, H - row0));
  SyncState sync{0ull, false};

  for (int l = 0; l < n_layers; ++l) {
    const Layer L = l == 0 ? first : to_layer(rest[l]);
    stamp(w, l, 0);
    // ------------------------------------------------------------------ phase 1
    // router row loads (waves 0 .. nrw-1, one row each) and shared gate_up row loads (16-lane
    // groups after the router waves: pair k -> groups 4*nrw + 2k (gate) and +1 (up))
    const int r_row = b + G * wave;
    const bool is_router = wave < nrw && r_row < E;
    u32x4_t rw[kRtCpl];
    const int gi = tid >> 4, j16 = tid & 15;
    const int sk = (gi - 4 * nrw) >> 1, s_up = (gi - 4 * nrw) & 1;
    const int s_i = b + G * sk;
    const bool is_shared = sh.has_shared && gi >= 4 * nrw && sk < nsp && s_i < I;
    u32x4_t swq[kGuCpl];
    uint32_t sws[kGuCpl];
    if (is_router) {
      const uint16_t* row = L.wr + (size_t)r_row * H;
#pragma unroll
      for (int t = 0; t < kRtCpl; ++t) {
        const int c = lane + t * kWave;
        rw[t] = c < (H >> 3) ? ld16(row + c * 8) : u32x4_t{0, 0, 0, 0};
      }
    }
    {
      const size_t row = (size_t)E * gu_rows + (size_t)(s_i + s_up * I);  // shared expert = index E
      load_fp4_row16(L.gq + row * gu_row_bytes, L.gs + row * nch_h, j16, nch_h, is_shared, swq, sws);
    }
    // x of the layer -> LDS
    for (int v = tid; v < M * H / 8; v += kThreads)
      *reinterpret_cast<u32x4_t*>(xs + v * 8) = ld16(L.x + (size_t)v * 8);
    __syncthreads();
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
        acc[m] = wave_sum(acc[m]);
      }
      if (lane == 0) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float v = acc[m] + (L.bias ? L.bias[(size_t)m * L.bias_stride + r_row] : 0.0f);
          st_coherent(w.logits + (size_t)m * E + r_row, v);
          if (L.logits_out) L.logits_out[(size_t)m * E + r_row] = v;
        }
      }
    }
    if (gi >= 4 * nrw && sh.has_shared) {
      float acc[M];
      dot_fp4_row16<M>(swq, sws, j16, nch_h, xs, H, (1u << M) - 1u, acc);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float h = group_sum<16>(acc[m]);
        const float partner = __shfl_xor(h, 16, kWave);
        if (is_shared && !s_up && j16 == 0) st_coherent(w.act + (size_t)m * I + s_i, silu(h) * partner);
      }
    }
    stamp(w, l, 1);
    grid_sync(w, sync, l, 8);
    stamp(w, l, 2);

    // ------------------------------------------------------------------ phase 2
    if (wave < M) {
      if (E <= 8 * kWave) topk_wave<8>(w.logits + (size_t)wave * E, E, K, &s_idx[wave][0], &s_w[wave][0]);
      else topk_wave<16>(w.logits + (size_t)wave * E, E, K, &s_idx[wave][0], &s_w[wave][0]);
    }
    __syncthreads();
    stamp(w, l, 14);
    if (wave == 0) {
      // union of the window's selections: slot 0 = shared expert (if any), then routed ids
      // ascending. Lane j holds selection j (token j / K); the loops run over a uniform index and
      // read other lanes with v_readlane.
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
      int pair0 = sh.has_shared ? M : 0, total = pair0;
      for (int i = 0; i < n; ++i)
        if ((firsts >> i) & 1ull) {
          const int ci = __builtin_amdgcn_readlane(cnt, i);
          pair0 += __builtin_amdgcn_readlane(rank, i) < rank ? ci : 0;
          total += ci;
        }
      if (first_occ) {
        const int slot = n_shared_slots + rank;
        un.id[slot] = e;
        un.mask[slot] = mask;
        un.cnt[slot] = cnt;
        un.pair0[slot] = pair0;
#pragma unroll
        for (int m = 0; m < M; ++m) un.w[slot][m] = wsum[m];
      }
      if (lane == 0) {
        if (sh.has_shared) {
          un.id[0] = E;
          un.mask[0] = (1u << M) - 1u;
          un.cnt[0] = M;
          un.pair0[0] = 0;
#pragma unroll
          for (int m = 0; m < M; ++m) un.w[0][m] = 1.0f;
        }
        un.n = __popcll(firsts) + n_shared_slots;
        un.n_pairs = total;
      }
    }
    if (b == 0 && tid < M * K) {
      if (L.topk_idx) L.topk_idx[tid] = s_idx[tid / K][tid % K];
      if (L.topk_w) L.topk_w[tid] = s_w[tid / K][tid % K];
    }
    __syncthreads();
    stamp(w, l, 3);
    const int U = un.n;                 // slots incl. shared
    const int n_routed_slots = U - n_shared_slots;

    // ------------------------------------------------------------------ phase 3
    const int g8 = tid >> 3, j8 = tid & 7;
    const int n_dtasks = U * R0;   // down tasks of this workgroup: t = slot * R0 + local row
    // routed gate_up: act index q = b + G * jj over [0, n_routed_slots * I); group gi takes
    // jj = gi/2 + 16 * k, rows gate (gi even) / up (gi odd); two rows in flight per group
    {
      const int total = n_routed_slots * I;
      const int up = gi & 1;
      for (int k0 = 0;; k0 += 2) {
        const int jjA = (gi >> 1) + 16 * k0, jjB = jjA + 16;
        const int qA = b + G * jjA, qB = b + G * jjB;
        if (!__any(qA < total)) break;   // wave-uniform exit
        u32x4_t wa[kGuCpl], wb[kGuCpl];
        uint32_t sa[kGuCpl], sb[kGuCpl];
        const int uA = qA < total ? n_shared_slots + qA / I : 0, iA = qA < total ? qA % I : 0;
        const int uB = qB < total ? n_shared_slots + qB / I : 0, iB = qB < total ? qB % I : 0;
        {
          const size_t row = (size_t)un.id[uA] * gu_rows + (size_t)(iA + up * I);
          load_fp4_row16(L.gq + row * gu_row_bytes, L.gs + row * nch_h, j16, nch_h, qA < total, wa, sa);
        }
        {
          const size_t row = (size_t)un.id[uB] * gu_rows + (size_t)(iB + up * I);
          load_fp4_row16(L.gq + row * gu_row_bytes, L.gs + row * nch_h, j16, nch_h, qB < total, wb, sb);
        }
        float acc[M];
        dot_fp4_row16<M>(wa, sa, j16, nch_h, xs, H, un.mask[uA], acc);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float h = group_sum<16>(acc[m]);
          const float partner = __shfl_xor(h, 16, kWave);
          if (qA < total && !up && j16 == 0 && ((un.mask[uA] >> m) & 1u)) {
            const int p = un.pair0[uA] + __popc(un.mask[uA] & ((1u << m) - 1u));
            st_coherent(w.act + (size_t)p * I + iA, silu(h) * partner);
          }
        }
        dot_fp4_row16<M>(wb, sb, j16, nch_h, xs, H, un.mask[uB], acc);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float h = group_sum<16>(acc[m]);
          const float partner = __shfl_xor(h, 16, kWave);
          if (qB < total && !up && j16 == 0 && ((un.mask[uB] >> m) & 1u)) {
            const int p = un.pair0[uB] + __popc(un.mask[uB] & ((1u << m) - 1u));
            st_coherent(w.act + (size_t)p * I + iB, silu(h) * partner);
          }
        }
      }
    }
    stamp(w, l, 4);
    grid_sync(w, sync, l, 10);
    stamp(w, l, 5);

    // ------------------------------------------------------------------ phase 4
    // first batch of this workgroup's down rows: issued before the activations are staged so
    // the two latencies overlap
    u32x4_t dq0[2][kDnCpl];
    uint32_t ds0[2][kDnCpl];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = g8 + kGroups8 * k;
      const int u = t / R0, rl = t % R0;
      const bool ok = t < n_dtasks && rl < my_rows;
      const size_t row = ok ? (size_t)un.id[u] * H + row0 + rl : 0;
#pragma unroll
      for (int c4 = 0; c4 < kDnCpl; ++c4) {
        const int c = j8 + 8 * c4;
        if (ok && c < nch_i) {
          dq0[k][c4] = ld16(L.dq + row * dn_row_bytes + (size_t)c * 16);
          ds0[k][c4] = L.ds[row * nch_i + c];
        } else {
          dq0[k][c4] = u32x4_t{0, 0, 0, 0};
          ds0[k][c4] = 127;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the down loads above issued before the staging below
    {
      // the activation rows, 64-bit device-coherent loads in batches of 8 per thread (in flight
      // together), into LDS
      const int n_words = un.n_pairs * I / 2;
      const unsigned long long* src = reinterpret_cast<const unsigned long long*>(w.act);
      unsigned long long* dst = reinterpret_cast<unsigned long long*>(acts);
      for (int v0 = 0; v0 < n_words; v0 += 8 * kThreads) {
        unsigned long long t[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) t[q] = ld_coherent(src + min(v0 + q * kThreads + tid, n_words - 1));
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (v0 + q * kThreads + tid < n_words) dst[v0 + q * kThreads + tid] = t[q];
      }
    }
    __syncthreads();
    stamp(w, l, 6);
    for (int k0 = 0; k0 * kGroups8 < n_dtasks; k0 += 2) {
      u32x4_t dqb[2][kDnCpl];
      uint32_t dsb[2][kDnCpl];
      if (k0 == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int c4 = 0; c4 < kDnCpl; ++c4) {
            dqb[k][c4] = dq0[k][c4];
            dsb[k][c4] = ds0[k][c4];
          }
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int t = g8 + kGroups8 * (k0 + k);
          const int u = t / R0, rl = t % R0;
          const bool ok = t < n_dtasks && rl < my_rows;
          const size_t row = ok ? (size_t)un.id[u] * H + row0 + rl : 0;
#pragma unroll
          for (int c4 = 0; c4 < kDnCpl; ++c4) {
            const int c = j8 + 8 * c4;
            if (ok && c < nch_i) {
              dqb[k][c4] = ld16(L.dq + row * dn_row_bytes + (size_t)c * 16);
              dsb[k][c4] = L.ds[row * nch_i + c];
            } else {
              dqb[k][c4] = u32x4_t{0, 0, 0, 0};
              dsb[k][c4] = 127;
            }
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int t = g8 + kGroups8 * (k0 + k);
        const int u = t < n_dtasks ? t / R0 : 0, rl = t % R0;
        const bool ok = t < n_dtasks && rl < my_rows;
        const unsigned mask = ok ? un.mask[u] : 0u;
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
        for (int c4 = 0; c4 < kDnCpl; ++c4) {
          const int c = j8 + 8 * c4;
          if (c < nch_i) {
            const float sc = e8m0_to_f32(dsb[k][c4]);
            float wf[32];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const f32x2_t p0 = fp4x2_to_f32x2<0>(dqb[k][c4][d], sc), p1 = fp4x2_to_f32x2<1>(dqb[k][c4][d], sc);
              const f32x2_t p2 = fp4x2_to_f32x2<2>(dqb[k][c4][d], sc), p3 = fp4x2_to_f32x2<3>(dqb[k][c4][d], sc);
              wf[8 * d + 0] = p0.x; wf[8 * d + 1] = p0.y; wf[8 * d + 2] = p1.x; wf[8 * d + 3] = p1.y;
              wf[8 * d + 4] = p2.x; wf[8 * d + 5] = p2.y; wf[8 * d + 6] = p3.x; wf[8 * d + 7] = p3.y;
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
              if ((mask >> m) & 1u) {
                const int p = un.pair0[u] + __popc(mask & ((1u << m) - 1u));
                const float* ap = acts + (size_t)p * I + c * 32;
                float s = acc[m];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                  const float4 a4 = *reinterpret_cast<const float4*>(ap + q * 4);
                  s = fmaf(wf[4 * q + 0], a4.x, s);
                  s = fmaf(wf[4 * q + 1], a4.y, s);
                  s = fmaf(wf[4 * q + 2], a4.z, s);
                  s = fmaf(wf[4 * q + 3], a4.w, s);
                }
                acc[m] = s;
              }
            }
          }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float v = group_sum<8>(acc[m]);
          if (ok && j8 == 0 && ((mask >> m) & 1u)) red[((size_t)u * R0 + rl) * M + m] = un.w[u][m] * v;
        }
      }
    }
    __syncthreads();
    for (int p = tid; p < my_rows * M; p += kThreads) {
      const int rl = p / M, m = p % M;
      float s = 0.0f;
      for (int u = 0; u < U; ++u)
        if ((un.mask[u] >> m) & 1u) s += red[((size_t)u * R0 + rl) * M + m];
      const size_t o = (size_t)m * H + row0 + rl;
      if (L.y32) st_coherent(L.y32 + o, s);
      if (L.y16) st_coherent(L.y16 + o, f32_to_bf16_rne(s));
    }
    stamp(w, l, 7);
    if (l + 1 < n_layers) grid_sync(w, sync, l, 12);   // layer l's output is written before layer l+1 starts
  }
}

// ------------------------------------------------------------------------------ host side
int g_grid[64];       // workgroups per launch, per device (one per CU)
unsigned long long* g_trace[64];  // per device: trace buffer registered by qws_debug_trace_buffer
size_t g_trace_bytes[64];

size_t lds_bytes(int M, int K, int H, int I, int R0) {
  return (size_t)M * H * 2 + (size_t)M * (K + 1) * I * 4 + (size_t)kMaxSlots * R0 * M * 4;
}

size_t ws_layout(int M, int K, int E, int I, char* base, Work* w) {
  const size_t sync = qws_host::align256(kSyncCounters * kSyncStride * 8);
  const size_t err = 256;
  const size_t lg = qws_host::align256((size_t)M * E * 4);
  const size_t act = qws_host::align256((size_t)M * (K + 1) * I * 4);
  if (w) {
    w->trace = nullptr;
    w->sync = reinterpret_cast<unsigned long long*>(base);
    w->errors = reinterpret_cast<unsigned*>(base + sync);
    w->logits = reinterpret_cast<float*>(base + sync + err);
    w->act = reinterpret_cast<float*>(base + sync + err + lg);
  }
  return sync + err + lg + act;
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


int check_layer(const qws_moe_layer& d, int M, int E, int K, int H, int I, int has_shared) {
  if (!d.x_bf16 || !d.w_router_bf16 || (!d.y_bf16 && !d.y_f32)) return QWS_ERR_ARG;
  const qws_mxfp4_experts& x = d.experts;
  if (x.format != QWS_FMT_MXFP4_E2M1_E8M0_B32) return QWS_ERR_FORMAT;
  if (!x.gate_up_q || !x.gate_up_s || !x.down_q || !x.down_s) return QWS_ERR_ARG;
  if (x.n_routed != E || x.hidden != H || x.inter != I || x.has_shared != has_shared) return QWS_ERR_SHAPE;
  if (d.bias && !(d.bias_row_stride == 0 || d.bias_row_stride == E)) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(d.x_bf16) || !qws_host::aligned16(d.w_router_bf16) || !qws_host::aligned16(x.gate_up_q) ||
      !qws_host::aligned16(x.down_q))
    return QWS_ERR_ALIGN;
  (void)M;
  (void)K;
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
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 4096);
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
  const qws_mxfp4_experts& x0 = host[0].experts;
  const int E = x0.n_routed, H = x0.hidden, I = x0.inter, hs = x0.has_shared;
  if (M < 1 || M > kMaxM || K < 1 || K > kMaxK || E < K || E > kMaxE) return QWS_ERR_SHAPE;
  if (H < 32 || H > kHMax || H % 32 || I < 32 || I > kIMax || I % 32 || (hs != 0 && hs != 1)) return QWS_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    const int st = check_layer(host[l], M, E, K, H, I, hs);
    if (st != QWS_OK) return st;
  }
  if (!workspace || workspace_bytes < ws_layout(M, K, E, I, nullptr, nullptr)) return QWS_ERR_WORKSPACE;
  if (!qws_host::aligned16(workspace)) return QWS_ERR_ALIGN;
  int G = 0;
  int st = grid_for_device(&G);
  if (st != QWS_OK) return st;
  const int nrw = (E + G - 1) / G, nsp = (I + G - 1) / G;
  if (nrw > kWaves || 4 * nrw + 2 * nsp > kGroups16) return QWS_ERR_SHAPE;
  const int R0 = (H + G - 1) / G;
  const size_t lds = lds_bytes(M, K, H, I, R0);
  if (lds > 160 * 1024 - 4096) return QWS_ERR_SHAPE;
  Work w;
  ws_layout(M, K, E, I, static_cast<char*>(workspace), &w);
  {
    int dev = 0;
    (void)hipGetDevice(&dev);
    const size_t need = (size_t)n_layers * G * kTracePoints * 8;
    w.trace = (dev >= 0 && dev < 64 && g_trace[dev] && g_trace_bytes[dev] >= need) ? g_trace[dev] : nullptr;
  }
  const Shape sh{E, K, H, I, hs, R0};
  const Layer first = to_layer(host[0]);
  const qws_moe_layer* rest = dev_copy;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (M) {
    case 1: return launch<1>(first, rest, n_layers, sh, w, G, lds, s);
    case 2: return launch<2>(first, rest, n_layers, sh, w, G, lds, s);
    case 3: return launch<3>(first, rest, n_layers, sh, w, G, lds, s);
    default: return launch<4>(first, rest, n_layers, sh, w, G, lds, s);
  }
}

}  // namespace

extern "C" size_t moe_layer_workspace_bytes(int M, int K, int E, int hidden, int inter) {
  if (M < 1 || M > kMaxM || K < 1 || K > kMaxK || E < 1 || E > kMaxE || hidden < 32 || hidden > kHMax || inter < 32 ||
      inter > kIMax)
    return 0;
  return ws_layout(M, K, E, inter, nullptr, nullptr);
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
  Work w;
  ws_layout(M, K, E, inter, static_cast<char*>(const_cast<void*>(workspace)), &w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(errors_out, w.errors, sizeof(unsigned), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? QWS_OK : qws_host::set_device_error(e);
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
