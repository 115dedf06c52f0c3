// Fused MoE layer(s) on gfx950: router GEMV, top-K, softmax, expert union, MXFP4 gate_up + SwiGLU,
// MXFP4 down + gate-weighted combine with the shared expert -- one persistent launch for one or
// more layers (each layer routes eight of E routed experts plus one shared expert:
// runbyai.xyz/posts/593 paragraph 2; a window of M <= 4 tokens reads each activated expert once:
// paragraph 5).
//
// Why one launch: a kernel boundary costs ~1.7 us on MI355X even inside a HIP graph, about a third
// of a layer's streaming time at M = 1. The grid is one 1024-thread workgroup per compute unit,
// all resident at once.
//
// Work decomposition. A "task" is (slot u, block j): the 32 gate rows and 32 up rows of activation
// block j of expert id(u), plus the 32-column block j of that expert's down projection for all H
// output rows. One workgroup issues all of a task's loads in one burst (2 x 32 x H/2 gate/up bytes
// + H x 16 down bytes: 120 KB of codes at H = 2560), computes the block's 32 activations itself --
// activations never cross workgroups -- and writes H partial sums per token, already multiplied by
// the token's gate weight. Experts are stored task-major (moe_pack_mxfp4): a task is one 128 KB
// record in the order its 16 waves read it, so each of a lane's eight loads is part of a 1 KB
// run per wave. On MI355X one compute unit streams ~50 GB/s alone and ~27 GB/s while 192 stream
// at once, and many narrow or scattered loads per lane lower that further. Weights are read with
// non-temporal loads: each byte is used once per step, and a burst of such loads streams ~2x
// faster than cached loads when the caches hold dirty lines.
//
// Hand-offs between workgroups carry their own validity: a 64-bit word holds a 32-bit value and a
// 32-bit tag unique to (launch, layer, kind), written with one device-coherent store and polled
// with device-coherent loads (64-bit accesses are single-copy atomic), so a reader needs no
// separate signal, fence or counter; a poll reloads only the words that are not yet valid. Words
// that every workgroup polls are written in several copies (kReplicas). Per layer:
//   1  x into LDS: layer 0 from the caller's buffer; in a chained sequence (x of layer l+1 is y of
//      layer l) from the tagged copy of y the previous layer published.
//   2  router dots of this workgroup's rows (prefetched into LDS during the previous layer) ->
//      tagged logits; workgroups G-J .. G-1 then run the shared expert's J tasks (they need no
//      routing).
//   3  every workgroup selects top-K itself from the tagged logits, in parallel: a threshold from
//      lane-group maxima leaves a few candidates, ranked by the candidates that beat them (logit
//      descending, index ascending; with several tokens sorted within a wave); softmax over the
//      selected; union of the window's selections (first-occurrence order).
//   4  routed tasks, round-robin over workgroups (at M = 1 one task per workgroup).
//   5  workgroup b owns output rows [b*R, b*R + R): it polls their tagged partial sums, sums them in
//      a fixed order (deterministic), writes y and, in a chained sequence, a tagged copy.
// Layers that are not chained are separated instead by a barrier on tagged per-workgroup words.
#pragma once
#include "qws_common.hpp"
#ifdef __HIPCC_RTC__
#include "qws.h"   // the descriptor type (compiled at run time: qws_common.hpp includes it otherwise)
#endif
#ifndef offsetof
#define offsetof(t, m) __builtin_offsetof(t, m)
#endif

namespace qws_moe {

using namespace qws;

constexpr int kThreads = 1024;   // 16 waves: 4 per SIMD to hide the task's load and LDS latency
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxM = 4;
constexpr int kMaxK = 8;
constexpr int kMaxSlots = kMaxM * kMaxK + 1;    // routed union + shared
constexpr int kMaxPairs = kMaxM * (kMaxK + 1);  // (slot, token) pairs
constexpr int kMaxE = 1024;
constexpr int kHMax = 2560;
constexpr int kIMax = 1024;
constexpr int kBlk = 32;        // activations per task: one MX block of the down projection
constexpr int kGuCpl = 5;       // 16-byte chunks per lane of a gate or up row: H <= 16 * 5 * 32
constexpr int kRtCpl = 5;       // 16-byte chunks per lane of a router row: H <= 64 * 5 * 8
constexpr int kDnRpl = 3;       // down rows per thread in a task: H <= 1024 * 3
constexpr int kMaxRows = 16;    // output rows owned by one workgroup
constexpr int kMaxGrid = 512;
// Tagged partial-sum words per thread in flight while an owner reads its lines: one token's 216
// lines fit one batch of 4 (64 line groups x 4; 8 left half the slots empty and cost 0.12 us per
// layer, 2 or 3 take two batches, 0.2 us slower); several tokens' ~300 lines, one batch of 8.
template <int M>
constexpr int kPollBatch = M == 1 ? 4 : 8;
constexpr int kLine = 16;       // 64-bit words per 128-byte line: hand-off words of one writer share no line
                                // (the one-token logits aside)
static_assert(kMaxRows <= kLine, "an owner's rows of one (pair, block) share one line");
static_assert(kMaxM <= kLine, "an expert's logits of all tokens share one line");
// Words between the tagged logits of consecutive experts: one token packs 16 experts' logits into
// a line (each workgroup polls a sixteenth of the lines: 0.01-0.12 us per layer faster than a line
// per expert over three runs); several tokens keep an expert's logits in a line of their own
// (packing was 0.1 us per layer slower at M = 4).
template <int M>
constexpr int kLgStride = M == 1 ? 1 : kLine;
// Copies of the words every workgroup polls (the one-token logits, the layer-done words, the tagged
// y of a chained sequence): each is written kReplicas times by as many lanes of the same stores,
// and workgroup b polls copy b % kReplicas, so that a line is polled by a 32nd of the grid instead
// of all of it (logits and done words: 13.93 -> 13.68 us per layer at M = 1; 16 or 32 copies were
// slower again).
constexpr int kReplicas = 8;
static_assert(kReplicas <= kLine, "the one-token logit copies fit the logits area (kMaxE x kLine words)");
constexpr int kCopyWaves = kWaves - 2;   // waves that copy the next layer's x during the barrier
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
  const uint8_t* rec;   // task-major experts: record (e, j) at (e * I/32 + j) * kTaskBytes
  int* topk_idx;
  float* topk_w;
  float* logits_out;
  uint16_t* y16;
  float* y32;
};

__host__ __device__ Layer to_layer(const qws_moe_layer& d) {
  return Layer{static_cast<const uint16_t*>(d.x_bf16), static_cast<const uint16_t*>(d.w_router_bf16), d.bias,
               d.bias_row_stride, d.experts.gate_up_q, d.topk_idx, d.topk_w, d.logits_out, static_cast<uint16_t*>(d.y_bf16), d.y_f32};
}

struct Shape {
  int E, K, H, I, has_shared;
  int R;        // output rows per workgroup (even)
  int P;        // (slot, token) pairs the partial buffer holds per block: M * (K + 1)
  int chained;  // x of layer l+1 is y (bf16) of layer l, for every l
  int nrw;      // router rows per workgroup (one wave each)
  float inv_r;     // 1 / R: owner of a row = floor((row + 0.5) / R) without an integer division
  int y_stride;    // tagged y words per row owner (M * R / 2, padded to whole lines)
  int x_fresh;  // no layer's x is written by this launch: x of layer l+1 is fetched during layer l's barrier
  int jg;       // partial lines per routed pair (J / blocks per task group); set per layer
};

struct Work {
  unsigned long long* trace;     // NULL, or [n_layers][G][kTracePoints] wall-clock stamps (100 MHz)
  unsigned long long* sync;      // kSyncCounters monotonic counters, kSyncStride apart
  unsigned long long* launches;  // launch counter (each workgroup adds 1 per launch)
  unsigned* errors;              // count of launches' waits that timed out (only ever increases)
  unsigned long long* abort;     // launch number + 1 of the last launch one of whose waits timed out
  unsigned long long launch1;    // this launch's number + 1 (set in the kernel)
  float* act;                    // NULL, or the W4A8 activations of a one-layer launch (diagnostics):
                                 // a [E+1][M][I] fp32, then codes [E+1][M][I] u8, then scale bytes [E+1][M][I/32]
  // Hand-off buffers. Each 128-byte line of the partial sums, y and the done words is written by
  // one workgroup only: on MI355X an exchange among all workgroups takes ~1.8 us that way and ~3 us
  // when writers share lines (the 256 done words packed into 16 lines: 1.7 us per layer slower).
  // The one-token logits are the exception (16 routers' words per line; see kLgStride).
  unsigned long long* logits;    // tagged logits: expert e, token m at e * kLgStride<M> + m (one token:
                                 // copy r at r * kMaxE + e)
  unsigned long long* logits_odd;  // the same for the odd layers of a chained sequence (one token:
                                   // logits + kReplicas * kMaxE, inside the logits area)
  unsigned long long* ytag;      // [kMaxGrid][y_stride] tagged bf16 pairs of y (chained sequences), copy 0:
                                 // owner b, token m, pair q at b*y_stride + m*R/2 + q
  unsigned long long* ytag_more; // copies 1 .. kReplicas-1, [kReplicas-1][kMaxGrid][y_stride] (after the
                                 // partial sums: the other buffers keep their places)
  unsigned long long* done;      // [kReplicas][kMaxGrid][kLine] tagged "layer finished" words (layers that
                                 // are not chained): copy r of workgroup b's word at (r * kMaxGrid + b) * kLine
  unsigned long long* partial;   // [P * J][H] tagged, gate-weighted partial sums: line (pair, block or block group), row
};
// Copy c of the tagged y words of a chained sequence.
__device__ __forceinline__ unsigned long long* ytag_copy(const Work& w, const Shape& sh, int c) {
  return c == 0 ? w.ytag : w.ytag_more + (size_t)(c - 1) * kMaxGrid * sh.y_stride;
}


// Routing of the current layer, shared by the workgroup (LDS).
struct Union {
  int n;                         // slots: 0 = shared (if any), then routed ids in first-occurrence order
  int id[kMaxSlots];
  unsigned mask[kMaxSlots];      // tokens using the slot
  int pair0[kMaxSlots];          // first (slot, token) pair index of the slot
  float w[kMaxSlots][kMaxM];     // gate weight of (slot, token)
  int n_pairs;
  int ptok[kMaxPairs];           // token of each (slot, token) pair (M > 1)
  int sel_slot[kMaxM * kMaxK];   // slot of selection (token, rank) at token * kMaxK + rank (M > 1)
};

// Trace stamps go to LDS and reach memory in one store per layer, issued where the workgroup waits
// for its stores anyway: a store per stamp would put its acknowledgement into the next wait for a
// load and stretch the phase it marks. Stamps 8, 9 and 14 are taken after that store and leave with
// the next layer's (the last layer's at the end of the kernel).
__shared__ unsigned long long s_stamp[kTracePoints];
constexpr unsigned kLateStamps = (1u << 8) | (1u << 9) | (1u << 14);

__device__ __forceinline__ void stamp(const Work& w, int l, int k) {
  (void)l;
  if (w.trace && threadIdx.x == 0) s_stamp[k] = wall_clock64();
}
// Lanes 0 .. kTracePoints-1 of wave 0 (the wave that takes the stamps): layer l's early stamps and
// layer l-1's late ones (only the late ones when `late_only`); a slot is cleared once written.
__device__ __forceinline__ void flush_stamps(const Work& w, int l, bool late_only) {
  const int k = threadIdx.x;
  if (w.trace && k < kTracePoints) {
    const bool late = (kLateStamps >> k) & 1u;
    const int layer = late ? (late_only ? l : l - 1) : l;
    if ((late || !late_only) && layer >= 0) {
      w.trace[((size_t)layer * gridDim.x + blockIdx.x) * kTracePoints + k] = s_stamp[k];
      s_stamp[k] = 0ull;
    }
  }
}

__device__ __forceinline__ unsigned long long tagged(uint32_t tag, uint32_t v) {
  return ((unsigned long long)tag << 32) | (unsigned long long)v;
}
__device__ __forceinline__ uint32_t tag_of(unsigned long long v) { return (uint32_t)(v >> 32); }

// True once a wait of THIS launch has timed out (a timeout of an earlier launch does not count).
__device__ __forceinline__ bool gave_up(const Work& w) { return ld_coherent(w.abort) == w.launch1; }

// Poll count, error check and back-off of a bounded wait; returns true when the wait must end.
// Once a wait of this launch has timed out, every other wait of the launch ends at its next check;
// the next launch waits normally again.
__device__ __forceinline__ bool wait_expired(const Work& w, unsigned& spins) {
  if ((++spins & 255u) == 0) {
    const bool other = gave_up(w);
    if (other || spins > kSpinLimit) {
      if (!other && (threadIdx.x % kWave) == 0) {
        st_coherent(w.abort, w.launch1);
        atomicAdd(w.errors, 1u);
      }
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

// One wave copies a router row (H bf16) into LDS with 16-byte DMA loads.
__device__ __forceinline__ void router_row_to_lds(const uint16_t* row, uint16_t* dst, int H, int lane) {
  for (int c0 = 0; c0 < (H >> 3); c0 += kWave)
    if (c0 + lane < (H >> 3))
      __builtin_amdgcn_global_load_lds((const QWS_GLOBAL void*)(row + (c0 + lane) * 8),
                                       (__attribute__((address_space(3))) void*)(dst + c0 * 8), 16, 0, 0);
}

// The barrier's wait: every workgroup's tagged word, kPer words per lane of one wave. The wait
// re-checks every slot each round, so kPer matches the grid (4 for G <= 256: 16 slots, sized for the
// largest grid, made each layer 0.09 us slower at M = 1 and 0.23 us at M = 4).
template <int kPer>
__device__ __forceinline__ void poll_done(const Work& w, const unsigned long long* src, int lane, uint32_t tag) {
  int idx[kPer];
  unsigned long long v[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) idx[q] = lane + q * kWave < (int)gridDim.x ? (lane + q * kWave) * kLine : -1;
  poll_tagged<kPer>(w, src, idx, tag, v);
}

// Between layers that are not chained: every workgroup publishes a tagged word once all of its
// stores have been acknowledged, then waits for every workgroup's word. No atomics, so no
// round trip to a counter before the wait starts. Meanwhile waves 0 .. kCopyWaves-1 copy the next
// layer's x into LDS, wave kWaves-2 stores the word and the last wave polls: neither issues any of
// the copies, which a wait for its loads would also wait for.
__device__ void tagged_barrier(const Work& w, uint32_t tag, int tid, int l, const uint16_t* next_x, uint16_t* xs,
                               int n_x) {
  wait_mem();
  __syncthreads();
  stamp(w, l, 14);
  // the word is stored by a wave that neither copies nor polls: the next wait of the storing wave
  // also waits for the store's acknowledgement, slow while every workgroup polls these lines
  if (const int r = tid - (kWaves - 2) * kWave; r >= 0 && r < kReplicas)
    st_coherent(w.done + ((size_t)r * kMaxGrid + blockIdx.x) * kLine, tagged(tag, 0u));
  if (next_x && tid < kCopyWaves * kWave) {
    // the next layer's x (written before this launch) -> LDS, in flight while the barrier waits
    const int lane = tid % kWave, c0 = tid - lane;
    for (int c = c0; c < n_x / 8; c += kCopyWaves * kWave)
      if (c + lane < n_x / 8)
        __builtin_amdgcn_global_load_lds((const QWS_GLOBAL void*)(next_x + (size_t)(c + lane) * 8),
                                         (__attribute__((address_space(3))) void*)(xs + (size_t)c * 8), 16, 0, 0);
  }
  if (tid >= kThreads - kWave) {
    const int lane = tid - (kThreads - kWave);
    const unsigned long long* src = w.done + (size_t)(blockIdx.x % kReplicas) * kMaxGrid * kLine;
    if (gridDim.x <= 4 * kWave) poll_done<4>(w, src, lane, tag);
    else poll_done<kMaxGrid / kWave>(w, src, lane, tag);
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------ FP8 activations
// The gate/up products run on the scaled matrix instruction with FP4 weights (A) and FP8
// activations (B): v_mfma_scale_f32_16x16x128_f8f6f4 takes 128 k per op in four blocks of 32, each
// with one E8M0 scale per row of A and per column of B. Measured operand layout on gfx950: lane
// (g, i) = (lane / 16, lane % 16) supplies block g of A row i as 16 bytes (element 2j in the low
// nibble of byte j: an MX chunk as stored) and A's scale byte for it; B column i's block b comes
// from lane groups 2 (b % 2) (elements 0 .. 15 of the block) and 2 (b % 2) + 1 (16 .. 31), in
// dwords 4 (b / 2) .. +3 of the lane's eight, and B's scale for block b from lane group b; D is as
// for the bf16 op (lane (g, i): rows 4g .. 4g+3 of column i).
typedef int i32x8_t __attribute__((ext_vector_type(8)));
template <int OPSEL_A>
__device__ __forceinline__ f32x4_t mfma_fp4_fp8(u32x4_t a, u32x4_t b_lo, u32x4_t b_hi, uint32_t scale_a,
                                                uint32_t scale_b, f32x4_t c) {
  // an FP4 operand is the low four registers of the tuple; the op never reads the high four
  const int u = __builtin_nondeterministic_value(0);
  const i32x8_t av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], u, u, u, u};
  const i32x8_t bv = {(int)b_lo[0], (int)b_lo[1], (int)b_lo[2], (int)b_lo[3],
                      (int)b_hi[0], (int)b_hi[1], (int)b_hi[2], (int)b_hi[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4 /* A: FP4 e2m1 */, 0 /* B: FP8 e4m3 */,
                                                          OPSEL_A, (int)scale_a, 0, (int)scale_b);
}

// The same instruction with the formats swapped: A FP8 (rows in the B layout above: row i, block
// b from lane groups 2 (b % 2) and 2 (b % 2) + 1, dwords 4 (b / 2) .. +3), B FP4 (column n, block
// b: lane (b, n), 16 bytes); the scale of A row i block b in lane (b, i), of B column n block b in
// lane (b, n) (measured on gfx950 with random operands).
__device__ __forceinline__ f32x4_t mfma_fp8_fp4(u32x4_t a_lo, u32x4_t a_hi, u32x4_t b, uint32_t scale_a,
                                                uint32_t scale_b, f32x4_t c) {
  const int u = __builtin_nondeterministic_value(0);
  const i32x8_t av = {(int)a_lo[0], (int)a_lo[1], (int)a_lo[2], (int)a_lo[3],
                      (int)a_hi[0], (int)a_hi[1], (int)a_hi[2], (int)a_hi[3]};
  const i32x8_t bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], u, u, u, u};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0 /* A: FP8 e4m3 */, 4 /* B: FP4 e2m1 */,
                                                          0, (int)scale_a, 0, (int)scale_b);
}

// A matrix instruction takes its operands from every lane of the wave, so it must run with all
// lanes enabled. When its result is used only under a lane condition (a store by some lanes), the
// compiler sinks the scaled instruction into that branch, where the disabled lanes supply no
// operands (observed: only the rows of the enabled lanes came out right). An empty asm statement
// that takes the result in place keeps the instruction where it is written.
__device__ __forceinline__ void mfma_result(f32x4_t& d) { asm volatile("" : "+v"(d)); }

// x (bf16, LDS) -> two E4M3 parts per element for the B operand, written to x8 [2M][H] (row 2m + s
// = part s of token m) with one E8M0 scale per (row, 32-element block) in xs8 [2M][H/32]. Part 0
// keeps the top four significant bits of x (the bf16 value with its low four fraction bits
// cleared), part 1 the low four (exactly x minus part 0). With e the largest bf16 exponent field
// of the block, part 0 is scaled by 2^(e-134) and part 1 by 2^(e-138) (scale bytes e - 7 and
// e - 11): both then lie within +-240 and, for every element whose exponent is within 13 of e, are
// E4M3 values exactly, so x = part 0 + part 1 enters the products exactly; smaller elements are
// rounded to nearest even at 2^-9 of their part's scale (at most 2^-16 of the block's largest
// magnitude). Threads t0 .. kThreads-1 take part: 8 lanes per block, 4 elements per lane (one
// 8-byte read, the block maximum by three lane swaps, two 4-byte writes).
__device__ __forceinline__ void stage_x8(const uint16_t* xs, uint8_t* x8, uint8_t* xs8, int M, int H, int tid, int t0) {
  const int nch = H >> 5, j = tid & 7;
  for (int u = (tid - t0) >> 3; u < M * nch; u += (kThreads - t0) >> 3) {
    const int m = u / nch, c = u - m * nch;
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(xs + (size_t)m * H + 32 * c + 4 * j);
    const uint32_t b0 = v[0] & 0xffffu, b1 = v[0] >> 16, b2 = v[1] & 0xffffu, b3 = v[1] >> 16;
    uint32_t e = max(max((b0 >> 7) & 0xffu, (b1 >> 7) & 0xffu), max((b2 >> 7) & 0xffu, (b3 >> 7) & 0xffu));
    e = max(e, dpp<0xB1>(e));    // lanes 8k .. 8k+7 share the block: quad swaps, then the half-row mirror
    e = max(e, dpp<0x4E>(e));
    e = max(e, dpp<0x141>(e));
    const int sh = min(max((int)e - 7, 1), 253), sl = min(max((int)e - 11, 1), 253);
    const float fh = __uint_as_float((uint32_t)(254 - sh) << 23), fl = __uint_as_float((uint32_t)(254 - sl) << 23);
    float hi[4], lo[4];
    const uint32_t bb[4] = {b0, b1, b2, b3};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float h = bf16_bits_to_f32(bb[q] & 0xfff0u);
      hi[q] = h * fh;                               // part 0 / 2^(sh - 127)
      lo[q] = (bf16_bits_to_f32(bb[q]) - h) * fl;   // part 1 / 2^(sl - 127)
    }
    const uint32_t ch = f32x2_to_e4m3x2<true>(hi[2], hi[3], f32x2_to_e4m3x2<false>(hi[0], hi[1], 0u));
    const uint32_t cl = f32x2_to_e4m3x2<true>(lo[2], lo[3], f32x2_to_e4m3x2<false>(lo[0], lo[1], 0u));
    *reinterpret_cast<uint32_t*>(x8 + (size_t)(2 * m) * H + 32 * c + 4 * j) = ch;
    *reinterpret_cast<uint32_t*>(x8 + (size_t)(2 * m + 1) * H + 32 * c + 4 * j) = cl;
    if (j == 0) {
      xs8[2 * m * nch + c] = (uint8_t)sh;
      xs8[(2 * m + 1) * nch + c] = (uint8_t)sl;
    }
  }
}

// x (bf16, LDS) -> MXFP8 for the W4A8 layer: E4M3 codes in x8 [M][H] (row m = token m) and one
// E8M0 scale per (token, 32-element block) in xs8 [M][H/32], by the OCP MX conversion: with e the
// largest bf16 exponent field of the block, the scale is 2^(e - 127 - 8) (byte e - 8, at least 0:
// the smallest E8M0 scale), and each element is x / scale (exact: a power of two) rounded to the
// nearest E4M3 value, ties to even, magnitudes past 448 clamped to it. Threads t0 .. kThreads-1
// take part: 8 lanes per block, 4 elements per lane.
__device__ __forceinline__ void stage_x8_mx(const uint16_t* xs, uint8_t* x8, uint8_t* xs8, int M, int H, int tid,
                                            int t0) {
  const int nch = H >> 5, j = tid & 7;
  for (int u = (tid - t0) >> 3; u < M * nch; u += (kThreads - t0) >> 3) {
    const int m = u / nch, c = u - m * nch;
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(xs + (size_t)m * H + 32 * c + 4 * j);
    const uint32_t b0 = v[0] & 0xffffu, b1 = v[0] >> 16, b2 = v[1] & 0xffffu, b3 = v[1] >> 16;
    uint32_t e = max(max((b0 >> 7) & 0xffu, (b1 >> 7) & 0xffu), max((b2 >> 7) & 0xffu, (b3 >> 7) & 0xffu));
    e = max(e, dpp<0xB1>(e));
    e = max(e, dpp<0x4E>(e));
    e = max(e, dpp<0x141>(e));
    const uint32_t sb = e >= 8u ? e - 8u : 0u;
    const float inv = __uint_as_float((254u - sb) << 23);   // 2^(127 - sb): exact, normal for sb <= 246
    const uint32_t code = f32x2_to_e4m3x2<true>(bf16_bits_to_f32(b2) * inv, bf16_bits_to_f32(b3) * inv,
                                                f32x2_to_e4m3x2<false>(bf16_bits_to_f32(b0) * inv,
                                                                       bf16_bits_to_f32(b1) * inv, 0u));
    *reinterpret_cast<uint32_t*>(x8 + (size_t)m * H + 32 * c + 4 * j) = code;
    if (j == 0) xs8[m * nch + c] = (uint8_t)sb;
  }
}

// Non-temporal 16-byte load of weights that are read once per step.
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const QWS_GLOBAL u32x4_t*)p);
}
__device__ __forceinline__ uint32_t ld4_stream(const void* p) {
  return __builtin_nontemporal_load((const QWS_GLOBAL uint32_t*)p);
}
__device__ __forceinline__ uint32_t ldb_stream(const uint8_t* p) {
  return __builtin_nontemporal_load((const QWS_GLOBAL uint8_t*)p);
}

// ------------------------------------------------------------------------------ tasks
// A task is (expert e, block j): gate rows 32j .. 32j+31 and up rows I+32j .. I+32j+31 of expert
// e, whose SwiGLU gives activations 32j .. 32j+31, then the H x 32 slice of the down projection
// that multiplies them. Both products run on the matrix cores (MFMA 16x16x32, bf16 operands
// dequantised exactly from e2m1 x E8M0, fp32 accumulation), with the tokens as the MFMA's 16
// columns. Gate/up: wave w takes row group rg = w / 4 (16 rows: gate 0-15, gate 16-31, up 0-15,
// up 16-31 of the block) and k-slice ks = w % 4 (chunks 20ks .. 20ks+19 of those rows; a chunk is
// 16 bytes = 32 codes = one MX block); MFMA lane (g, i) = (lane / 16, lane % 16) supplies row i at
// k-group g, i.e. chunk 20ks + 4t + g for t < 5. Down: wave w takes the 16-row tiles w + 16q
// (q < 10) of the block; lane (g, i) supplies word g (codes 8g .. 8g+7) of tile row i. The
// task-major record (moe_pack_mxfp4) holds exactly these operands, lane by lane, in eight 16-byte
// pieces per lane; the first carries the scales, so the first gate/up chunk waits for two loads.
constexpr int kGuCpk = 4 * kGuCpl;            // chunks of a row per k-slice: H <= 4 * 20 * 32
constexpr int kDnTpw = kHMax / 16 / kWaves;   // down-projection row tiles (16 rows) per wave
constexpr int kPieces = 8;                    // 16-byte pieces per lane of a task record
// a lane's down sums kept across a task group: 3 ops x up to 4 tokens (W4A8) or up to 3 x 4 ops
template <bool A8>
constexpr int kOutv = 12;
// At M = 1 the shared expert's J tasks run before selection on the last J workgroups (the routed
// tasks leave them idle). With more tokens the union needs most workgroups for several tasks, so
// the shared expert joins the grouped task pool after selection instead.
template <int M>
constexpr bool kEarlyShared = M == 1;
constexpr int kTaskBytes = kPieces * kThreads * 16;
static_assert(kTaskBytes == QWS_TASK_BYTES, "task record size");
static_assert(kGuCpl == 5 && kDnTpw == 10, "piece layout: 5 gate/up chunks + 10 down words + scales per lane");
struct TaskRegs {
  u32x4_t p[kPieces];   // piece 0: down words q 8, 9 + scales; 1-5: gate/up chunks t; 6, 7: down words q 0..7
};

// This thread's first byte in the record of task (expert e, block j).
__device__ __forceinline__ const uint8_t* task_rec(const Layer& L, const Shape& sh, int e, int j, unsigned tid) {
  return L.rec + ((size_t)e * (sh.I / kBlk) + j) * kTaskBytes + (size_t)tid * 16;
}
// Issues the loads of pieces P0 .. P1-1 of a task record into registers: for each piece, the 64
// lanes of a wave read 1 KB of consecutive bytes. All task loads are plain vector loads: vector
// memory operations of one kind complete in order, so the compute can wait for each gate/up chunk
// alone (an LDS DMA among them would be another kind, and the compiler then waits for all of them
// before the first use).
template <int P0, int P1>
__device__ __forceinline__ void task_load(const uint8_t* rec, TaskRegs& r) {
#pragma unroll
  for (int q = P0; q < P1; ++q) r.p[q] = ld16_stream(rec + (size_t)q * kThreads * 16);
}

// Computes task (slot u: tokens in `mask` (un.mask[u]), pairs un.pair0[u] + rank, gate weights un.w[u][m],
// block j) from its loaded registers, and stores
// partial[p][j][row] = w * sum_k W_down[row][32j+k] * a[k] for every row, tagged, at the row's
// offset in its owner's region. gu_s (LDS: 4 x M x 64 floats, then the activations) takes the
// k-slice sums of gate/up and the activations: M x 4 x 32 bf16 parts, or for the W4A8 layer (A8)
// M x 32 E4M3 codes and M scale bytes.
template <int M, bool A8>
__device__ __forceinline__ void task_compute(const Shape& sh, const Work& w, TaskRegs& r, const Union& un,
                                             int u, unsigned mask, const uint8_t* x8, const uint8_t* xs8, float* gu_s,
                                             unsigned tid, uint32_t tag, const uint8_t* nrec, int line_shared,
                                             int line_routed, bool first, bool last, float (&outv)[kOutv<A8>],
                                             int jblk) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & (kWave - 1);
  const int g = lane >> 4, i = lane & 15, rg = wave >> 2, ks = wave & 3;
  const int H = sh.H, nch = H >> 5, J = sh.I / kBlk, R = sh.R;
  (void)R;
  // gate/up: FP4 weights x FP8 activations, one scaled op per piece (4 chunks = 128 k). B column i
  // is x8 row i, read from LDS by the lanes of this slot's tokens only; other columns are zero. The
  // bf16 layer stages x as two parts per token (row i = part i % 2 of token i / 2), the W4A8 layer
  // as one (row i = token i).
  constexpr int kRows = A8 ? M : 2 * M;
  const bool xcol = i < kRows && (M == 1 || ((mask >> (A8 ? i : i >> 1)) & 1u));
  const uint8_t* xrow = x8 + (size_t)min(i, kRows - 1) * H;
  const uint8_t* srow = xs8 + min(i, kRows - 1) * nch;
  f32x4_t d0 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int t = 0; t < kGuCpl; ++t) {
    // chunks past the row end are zero in the record (codes and scales): they add zeros
    const int cb = kGuCpk * ks + 4 * t;
    u32x4_t blo = {0u, 0u, 0u, 0u}, bhi = blo;
    uint32_t bsc = 127u;
    if (xcol) {
      blo = *reinterpret_cast<const u32x4_t*>(xrow + 32 * min(cb + (g >> 1), nch - 1) + 16 * (g & 1));
      bhi = *reinterpret_cast<const u32x4_t*>(xrow + 32 * min(cb + 2 + (g >> 1), nch - 1) + 16 * (g & 1));
      bsc = srow[min(cb + g, nch - 1)];
    }
    const uint32_t asc = t < 4 ? (r.p[0][2] >> (8 * t)) & 0xffu : r.p[0][3] & 0xffu;   // this lane's chunk scale
    d0 = mfma_fp4_fp8<0>(r.p[1 + t], blo, bhi, asc, bsc, d0);
  }
  mfma_result(d0);
  f32x4_t dsum = d0;
  if constexpr (!A8) {
    // the two parts of token m are columns 2m and 2m + 1: adjacent lanes
    // (four scalar swaps: the same swap written on the vector's elements in a loop was compiled into
    // one swap of element 0 added to every element)
    const float s0 = d0[0], s1 = d0[1], s2 = d0[2], s3 = d0[3];
    const float t0 = __uint_as_float(dpp<0xB1>(__float_as_uint(s0))), t1 = __uint_as_float(dpp<0xB1>(__float_as_uint(s1)));
    const float t2 = __uint_as_float(dpp<0xB1>(__float_as_uint(s2))), t3 = __uint_as_float(dpp<0xB1>(__float_as_uint(s3)));
    dsum = f32x4_t{s0 + t0, s1 + t1, s2 + t2, s3 + t3};
  }
  if (w.trace && tid == 0) {
    // trace only: every piece of this thread's record has arrived (waits for them here, in wave 0)
    __builtin_amdgcn_s_waitcnt(0);
    s_stamp[15] = wall_clock64();
  }
  // lane (g, 2m) (bf16 layer) or (g, m) (W4A8) holds rows 4g .. 4g+3 of the row group for token m
  if (A8 ? i < M : ((i & 1) == 0 && (i >> 1) < M))
    *reinterpret_cast<f32x4_t*>(gu_s + (ks * M + (A8 ? i : i >> 1)) * 64 + rg * 16 + 4 * g) = dsum;
  // the next task's (nrec) gate/up pieces load into these registers during this task's down
  // projection, its down pieces after it; the down-phase words of piece 0 are kept first
  const uint32_t dn8 = r.p[0][0], dn9 = r.p[0][1], dsw = r.p[0][3];
  if (nrec) task_load<0, kPieces - 2>(nrec, r);
  __syncthreads();

  const int n = lane & 15;
  constexpr int MP = M == 1 ? 1 : (M == 2 ? 2 : 4);   // M rounded up to a power of two
  // partial line of (pair pm, this task's block or block group): at M = 1 the shared slot's pairs
  // (run early) come first with one line per block, then the other pairs with one line per group
  // (a line is one row-contiguous vector of H tagged words: a store of 16 rows fills a 128-byte
  // line of memory, and a row owner reads its R consecutive words of every line)
  const int nsm = kEarlyShared<M> && sh.has_shared ? M : 0;
  const int ntile = H >> 4;
  // The activations of the slot's tokens go to LDS as E4M3 codes with E8M0 scales per (token,
  // part): one part (W4A8: the MXFP8 value), or four parts whose sum is the float32 activation to
  // ~2^-16 of the block's largest (each part the next four significant bits, truncated, the last
  // rounded; scale byte e - 7 - 4p for the block's largest exponent field e: parts of every
  // activation within 2^13 of the largest are E4M3 values exactly). Lanes 32m .. 32m+31 hold
  // token m's 32 activations.
  constexpr int NP = A8 ? 1 : 4;
  uint8_t* a8 = reinterpret_cast<uint8_t*>(gu_s + 4 * M * 64);   // [M][NP][32] codes, then [M][NP] scale bytes
  constexpr int kScaleAt = M * NP * 32;   // M * 132 bytes in all, within the M * 256 the layout reserves
  if (tid < 32 * M) {
    const int am = tid >> 5, k = tid & 31;
    const float* gp = gu_s + am * 64 + k;
    float gate = gp[0], up = gp[32];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      gate += gp[q * M * 64];
      up += gp[q * M * 64 + 32];
    }
    const bool in = M == 1 || ((mask >> am) & 1u);
    const float av = in ? silu(gate) * up : 0.0f;
    uint32_t e = (__float_as_uint(av) >> 23) & 0xffu;
    e = max(e, dpp<0xB1>(e));    // lanes 8k .. 8k+7
    e = max(e, dpp<0x4E>(e));
    e = max(e, dpp<0x141>(e));
    e = max(e, dpp<0x140>(e));   // row mirror: lanes 16k .. 16k+15
    const auto pr = __builtin_amdgcn_permlane16_swap(e, e, false, false);   // rows 2k and 2k+1
    e = max(pr[0], pr[1]);
    float rem = av;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      // W4A8: 2^(e - 127 - 8), the OCP MX scale; parts: 2^(e - 127 - 7 - 4p)
      const uint32_t sb = A8 ? (e >= 8u ? e - 8u : 0u) : (e >= 7u + 4u * p ? e - 7u - 4u * p : 0u);
      float part = rem;
      if (p + 1 < NP) {
        part = __uint_as_float(__float_as_uint(rem) & 0xfff00000u);   // the top four significant bits
        rem -= part;                                                   // exact
      }
      const float inv = __uint_as_float((254u - sb) << 23);   // 2^(127 - sb): exact, normal for sb <= 247
      const uint8_t code = (uint8_t)(f32x2_to_e4m3x2<false>(part * inv, 0.0f, 0u) & 0xffu);
      a8[(am * NP + p) * 32 + k] = code;
      if (k == 0) a8[kScaleAt + am * NP + p] = (uint8_t)sb;
      if (A8 && w.act && in) {
        // diagnostics: this token's activation, code and scale of expert un.id[u], block jblk
        const size_t na = (size_t)(sh.E + 1) * M * sh.I, at = ((size_t)un.id[u] * M + am) * sh.I + kBlk * jblk + k;
        w.act[at] = av;
        reinterpret_cast<uint8_t*>(w.act + na)[at] = code;
        if (k == 0) reinterpret_cast<uint8_t*>(w.act + na)[na + at / kBlk] = (uint8_t)sb;
      }
    }
  }
  __syncthreads();

  // down on the scaled instruction: activations as A (FP8), weights as B (FP4), 64 output rows
  // per op. B block b = row n of tile 4Q + b of this wave's tiles w + 16 q, exactly as the record
  // holds it (Q = 0, 1: pieces 6 and 7; Q = 2: tiles 8 and 9, whose second halves come from lane
  // groups 2 and 3 by one lane-group swap), its scale the lane's byte 13 + Q of piece 0. A row i
  // holds one (tile slot, token, part)'s 32 codes in that tile slot's block and zeros elsewhere,
  // so D row i, column n is that tile row for that token and part.
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const uint32_t sw8 = __builtin_amdgcn_permlane32_swap(dn8, dn8, false, false)[1];
  const uint32_t sw9 = __builtin_amdgcn_permlane32_swap(dn9, dn9, false, false)[1];
  const u32x4_t wq[3] = {r.p[6], r.p[7], u32x4_t{dn8, dn9, sw8, sw9}};
  if constexpr (A8) {
    // A row 4 bq + c: token c's codes in block bq (T = 4 tiles per op, all tokens in one op);
    // lane (g, n) register c of D is token c's sum for row n of tile 4Q + g
    const int ca = n & 3, ba = n >> 2;
    const bool toka = ca < M && (M == 1 || ((mask >> ca) & 1u));
    const u32x4_t av16 = toka ? *reinterpret_cast<const u32x4_t*>(a8 + min(ca, M - 1) * 32 + 16 * (g & 1)) : zero;
    const u32x4_t alo = ba == (g >> 1) ? av16 : zero, ahi = ba == 2 + (g >> 1) ? av16 : zero;
    const uint32_t asc = a8[kScaleAt + min(ca, M - 1)];
    unsigned long long* pdst[M];
    float wt[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int pm = un.pair0[u] + __popc(mask & ((1u << m) - 1u));
      pdst[m] = w.partial + (size_t)(pm < nsm ? pm * J + line_shared : line_routed + (pm - nsm) * sh.jg) * H;
      wt[m] = un.w[u][m];
    }
#pragma unroll
    for (int Q = 0; Q < 3; ++Q) {
      f32x4_t dd = mfma_fp8_fp4(alo, ahi, wq[Q], asc, (dsw >> (8 + 8 * Q)) & 0xffu, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
      mfma_result(dd);
#pragma unroll
      for (int m = 0; m < M; ++m) outv[Q * M + m] = first ? dd[m] : outv[Q * M + m] + dd[m];
    }
    // the stores after every product: a use of the record's registers after a store would make the
    // compiler wait for the store's acknowledgement too (vector memory counts both)
    if (last) {
#pragma unroll
      for (int Q = 0; Q < 3; ++Q) {
        const int rt = wave + kWaves * (4 * Q + g);
#pragma unroll
        for (int m = 0; m < M; ++m)
          if ((M == 1 || ((mask >> m) & 1u)) && 4 * Q + g < kDnTpw && rt < ntile)
            st_coherent(pdst[m] + rt * 16 + n, tagged(tag, __float_as_uint(wt[m] * outv[Q * M + m])));
      }
    }
  } else {
    // A row i = (tile slot i / (4 MP), token (i / 4) % MP, part i % 4): T = 4 / MP tiles per op, MP
    // ops per group of four tiles. Lane (g, n) of D holds the four parts of (tile slot g / MP,
    // token g % MP) for row n: their sum is that token's partial for the row.
    constexpr int T = 4 / MP;
    const int bl = n / (4 * MP), ma = (n >> 2) % MP, pa = n & 3;
    const bool toka = ma < M && (M == 1 || ((mask >> ma) & 1u));
    const u32x4_t av16 =
        toka ? *reinterpret_cast<const u32x4_t*>(a8 + (min(ma, M - 1) * NP + pa) * 32 + 16 * (g & 1)) : zero;
    const uint32_t asc = a8[kScaleAt + min(ma, M - 1) * NP + pa];
    const int mg = g % MP, bg = g / MP;
    const bool tokg = mg < M && (M == 1 || ((mask >> mg) & 1u));
    const float wt = un.w[u][min(mg, M - 1)];
    const int pm = un.pair0[u] + __popc(mask & ((1u << mg) - 1u));
    unsigned long long* pdst =
        w.partial + (size_t)(pm < nsm ? pm * J + line_shared : line_routed + (pm - nsm) * sh.jg) * H;
#pragma unroll
    for (int Q = 0; Q < 3; ++Q)
#pragma unroll
      for (int o = 0; o < MP; ++o) {
        if (Q == 2 && T * o >= 2) continue;   // tiles 10, 11 do not exist
        const int blk = T * o + bl;            // this A row's block
        const u32x4_t alo = blk == (g >> 1) ? av16 : zero, ahi = blk == 2 + (g >> 1) ? av16 : zero;
        f32x4_t dd = mfma_fp8_fp4(alo, ahi, wq[Q], asc, (dsw >> (8 + 8 * Q)) & 0xffu, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f});
        mfma_result(dd);
        const float v = (dd[0] + dd[1]) + (dd[2] + dd[3]);
        // a workgroup's tasks of one group (same slot, consecutive blocks) add up in registers and
        // store once, after the last
        outv[Q * MP + o] = first ? v : outv[Q * MP + o] + v;
      }
    // the stores after every product (see above)
    if (last) {
#pragma unroll
      for (int Q = 0; Q < 3; ++Q)
#pragma unroll
        for (int o = 0; o < MP; ++o) {
          if (Q == 2 && T * o >= 2) continue;
          const int qt = 4 * Q + T * o + bg, rt = wave + kWaves * qt;
          if (tokg && qt < kDnTpw && rt < ntile)
            st_coherent(pdst + rt * 16 + n, tagged(tag, __float_as_uint(wt * outv[Q * MP + o])));
        }
    }
  }
  if (nrec) task_load<kPieces - 2, kPieces>(nrec, r);
  __syncthreads();  // gu_s is rewritten by the next task
}

// ------------------------------------------------------------------------------ top-K + union
// Every workgroup selects the top-K of each token from the tagged logits (the same result in every
// workgroup). A lane holds experts lane + 64 q. A candidate must reach T = the smallest of the
// maxima of the 8 lane groups (lanes 8g .. 8g+7) when at least K groups hold experts (then >= K
// logits reach T, so all of the top K do); otherwise T admits every expert. Candidates are ordered
// by the key (logit desc, index asc) and the first K are the selection, in order: a candidate's
// rank is the number of candidates that beat it, counted by all waves with one ballot per 64 of
// them (one token), or, with several tokens, each token's candidates (~19, p99 48) are sorted by
// one bitonic sort across the wave that found them when they fit in it. (A wave's sort is a chain
// of 10-21 dependent compare-exchange stages; with one token the 16 waves' ballots finish
// ~0.2 us sooner, with four tokens the four waves' sorts ~0.3 us sooner than ranking them all.)

// One token: wave 0 polls the logits (fewer polling waves make the exchange faster), finds T and
// writes the candidates to LDS in (q, lane) order with straight-line code; then every wave ranks
// its share of the candidates (one ballot per 64 of them) and enters the selected ones into the
// union (the shared expert, then the selection in rank order). The gate weights come last, from
// wave 0 after the final barrier: a task reads them only after its own first barrier, so the other
// waves issue their task loads meanwhile.
template <int kQ>
__device__ __forceinline__ void select_top_one(const Shape& sh, const Work& w, const unsigned long long* lgs,
                                               uint32_t tag, int wave, int lane,
                                               unsigned long long* cand, Union& un, int (*s_idx)[kMaxK],
                                               float (*s_w)[kMaxK], uint32_t (*s_sel)[kMaxK], int l) {
  const int E = sh.E, K = sh.K;
  const int ns = sh.has_shared ? 1 : 0;
  // LDS: candidates [0, nc), then one slot per lane for the lanes without one, then the count
  unsigned long long* const n_slot = cand + E + kWave;
  if (wave == 0) {
    const unsigned long long lt = (1ull << lane) - 1ull;
    int idx[kQ];
    unsigned long long v[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int e = lane + kWave * q;
      idx[q] = e < E ? e * kLgStride<1> : -1;
    }
    poll_tagged<kQ>(w, lgs + (size_t)(blockIdx.x % kReplicas) * kMaxE, idx, tag, v);
    stamp(w, l, 4);
    // absent experts (past E) get key 0 by a mask rather than a branch per q
    uint32_t key[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      key[q] = sel_key(__uint_as_float((uint32_t)v[q])) & (0u - (uint32_t)(lane + kWave * q < E));
    // T: group maxima (quad swaps, half-row mirror), then their minimum by lane moves (groups 8
    // lanes apart within a row, then across rows and half-waves). A group without experts has
    // maximum 0, which admits every expert; T >= 1 keeps absent ones out.
    uint32_t lm = key[0];
#pragma unroll
    for (int q = 1; q < kQ; ++q) lm = max(lm, key[q]);
    lm = max(lm, dpp<0xB1>(lm));
    lm = max(lm, dpp<0x4E>(lm));
    lm = max(lm, dpp<0x141>(lm));
    uint32_t t = min(lm, dpp<0x128>(lm));
    const auto h16 = __builtin_amdgcn_permlane16_swap(t, t, false, false);
    t = min((uint32_t)h16[0], (uint32_t)h16[1]);
    const auto h32 = __builtin_amdgcn_permlane32_swap(t, t, false, false);
    t = min((uint32_t)h32[0], (uint32_t)h32[1]);
    const uint32_t T = max((uint32_t)__builtin_amdgcn_readfirstlane(t), 1u);
    stamp(w, l, 10);
    // every lane writes: a lane without a candidate to a slot of its own past the table
    int nc = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const bool f = key[q] >= T;
      const unsigned long long bl = __ballot(f);
      cand[f ? nc + __popcll(bl & lt) : E + lane] = rank_key(key[q], lane + kWave * q);
      nc += __popcll(bl);
    }
    if (lane == 0) {
      *n_slot = (unsigned long long)nc;
      if (ns) {
        un.id[0] = E;
        un.mask[0] = 1u;
        un.pair0[0] = 0;
        un.w[0][0] = 1.0f;
      }
      un.n = ns + K;
      un.n_pairs = ns + K;
    }
    stamp(w, l, 11);
  }
  __syncthreads();
  {
    // candidate c = wave + 16 k: its rank counts the candidates above it, 64 per ballot (stopping
    // once it is known to be outside the top K)
    const int nc = (int)*n_slot;
    const unsigned long long o0 = lane < nc ? cand[lane] : 0ull;
    for (int c = wave; c < nc; c += kWaves) {
      const unsigned long long cc = cand[c];
      int rank = __popcll(__ballot(o0 > cc));
      for (int j0 = kWave; j0 < nc && rank < K; j0 += kWave) {
        const unsigned long long o = j0 + lane < nc ? cand[j0 + lane] : 0ull;
        rank += __popcll(__ballot(o > cc));
      }
      if (rank < K && lane == 0) {
        const int e = (int)(0xffffffffu - (uint32_t)cc), slot = ns + rank;
        s_sel[0][rank] = (uint32_t)(cc >> 32);
        s_idx[0][rank] = e;
        un.id[slot] = e;
        un.mask[slot] = 1u;
        un.pair0[slot] = slot;
      }
    }
  }
  __syncthreads();
  stamp(w, l, 12);
  if (wave == 0) {
    // softmax over the K selected logits, summed in rank order (the same sum in every lane)
    const float z = lane < K ? expf(key_to_float(s_sel[0][lane]) - key_to_float(s_sel[0][0])) : 0.0f;
    float sum = 0.0f;
    for (int r = 0; r < K; ++r) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), r));
    const float wr = z / sum;
    if (lane < K) {
      s_w[0][lane] = wr;
      un.w[ns + lane][0] = wr;
    }
  }
}

// Several tokens: the union, per lane and the same in every wave. Lane j < M * kMaxK holds
// selection (token j / kMaxK, rank j % kMaxK): its expert, whether it is that expert's first
// selection in (token, rank) order (the one that owns the slot), the slot, and where first the
// slot's token mask and first pair. Slot 0 is the shared expert (if any), then the routed
// experts in first-occurrence order.
struct UnionLane {
  int e;            // expert of the selection (-1: no selection)
  bool first;
  int slot;
  unsigned mask;    // where first
  int pair0;        // where first
  int n, n_pairs;   // slots and (slot, token) pairs, wave-uniform
};

template <int M>
__device__ __forceinline__ UnionLane union_lanes(const int (*s_idx)[kMaxK], int K, int ns, int lane, uint32_t* tab,
                                                int E) {
  constexpr int N = M * kMaxK;
  static_assert(N <= kWave, "one wave holds every selection");
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int rj = lane % kMaxK;
  const bool valid = lane < N && rj < K;
  UnionLane u;
  u.e = valid ? s_idx[lane / kMaxK][rj] : -1;
  // per selected expert, through LDS tables indexed by expert (this wave's LDS operations complete
  // in order): the first lane that selects it (atomic minimum) and its tokens (atomic or). Against
  // comparing every selection with every other through lane reads (N rounds): 0.6 us per layer
  // faster at M = 4.
  uint32_t* const first_lane = tab;   // [E]
  uint32_t* const tok_mask = tab + E;   // [E]
  if (valid) {
    first_lane[u.e] = 0xffffffffu;
    tok_mask[u.e] = 0u;
  }
  if (valid) {
    atomicMin(first_lane + u.e, (uint32_t)lane);
    atomicOr(tok_mask + u.e, 1u << (lane / kMaxK));
  }
  const int fl = valid ? (int)first_lane[u.e] : lane;
  const unsigned mask = valid ? tok_mask[u.e] : 0u;
  u.first = valid && fl == lane;
  const unsigned long long firsts = __ballot(u.first);
  u.slot = __builtin_amdgcn_ds_bpermute(fl << 2, ns + (int)__popcll(firsts & lt));
  u.mask = mask;
  // exclusive prefix sum of the first lanes' token counts (at most M <= 4: three bit planes)
  const int cnt = u.first ? __popc(mask) : 0;
  int before = 0, total = ns * M;
#pragma unroll
  for (int bit = 0; bit < 3; ++bit) {
    const unsigned long long bb = __ballot((cnt >> bit) & 1);
    before += __popcll(bb & lt) << bit;
    total += __popcll(bb) << bit;
  }
  u.pair0 = ns * M + before;
  u.n = ns + __popcll(firsts);
  u.n_pairs = total;
  return u;
}
// Several tokens: every thread polls (word i = (expert i / M, token i % M) of the logits, so the
// M words of a line are read by adjacent lanes of one instruction and every line is requested
// once) and the keys go to LDS; wave m < M then finds token m's T and writes its candidates as in
// the one-token case (token m's region: E candidates, 64 slots for the lanes without one, the
// count) and sorts them when they fit in the wave (otherwise every wave ranks its share of that
// token's candidates after the barrier); then wave 0 forms the union while
// wave 1 + m forms token m's weights, and a barrier publishes both (the weights go into the union
// after it: a task reads them only past its own first barrier).
template <int M, int kQ>
__device__ __forceinline__ void select_multi(const Shape& sh, const Work& w, const unsigned long long* lgs,
                                             const Layer& L, uint32_t tag, int tid,
                                             int wave, int lane, unsigned long long* cand, Union& un,
                                             int (*s_idx)[kMaxK], float (*s_w)[kMaxK], uint32_t (*s_sel)[kMaxK],
                                             int l) {
  static_assert(M > 1 && M + 1 <= kWaves, "one token: select_top_one");
  const int E = sh.E, K = sh.K;
  const int ns = sh.has_shared ? 1 : 0;
  const int stride = E + kWave + 1;
  uint32_t* keys = reinterpret_cast<uint32_t*>(cand + (size_t)M * stride);   // [M][E]
  {
    constexpr int N = (M * kQ * kWave + kThreads - 1) / kThreads;
    int idx[N];
    unsigned long long v[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int i = tid + kThreads * k, e = i / M, m = i - e * M;
      idx[k] = e < E ? e * kLgStride<M> + m : -1;
    }
    poll_tagged<N>(w, lgs, idx, tag, v);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int i = tid + kThreads * k, e = i / M, m = i - e * M;
      if (e < E) keys[m * E + e] = sel_key(__uint_as_float((uint32_t)v[k]));
    }
  }
  __syncthreads();
  stamp(w, l, 4);
  if (wave < M) {
    const int m = wave;
    unsigned long long* cm = cand + (size_t)m * stride;
    const unsigned long long lt = (1ull << lane) - 1ull;
    uint32_t key[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int e = lane + kWave * q;
      key[q] = keys[m * E + min(e, E - 1)] & (0u - (uint32_t)(e < E));
    }
    uint32_t lm = key[0];
#pragma unroll
    for (int q = 1; q < kQ; ++q) lm = max(lm, key[q]);
    lm = max(lm, dpp<0xB1>(lm));
    lm = max(lm, dpp<0x4E>(lm));
    lm = max(lm, dpp<0x141>(lm));
    uint32_t t = min(lm, dpp<0x128>(lm));
    const auto h16 = __builtin_amdgcn_permlane16_swap(t, t, false, false);
    t = min((uint32_t)h16[0], (uint32_t)h16[1]);
    const auto h32 = __builtin_amdgcn_permlane32_swap(t, t, false, false);
    t = min((uint32_t)h32[0], (uint32_t)h32[1]);
    const uint32_t T = max((uint32_t)__builtin_amdgcn_readfirstlane(t), 1u);
    stamp(w, l, 10);
    int nc = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const bool f = key[q] >= T;
      const unsigned long long bl = __ballot(f);
      cm[f ? nc + __popcll(bl & lt) : E + lane] = rank_key(key[q], lane + kWave * q);
      nc += __popcll(bl);
    }
    if (lane == 0) cm[E + kWave] = (unsigned long long)nc;
    stamp(w, l, 11);
    if (nc <= kWave) {
      // this token's candidates, one per lane, sorted across the wave: lane r holds rank r
      const unsigned long long c = sort_candidates(lane < nc ? cm[lane] : 0ull, nc, lane);
      if (lane < K) {
        s_sel[m][lane] = (uint32_t)(c >> 32);
        s_idx[m][lane] = (int)(0xffffffffu - (uint32_t)c);
      }
    }
  }
  __syncthreads();
  {
    // tokens with more candidates than a wave holds: every wave ranks its share of them
    int nc[M];
    bool many = false;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      nc[m] = (int)cand[(size_t)m * stride + E + kWave];
      many |= nc[m] > kWave;
    }
    if (many) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (nc[m] <= kWave) continue;
        const unsigned long long* cm = cand + (size_t)m * stride;
        for (int c = wave; c < nc[m]; c += kWaves) {
          const unsigned long long cc = cm[c];
          int rank = 0;
          for (int j0 = 0; j0 < nc[m] && rank < K; j0 += kWave) {
            const unsigned long long o = j0 + lane < nc[m] ? cm[j0 + lane] : 0ull;
            rank += __popcll(__ballot(o > cc));
          }
          if (rank < K && lane == 0) {
            s_sel[m][rank] = (uint32_t)(cc >> 32);
            s_idx[m][rank] = (int)(0xffffffffu - (uint32_t)cc);
          }
        }
      }
      __syncthreads();
    }
  }
  stamp(w, l, 12);
  float wr = 0.0f;
  if (wave == 0) {
    // the candidate area is free again: its tables serve the union
    const UnionLane u = union_lanes<M>(s_idx, K, ns, lane, reinterpret_cast<uint32_t*>(cand), E);
    if (u.first) {
      un.id[u.slot] = u.e;
      un.mask[u.slot] = u.mask;
      un.pair0[u.slot] = u.pair0;
#pragma unroll
      for (int m = 0; m < M; ++m)
        if ((u.mask >> m) & 1u) un.ptok[u.pair0 + __popc(u.mask & ((1u << m) - 1u))] = m;
    }
    if (u.e >= 0) un.sel_slot[lane] = u.slot;   // slot of selection (lane / kMaxK, lane % kMaxK)
    // the shared slot's weight and token of pair m from lane m (a vector of M ones written by one
    // lane was kept in scratch memory across the layer loop and reloaded here)
    if (ns && lane < M) {
      un.w[0][lane] = 1.0f;
      un.ptok[lane] = lane;
    }
    if (lane == 0) {
      if (ns) {
        un.id[0] = E;
        un.mask[0] = (1u << M) - 1u;
        un.pair0[0] = 0;
      }
      un.n = u.n;
      un.n_pairs = u.n_pairs;
    }
  } else if (wave <= M) {
    // softmax over token m's K selections, summed in rank order
    const int m = wave - 1;
    const float z = lane < K ? expf(key_to_float(s_sel[m][lane]) - key_to_float(s_sel[m][0])) : 0.0f;
    float sum = 0.0f;
    for (int r = 0; r < K; ++r) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), r));
    wr = z / sum;
    if (lane < K) {
      s_w[m][lane] = wr;
      if (blockIdx.x == 0) {
        if (L.topk_idx) stg(L.topk_idx + m * K + lane, s_idx[m][lane]);
        if (L.topk_w) stg(L.topk_w + m * K + lane, wr);
      }
    }
  }
  __syncthreads();
  if (wave >= 1 && wave <= M && lane < K) un.w[un.sel_slot[(wave - 1) * kMaxK + lane]][wave - 1] = wr;
}

// ------------------------------------------------------------------------------ the kernel
// Blocks per task group: the smallest divisor of J, at least kmin, for which the nsr routed slots'
// groups fit in G workgroups. A group stores one partial vector per token of its slot after summing
// its blocks in registers, so with several tokens per slot single-block groups multiply the
// partial-sum traffic: the same-expert window at M = 4 (9 slots, 4 tokens each) wrote 17.3 MB of
// partial sums per layer and took 25.3 us per layer; with kmin = 2 for M > 1, 22.5 us (the other
// windows choose 2 or more anyway; one token keeps single blocks, whose burst is the shorter).
__device__ __forceinline__ int group_size(int nsr, int J, int G, int kmin) {
  for (int k = kmin; k < J; ++k)
    if (J % k == 0 && nsr * (J / k) <= G) return k;
  return J;
}

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

// Compiled at run time for one layer shape (hipRTC), the shape's E, K, H, I and shared expert are
// constants; the argument carries the same values.
__device__ __forceinline__ void spec_shape(Shape& sh) {
#ifdef QWS_SPEC_H
  sh.E = QWS_SPEC_E;
  sh.K = QWS_SPEC_K;
  sh.H = QWS_SPEC_H;
  sh.I = QWS_SPEC_I;
  sh.has_shared = QWS_SPEC_SHARED;
#else
  (void)sh;
#endif
}

// One lane's part of a router row's product with one token's x (both bf16 in LDS), summed in the
// order of the two-call router kernel; the caller reduces it across the wave. Every operand read
// is issued before the first product (a scheduling barrier keeps the compiler from interleaving
// them with the products, which made it issue them one or two at a time, each waiting for the
// previous products). Chunks past the row end read the last chunk and use a zero router operand:
// their products add exact zeros, so the sum and its order equal the two-call router's.
__device__ __forceinline__ float router_dot(const uint16_t* wrow, const uint16_t* xm, int H, int lane) {
  const int nrc = H >> 3;
  u32x4_t rv[kRtCpl], xv[kRtCpl];
#pragma unroll
  for (int t = 0; t < kRtCpl; ++t) {
    const int cc = min(lane + t * kWave, nrc - 1);
    rv[t] = *reinterpret_cast<const u32x4_t*>(wrow + cc * 8);
    xv[t] = *reinterpret_cast<const u32x4_t*>(xm + cc * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < kRtCpl; ++t) {
    const uint32_t keep = 0u - (uint32_t)(lane + t * kWave < nrc);
#pragma unroll
    for (int d = 0; d < 4; ++d) acc = dot2(as_bf16x2(rv[t][d] & keep), as_bf16x2(xv[t][d]), acc);
  }
  return acc;
}

// CH: a chained sequence (x of layer l+1 is layer l's bf16 y), whose layers hand x over through
// tagged y words with no barrier between them; otherwise layers are separated by the tagged
// barrier. (A template parameter rather than a flag: the chained-only work, the logits buffers
// alternating by layer parity, cost the other kind 0.1 us per layer when selected at run time.)
template <int M, bool A8, bool CH>
__global__ __launch_bounds__(kThreads) void moe_layers_kernel(Layer first, const qws_moe_layer* __restrict__ rest,
                                                              int n_layers, Shape sh_arg, Work w_arg) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ Union un;
  __shared__ int s_idx[kMaxM][kMaxK];
  __shared__ float s_w[kMaxM][kMaxK];
  __shared__ uint32_t s_sel[kMaxM][kMaxK];
  __shared__ float s_y[kMaxM][kMaxRows];
  __shared__ __attribute__((aligned(16))) unsigned long long s_desc[2][kDescWords];
  __shared__ unsigned long long s_launch;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int G = gridDim.x, b = blockIdx.x;
  Shape sh_k = sh_arg;
  spec_shape(sh_k);
  const Shape& sh = sh_k;
  const int E = sh.E, H = sh.H, I = sh.I, R = sh.R;
  const int J = I / kBlk;

  // dynamic LDS: x [M][H] bf16 | router rows [nrw][H] bf16 | scratch: selection candidates [M][E]
  // u64 (+ 65 u64 per token; + keys [M][E] u32 when M > 1), then a task's gate/up k-slice sums [4][M][64] fp32 and activation parts [M][4][32] bf16,
  // then the combine's per-wave row sums [waves][M][kLine] fp32
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  uint16_t* wr_s = reinterpret_cast<uint16_t*>(lds + (size_t)M * H * 2);
  uint8_t* x8 = lds + (size_t)M * H * 2 + (size_t)sh.nrw * H * 2;
  uint8_t* xs8 = x8 + (size_t)2 * M * H;
  unsigned char* scratch = xs8 + (((size_t)2 * M * (H >> 5) + 15) & ~(size_t)15);
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(scratch);
  float* red = reinterpret_cast<float*>(scratch);

  const int r_row0 = b + G * wave;                      // this wave's router row
  SyncState sync{0ull, false};

  if (tid < kTracePoints) s_stamp[tid] = 0ull;
  // launch number -> this launch's tag base (every workgroup adds 1 per launch)
  if (tid == 0)
    s_launch = __hip_atomic_fetch_add(w_arg.launches, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) / (unsigned)G;
  __syncthreads();
  Work w = w_arg;
  w.launch1 = uniform_u64(s_launch) + 1ull;
  const uint32_t tag_base = (uint32_t)(s_launch * kTagsPerLaunch);
  if (s_launch > 0 && tag_base == 0) {
    // tags repeat from here on: clear every tagged word (tag 0 is never valid) before any use
    const size_t n_part = (size_t)sh.P * J * H;
    for (size_t i = (size_t)b * kThreads + tid; i < n_part; i += (size_t)G * kThreads) st_coherent(w.partial + i, 0ull);
    for (int i = b * kThreads + tid; i < kMaxE * kLine; i += G * kThreads) {
      st_coherent(w.logits + i, 0ull);
      if constexpr (M > 1) st_coherent(w.logits_odd + i, 0ull);   // one token: inside the area above
    }
    for (int i = tid; i < kReplicas * sh.y_stride; i += kThreads)
      st_coherent(ytag_copy(w, sh, i / sh.y_stride) + (size_t)b * sh.y_stride + i % sh.y_stride, 0ull);
    if (tid < kReplicas * kLine) st_coherent(w.done + ((size_t)(tid / kLine) * kMaxGrid + b) * kLine + tid % kLine, 0ull);
    grid_sync(w, sync);
  }

  // router rows of layer 0 -> LDS (asynchronous; this wave waits for them before its dots)
  if (wave < sh.nrw && r_row0 < E) router_row_to_lds(first.wr + (size_t)r_row0 * H, wr_s + (size_t)wave * H, H, lane);

  for (int l = 0; l < n_layers; ++l) {
    // opaque copies of the thread index and the shape per layer: values derived from them are
    // recomputed where they are used instead of being hoisted out of the layer loop and kept live
    // (spilled to memory) across it
    unsigned tid_l = threadIdx.x;
    asm volatile("" : "+v"(tid_l));
    const int tid = (int)tid_l, lane = tid % kWave;   // shadow the kernel-level indices in this layer
    Shape sh = sh_arg;
    asm volatile("" : "+s"(sh.E), "+s"(sh.K), "+s"(sh.H), "+s"(sh.I), "+s"(sh.has_shared), "+s"(sh.R), "+s"(sh.P),
                 "+s"(sh.chained), "+s"(sh.nrw), "+s"(sh.inv_r), "+s"(sh.y_stride), "+s"(sh.x_fresh));
    spec_shape(sh);
    const int E = sh.E, H = sh.H, I = sh.I, R = sh.R;
    const int J = I / kBlk;
    const int ns = sh.has_shared ? 1 : 0;
    const int row0 = b * R;
    const int my_rows = max(0, min(R, H - row0));
    const bool shared_task = kEarlyShared<M> && sh.has_shared && b >= G - J;
    const int r_row = b + G * wave;                       // this wave's router row
    const bool is_router = wave < sh.nrw && r_row < E;
    uint16_t* const my_wr_s = wr_s + (size_t)wave * H;    // its LDS copy (router waves only)
    // descriptor of layer l: layer 0 from the kernel arguments, later ones from the LDS copy made
    // during the previous layer
    Layer L = first;
    if (l > 0) L = desc_from_lds(s_desc[l & 1]);
    // tags never 0: a zero-filled workspace holds tag 0
    const uint32_t tag_lg = tag_base + 4u * (uint32_t)l + 1u, tag_pt = tag_lg + 1u, tag_y = tag_lg + 2u;
    // a chained sequence alternates two logits buffers: a workgroup with no task and no rows may
    // still read layer l's while the others write layer l+1's (they cannot reach layer l+2's,
    // whose logits need this workgroup's router rows of layer l+1); one token's odd buffer is the
    // upper half of the logits area
    unsigned long long* const lgs =
        CH && (l & 1) ? (M == 1 ? w.logits + (size_t)kReplicas * kMaxE : w.logits_odd) : w.logits;
    const bool has_next = l + 1 < n_layers;
    stamp(w, l, 0);

    // ------------------------------------------------------------------ 1: x
    if (l == 0) {
      for (int v = tid; v < M * H / 8; v += kThreads)
        *reinterpret_cast<u32x4_t*>(xs + v * 8) = ld16(L.x + (size_t)v * 8);
    } else if (CH) {
      // y of the previous layer, as its owners published it: bf16 pair i = (m, row 2q) of x
      const int n = M * H / 2, half_r = R / 2;
      constexpr int kXw = (M * kHMax / 2 + kThreads - 1) / kThreads;
      int idx[kXw];
      unsigned long long v[kXw];
#pragma unroll
      for (int q = 0; q < kXw; ++q) {
        const int i = tid + q * kThreads, m = i / (H / 2), qq = i - m * (H / 2);
        const int owner = (int)(((float)qq + 0.5f) * (2.0f * sh.inv_r));
        idx[q] = i < n ? owner * sh.y_stride + m * half_r + (qq - owner * half_r) : -1;
      }
      poll_tagged<kXw>(w, ytag_copy(w, sh, b % kReplicas), idx, tag_y - 4u, v);
#pragma unroll
      for (int q = 0; q < kXw; ++q)
        if (tid + q * kThreads < n) reinterpret_cast<uint32_t*>(xs)[tid + q * kThreads] = (uint32_t)v[q];
    } else if (sh.x_fresh) {
      // the copy of x into LDS issued during the barrier has landed (only the waves that issued
      // part of it wait: another wait would also wait for the barrier word's store)
      if (wave < kCopyWaves && wave * kWave < M * H / 8) wait_mem();
    } else {
      // x may have been written earlier in this launch: device-coherent loads
      const unsigned long long* src = reinterpret_cast<const unsigned long long*>(L.x);
      for (int v = tid; v < M * H / 4; v += kThreads) reinterpret_cast<unsigned long long*>(xs)[v] = ld_coherent(src + v);
    }
    // the router rows copied into LDS by waves 0 .. nrw-1 have landed before this barrier, so that
    // any wave may read them
    if (wave < sh.nrw) wait_mem();
    __syncthreads();
    stamp(w, l, 1);
    // the next layer's descriptor -> registers now (after the x wait: a load issued before it would
    // hold up this layer's x), LDS after the router
    unsigned long long next_desc = 0;
    if (has_next && wave == kWaves - 1 && lane < kDescWords)
      next_desc = ldg(reinterpret_cast<const unsigned long long*>(rest + (l + 1)) + lane);

    // ------------------------------------------------------------------ 2: router, shared task
    // One token (or too many rows per workgroup): wave r takes router row r for every token.
    // Several tokens: wave r * M + m takes row r for token m, so that each wave issues one token's
    // operand reads at once (a wave with four tokens' reads in flight runs out of registers and
    // issues them two at a time).
    if (M > 1 && sh.nrw * M <= kWaves) {
      const int rs = wave / M, mt = wave - rs * M, row = b + G * rs;
      if (rs < sh.nrw && row < E) {
        const float bias = L.bias ? ldg(L.bias + (size_t)mt * L.bias_stride + row) : 0.0f;
        const float lg = wave_sum(router_dot(wr_s + (size_t)rs * H, xs + (size_t)mt * H, H, lane)) + bias;
        if (lane == 0) {
          st_coherent(lgs + (size_t)row * kLgStride<M> + mt, tagged(tag_lg, __float_as_uint(lg)));
          if (L.logits_out) stg(L.logits_out + (size_t)mt * E + row, lg);
        }
      }
    } else if (is_router) {
      // bias loads first (their latency overlaps the dot products), and before any store: a wait
      // for a load between the stores would also wait for the previous store's acknowledgement,
      // slow while other workgroups poll these lines
      float bias[M];
#pragma unroll
      for (int m = 0; m < M; ++m) bias[m] = L.bias ? ldg(L.bias + (size_t)m * L.bias_stride + r_row) : 0.0f;
      float lg[M];
#pragma unroll
      for (int m = 0; m < M; ++m) lg[m] = wave_sum(router_dot(my_wr_s, xs + (size_t)m * H, H, lane)) + bias[m];
      if constexpr (M == 1) {
        if (lane < kReplicas) st_coherent(lgs + (size_t)lane * kMaxE + r_row, tagged(tag_lg, __float_as_uint(lg[0])));
      }
      if (lane == 0) {
        if constexpr (M > 1)
#pragma unroll
          for (int m = 0; m < M; ++m)
            st_coherent(lgs + (size_t)r_row * kLgStride<M> + m, tagged(tag_lg, __float_as_uint(lg[m])));
        if (L.logits_out)
#pragma unroll
          for (int m = 0; m < M; ++m) stg(L.logits_out + (size_t)m * E + r_row, lg[m]);
      }
    }
    if (has_next && wave == kWaves - 1 && lane < kDescWords) s_desc[(l + 1) & 1][lane] = next_desc;
    stamp(w, l, 2);
    // x in FP8 parts for the tasks' gate/up products (published by the next barrier: the shared
    // task's, or the selection's). With one token wave 0 polls the logits meanwhile, so waves 1 ..
    // 15 stage x unless this workgroup runs the shared task first.
    if (tid >= (M == 1 && !shared_task ? kWave : 0)) {
      if constexpr (A8) stage_x8_mx(xs, x8, xs8, M, H, tid, M == 1 && !shared_task ? kWave : 0);
      else stage_x8(xs, x8, xs8, M, H, tid, M == 1 && !shared_task ? kWave : 0);
    }
    if (shared_task) {
      // the shared expert needs no routing: its tasks run while the logits are exchanged
      if (tid == 0) {
        un.id[0] = E;
        un.mask[0] = (1u << M) - 1u;
        un.pair0[0] = 0;
#pragma unroll
        for (int m = 0; m < M; ++m) un.w[0][m] = 1.0f;
      }
      __syncthreads();
      TaskRegs sreg;
      float sout[kOutv<A8>];
      task_load<0, kPieces>(task_rec(L, sh, E, b - (G - J), tid), sreg);
      task_compute<M, A8>(sh, w, sreg, un, 0, (1u << M) - 1u, x8, xs8, red, tid, tag_pt, nullptr, b - (G - J), 0, true, true,
                          sout, b - (G - J));
    }
    stamp(w, l, 3);

    // ------------------------------------------------------------------ 3: top-K and union
    // a lane holds experts lane + 64 q for q < kQ: 8 registers suffice up to 512 experts
    if constexpr (M == 1) {
      if (E <= 8 * kWave) select_top_one<8>(sh, w, lgs, tag_lg, wave, lane, cand, un, s_idx, s_w, s_sel, l);
      else select_top_one<kMaxE / kWave>(sh, w, lgs, tag_lg, wave, lane, cand, un, s_idx, s_w, s_sel, l);
      // no barrier: the gate weights (wave 0, just formed) are read only past a task's first
      // barrier; wave 0 wrote s_idx and s_w itself
      if (b == 0 && tid < sh.K) {
        if (L.topk_idx) stg(L.topk_idx + tid, s_idx[0][tid]);
        if (L.topk_w) stg(L.topk_w + tid, s_w[0][tid]);
      }
    } else {
      // the union is in LDS (its weights are read only past a task's first barrier)
      if (E <= 8 * kWave) select_multi<M, 8>(sh, w, lgs, L, tag_lg, tid, wave, lane, cand, un, s_idx, s_w, s_sel, l);
      else select_multi<M, kMaxE / kWave>(sh, w, lgs, L, tag_lg, tid, wave, lane, cand, un, s_idx, s_w, s_sel, l);
    }
    stamp(w, l, 5);

    // ------------------------------------------------------------------ 4: routed tasks
    {
      // groups of kg consecutive blocks of one slot (kg = the smallest divisor of J, at least 2 with
      // several tokens, that leaves at most G groups): workgroup b takes groups b, b + G, ...; a
      // group's partials add up in
      // registers and are stored once. Each task's loads are issued during the previous one's
      // compute.
      const int s0 = kEarlyShared<M> ? ns : 0;   // first slot of the pool
      const int nsr = un.n - s0, kg = group_size(nsr, J, G, M > 1 ? 2 : 1), jg = J / kg, n_gr = nsr * jg;
      sh.jg = jg;
      int gi = b;
      if (gi < n_gr) {
        TaskRegs cur;
        float outv[kOutv<A8>];
        int t = 0;
        task_load<0, kPieces>(task_rec(L, sh, un.id[s0 + gi / jg], (gi % jg) * kg, tid), cur);
        for (;;) {
          int gn = gi, tn = t + 1;
          if (tn == kg) {
            gn = gi + G;
            tn = 0;
          }
          const uint8_t* nrec =
              gn < n_gr ? task_rec(L, sh, un.id[s0 + gn / jg], (gn % jg) * kg + tn, tid) : nullptr;
          task_compute<M, A8>(sh, w, cur, un, s0 + gi / jg, un.mask[s0 + gi / jg], x8, xs8, red, tid, tag_pt, nrec, 0,
                              s0 * M * J + gi % jg, t == 0, t == kg - 1, outv, (gi % jg) * kg + t);
          if (!nrec) break;
          gi = gn;
          t = tn;
        }
      }
    }
    // the next layer's router rows (weights, which no layer's result changes) -> LDS, here, after
    // this layer's task loads (an LDS DMA pending among them would make every wait for a task load
    // wait for it). During the barrier instead, the last workgroup to arrive passed it at once and
    // then waited for its rows' DMA, which held up every workgroup's logits (0.1 us per layer).
    const uint16_t* next_row = nullptr;
    if (has_next && is_router)
      next_row = reinterpret_cast<const uint16_t*>(
                     uniform_u64(s_desc[(l + 1) & 1][offsetof(qws_moe_layer, w_router_bf16) / 8])) +
                 (size_t)r_row * H;
    if (next_row) router_row_to_lds(next_row, my_wr_s, H, lane);

    stamp(w, l, 6);

    // ------------------------------------------------------------------ 5: combine owned rows
    if (my_rows > 0) {
      // this owner's rows are words row0 .. row0 + my_rows - 1 of every line. Thread t polls row
      // t % 16 of lines t / 16 + 64 k and sums them per token in registers (k ascending), then the
      // four lanes of a wave with that row, then the 16 waves: a fixed order (deterministic)
      // lines: the shared slot's pairs x J blocks, then the routed pairs x jg block groups
      constexpr int kStep = kThreads / kLine;
      const int nsm = kEarlyShared<M> ? ns * M : 0, n_sh = nsm * J;
      const int n_lines = n_sh + (un.n_pairs - nsm) * sh.jg;
      const float inv_jg = 1.0f / (float)sh.jg;
      const unsigned long long* src = w.partial + row0;
      const int r = tid % kLine, L0 = tid / kLine;
      const bool my_row = r < my_rows;
      const float inv_j = 1.0f / (float)J;
      float acc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = 0.0f;
      for (int k0 = 0; k0 * kStep < n_lines; k0 += kPollBatch<M>) {
        int idx[kPollBatch<M>];
        unsigned long long v[kPollBatch<M>];
#pragma unroll
        for (int q = 0; q < kPollBatch<M>; ++q) {
          const int Lq = L0 + (k0 + q) * kStep;
          idx[q] = Lq < n_lines && my_row ? Lq * H + r : -1;
        }
        poll_tagged<kPollBatch<M>>(w, src, idx, tag_pt, v);
#pragma unroll
        for (int q = 0; q < kPollBatch<M>; ++q) {
          if (idx[q] >= 0) {
            const float x = __uint_as_float((uint32_t)v[q]);
            if constexpr (M == 1) {
              acc[0] += x;
            } else {
              const int Lq = L0 + (k0 + q) * kStep;
              const int pq = Lq < n_sh ? (int)(((float)Lq + 0.5f) * inv_j)
                                       : nsm + (int)(((float)(Lq - n_sh) + 0.5f) * inv_jg);
              const int mt = un.ptok[pq];
#pragma unroll
              for (int m = 0; m < M; ++m) acc[m] += m == mt ? x : 0.0f;
            }
          }
        }
      }
      float* wsum = red;   // [wave][M][kLine]
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float x = acc[m];
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(q[0]) + __uint_as_float(q[1]);
        if (lane < kLine) wsum[(wave * M + m) * kLine + lane] = x;
      }
      __syncthreads();
      stamp(w, l, 7);
      if (tid < M * kLine) {
        const int m = tid / kLine, rr = tid % kLine;
        float y = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) y += wsum[(wv * M + m) * kLine + rr];
        if (rr < my_rows) s_y[m][rr] = y;
      }
      __syncthreads();
      stamp(w, l, 13);
      // outputs: a thread takes two adjacent rows of one token (the tagged copy holds a bf16 pair);
      // chained, threads n_out .. kReplicas * n_out - 1 write the other copies of the tagged pairs
      const int n_out = (my_rows / 2) * M;
      const int n_thr = CH && l + 1 < n_layers ? kReplicas * n_out : n_out;
      for (int t = tid; t < n_thr; t += kThreads) {
        const int c = t / n_out, tt = t - c * n_out, rp = tt / M, m = tt - rp * M;
        const float y0 = s_y[m][2 * rp], y1 = s_y[m][2 * rp + 1];
        const size_t o = (size_t)m * H + row0 + 2 * rp;
        const uint16_t h0 = f32_to_bf16_rne(y0), h1 = f32_to_bf16_rne(y1);
        if (c == 0 && L.y32) {
          st_coherent(L.y32 + o, y0);
          st_coherent(L.y32 + o + 1, y1);
        }
        if (c == 0 && L.y16) {
          st_coherent(L.y16 + o, h0);
          st_coherent(L.y16 + o + 1, h1);
        }
        if (CH && l + 1 < n_layers)
          st_coherent(ytag_copy(w, sh, c) + (size_t)b * sh.y_stride + m * (R / 2) + rp,
                      tagged(tag_y, (uint32_t)h0 | ((uint32_t)h1 << 16)));
      }
    }
    flush_stamps(w, l, false);
    stamp(w, l, 8);
    if (!CH && l + 1 < n_layers) {
      // layer l's output is written before layer l+1 starts
      const uint16_t* next_x = nullptr;
      if (sh.x_fresh)
        next_x = reinterpret_cast<const uint16_t*>(uniform_u64(s_desc[(l + 1) & 1][offsetof(qws_moe_layer, x_bf16) / 8]));
      tagged_barrier(w, tag_y, tid, l, next_x, xs, M * H);
      stamp(w, l, 9);
    } else {
      __syncthreads();      // LDS (union, s_y, red) is rewritten by the next layer
    }
  }
  flush_stamps(w, n_layers - 1, true);
}

}  // namespace qws_moe
