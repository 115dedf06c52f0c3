// Vocabulary LM head on gfx950: online per-row FP8 (E4M3) quantisation of a bf16 head, and the
// head GEMV in FP8 and in bf16, for M <= 4 token vectors, float32 logits.
// The head is 157,184 x 2,560 and every token reads all of it: ~805 MB in bf16, half in FP8
// (runbyai.xyz/posts/593 paragraph 3; Netics, "Online FP8 quantization halves the LM head weight
// reads"). For M <= 4 the GEMV is a pure HBM stream, so the kernels are built around keeping many
// 128-bit loads in flight per lane, and the weights are read with non-temporal loads (measured on
// MI355X with an earlier row-major FP8 GEMV over the 402 MB head: 63.6 us against 71.4 us with
// ordinary loads, whose lines are kept in the caches that a read-once stream never revisits):
//  - FP8: the quantiser writes the codes tile-major (16-row tiles) and the GEMV runs each tile on
//    the matrix cores, with x in LDS: the code registers a wave needs do not grow with M (x held
//    in registers for every token did, and the M = 4 GEMV ran at half speed for want of waves).
//    E4M3 -> bf16 is exact and one VALU op per pair; the products accumulate in fp32; the row
//    scale multiplies the reduced sum once.
//  - bf16: one wave per row, 5 x 16 B per lane, x in registers, the next row's loads issued
//    before the current row is reduced.
#include <mutex>

#include "head_fp8.hpp"

namespace {

using namespace qws;
using namespace qws_head;

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kCpl = 5;          // chunks per lane; cols <= 2560 for both variants

__device__ __forceinline__ float group_max64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// --------------------------------------------------------------------------- quantise
// Byte offset of codes (row r, columns 16c .. 16c+15) in the tile-major FP8 layout: tiles of 16
// rows, tile t at byte 16 t cols; inside a tile, chunk c of tile row r at byte 16 (16c + r).
__host__ __device__ __forceinline__ long long tile_byte(long long r, int c, int cols) {
  return (r >> 4) * 16 * (long long)cols + (16ll * c + (r & 15)) * 16;
}

// One wave per row: absmax, s = fl32(absmax / 448), codes = E4M3_RNE(fl32(w / s)), written
// tile-major; the rows that pad the last tile get zero codes.
__global__ __launch_bounds__(kBlock) void quantize_fp8_kernel(const uint16_t* __restrict__ w, long long rows,
                                                              int cols, uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int lane = threadIdx.x % kWave;
  const long long nwaves = (long long)gridDim.x * kWavesPerBlock;
  const long long rows_pad = (rows + 15) & ~15ll;
  const int nch = cols >> 3;  // chunks of 8 bf16
  for (long long row = (long long)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; row < rows_pad; row += nwaves) {
    const bool real = row < rows;
    const uint16_t* src = w + row * cols;
    u32x4_t v[kCpl];
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int c = lane + t * kWave;
      v[t] = real && c < nch ? ld16(src + c * 8) : u32x4_t{0, 0, 0, 0};
    }
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < kCpl; ++t)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[t][d] & 0xffffu)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[t][d] >> 16)));
      }
    amax = group_max64(amax);
    const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int c = lane + t * kWave;   // 8 codes: half c % 2 of 16-byte chunk c / 2
      if (c < nch) {
        u32x2_t out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float a0 = __fdiv_rn(bf16_bits_to_f32(v[t][2 * h] & 0xffffu), s);
          const float a1 = __fdiv_rn(bf16_bits_to_f32(v[t][2 * h] >> 16), s);
          const float a2 = __fdiv_rn(bf16_bits_to_f32(v[t][2 * h + 1] & 0xffffu), s);
          const float a3 = __fdiv_rn(bf16_bits_to_f32(v[t][2 * h + 1] >> 16), s);
          out[h] = f32x2_to_e4m3x2<true>(a2, a3, f32x2_to_e4m3x2<false>(a0, a1, 0u));
        }
        *reinterpret_cast<u32x2_t*>(codes + tile_byte(row, c >> 1, cols) + 8 * (c & 1)) = out;
      }
    }
    if (real && lane == 0) scales[row] = s;
  }
}

// Row-major E4M3 codes -> tile-major: one thread per 16-byte chunk of the output (chunk c of tile
// row i of tile t); the pad rows of the last tile get zero codes. Bytes move, values never change.
__global__ void tile_major_fp8_kernel(const uint8_t* __restrict__ src, long long rows, int cols,
                                      uint8_t* __restrict__ out, long long n_chunks) {
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < n_chunks;
       o += (long long)gridDim.x * blockDim.x) {
    const long long t = o / cols;          // a tile holds 16 x cols bytes = cols chunks
    const int p = (int)(o - t * cols), c = p >> 4, i = p & 15;
    const long long row = 16 * t + i;
    const u32x4_t v = row < rows ? ld16(src + row * cols + 16 * c) : u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(out + o * 16) = v;
  }
}

// --------------------------------------------------------------------------- greedy verification
// After head_fp8_kernel<M, kKeys>: one workgroup reduces the head workgroups' largest keys of each
// position to its target (the argmax, ties to the lower row) and forms the accepted prefix of the
// M - 1 drafts (draft i accepted while it equals target i; then the first target not accepted).
// A separate launch measured 1.1 us faster than the same reduction in the head kernel's last
// workgroup (which every workgroup must first announce itself to).
constexpr int kFinishThreads = 512;

template <int M>
__global__ __launch_bounds__(kFinishThreads) void greedy_finish_kernel(const unsigned long long* __restrict__ keys,
                                                                      int G, const int* __restrict__ draft,
                                                                      int* __restrict__ target_out,
                                                                      int* __restrict__ emitted_out,
                                                                      int* __restrict__ n_out) {
  __shared__ unsigned long long s_best[kFinishThreads / kWave][M];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  constexpr int kPer = (kHeadGrid + kFinishThreads - 1) / kFinishThreads;
  // the drafts, loaded while the keys are (the prefix below would otherwise wait on each in turn)
  int dr[M > 1 ? M - 1 : 1];
#pragma unroll
  for (int m = 0; m < M - 1; ++m) dr[m] = draft[m];
  unsigned long long kk[M];
#pragma unroll
  for (int m = 0; m < M; ++m) kk[m] = 0ull;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    // past the grid: the last key again (no branch, so the loads issue together)
    const int b = min(tid + j * kFinishThreads, G - 1);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const unsigned long long k = keys[(size_t)m * G + b];
      kk[m] = k > kk[m] ? k : kk[m];
    }
  }
  // each token's wave maximum by DPP and lane-group swaps (no LDS round trips)
#pragma unroll
  for (int m = 0; m < M; ++m) {
    unsigned long long o = xor_lane64<1>(kk[m], lane);
    kk[m] = o > kk[m] ? o : kk[m];
    o = xor_lane64<2>(kk[m], lane);
    kk[m] = o > kk[m] ? o : kk[m];
    o = xor_lane64<4>(kk[m], lane);
    kk[m] = o > kk[m] ? o : kk[m];
    o = xor_lane64<8>(kk[m], lane);
    kk[m] = o > kk[m] ? o : kk[m];
    o = xor_lane64<16>(kk[m], lane);
    kk[m] = o > kk[m] ? o : kk[m];
    o = xor_lane64<32>(kk[m], lane);
    kk[m] = o > kk[m] ? o : kk[m];
    if (lane == 0) s_best[wave][m] = kk[m];
  }
  __syncthreads();
  if (tid == 0) {
    int target[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      unsigned long long k = s_best[0][m];
#pragma unroll
      for (int w = 1; w < kFinishThreads / kWave; ++w) k = s_best[w][m] > k ? s_best[w][m] : k;
      target[m] = (int)(0xffffffffu - (uint32_t)k);
      target_out[m] = target[m];
    }
    // accepted drafts equal their targets: emitted is the targets up to the first rejection
    int a = 0;
#pragma unroll
    for (int m = 0; m < M - 1; ++m)
      if (a == m && dr[m] == target[m]) ++a;
#pragma unroll
    for (int m = 0; m < M; ++m) emitted_out[m] = m <= a ? target[m] : -1;
    *n_out = a + 1;
  }
}

// --------------------------------------------------------------------------- sampled verification
// The window's positions sampled from the FP8 head's logits (temperature, top_k, top_p, a uniform u
// per position from the caller), then the accepted prefix of the drafts. Runs after
// head_fp8_kernel<M, kKeys4>, which leaves the logits and, per head workgroup and token, the four
// largest 64-bit keys (ordered logit, ~row) of the workgroup's rows. One workgroup per position;
// its time is VALU issue (two waves per SIMD, a few dependent lane exchanges per step), so the
// steps work on as few and as narrow values as they can:
//  1. t = a lower bound of the k-th largest workgroup maximum, on their upper 32 bits (the ordered
//     logit): each of the eight waves takes its ceil(k / 8) largest distinct values (rounds of a
//     32-bit wave maximum), one wave sorts those and takes the k-th. At least k maxima reach it,
//     so every key of the token's top k is >= t = (that value, 0) and lies in a workgroup whose
//     maximum reaches t: k of them when the waves split the top k evenly, a few more otherwise
//     (more than 64, e.g. many equal logits: t becomes the exact k-th largest maximum by radix
//     select, which exactly k workgroups reach).
//  2. Candidates: the keys >= t of those workgroups, one listed key per thread. A list holds all
//     of its workgroup's keys >= t unless its fourth key reaches t too (a "full" list: there may
//     be more); only a full list's workgroup has its rows read back from the logits (normal
//     logits: a few positions in a million). They are the top k and a few other keys >= t (k to
//     k + 3 in simulations of normal logits), so one wave sorts them; more than 64 go through a
//     radix select first.
//  3. Softmax at the temperature, the shortest prefix reaching top_p, inversion at u.
//  4. Arrival on a counter that also collects each position's acceptance bit (draft m equals its
//     token): the last position's workgroup reads the window's result off the counter.
// Measured against the earlier form of this kernel (8.1 us; now 6.2 us): 64-bit keys in step 1
// took 1.0 us against 0.4; reading back every candidate workgroup's rows, ~1 us; the tokens
// collected through memory after the arrival, ~1.2 us. Tried and slower: every wave sorting the
// values for t itself (no second barrier), the candidates appended by the threads holding their
// lists in registers (nested appends: ~500 instructions, 1.7 us), sorting each wave's 256 keys
// and merging the waves' top 64, each wave reading its top workgroups' rows ahead of t.
constexpr int kSampleThreads = 512;
constexpr int kMaxTopK = 32;
constexpr int kMaxTilesPerGroup = kListTiles;   // rows <= kHeadGrid x 16 x 8 = 262,144
constexpr int kCandWg = 64;                     // candidate workgroups the fast path holds
constexpr int kCandMax = kCandWg * kMaxTilesPerGroup * 16;

// Inclusive prefix sum over the wave's 64 lanes by DPP: shifts by 1, 2, 4 and 8 lanes inside each
// row of 16 (lanes without a source add 0), then the row totals (lane 15 into the next row, lane
// 31 into the upper two).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_inclusive_sum(float c) {
  c += dpp_or_zero<0x111>(c);
  c += dpp_or_zero<0x112>(c);
  c += dpp_or_zero<0x114>(c);
  c += dpp_or_zero<0x118>(c);
  c += dpp_or_zero<0x142, 0xA>(c);
  return c + dpp_or_zero<0x143, 0xC>(c);
}

// The k-th largest (1 <= k <= n) of the n 64-bit keys a[0 .. n) in LDS, by radix select on 8-bit
// digits from the top (a histogram per digit; the digit where the count from above reaches k).
// Every thread of the workgroup calls it.
__device__ unsigned long long block_kth_largest(const unsigned long long* a, int n, int k, unsigned (*hist)[256],
                                                unsigned long long* s_sel, int* s_need) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  unsigned long long prefix = 0ull;
  int need = k;
  for (int i = tid; i < 256; i += kSampleThreads) hist[0][i] = 0u;
  __syncthreads();
  for (int shift = 56, h = 0; shift >= 0; shift -= 8, h ^= 1) {
    // count this digit into hist[h] and clear the other buffer for the next digit (its last
    // reader, the scan of the previous digit, finished before the barrier that ended it)
    for (int i = tid; i < 256; i += kSampleThreads) hist[h ^ 1][i] = 0u;
    const unsigned long long hi = shift == 56 ? 0ull : ~0ull << (shift + 8);
    for (int i = tid; i < n; i += kSampleThreads) {
      const unsigned long long v = a[i];
      if ((v & hi) == prefix) atomicAdd(&hist[h][(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l counts digits 255 - 4l .. 252 - 4l (from the top)
      unsigned c[4], sum = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[h][255 - 4 * lane - j];
        sum += c[j];
      }
      unsigned incl = sum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const unsigned v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      const unsigned long long reach = __ballot(incl >= (unsigned)need);   // nonzero: the total is >= need
      if (lane == __builtin_ctzll(reach)) {
        unsigned above = incl - sum;
        int d = 252 - 4 * lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (above + c[j] >= (unsigned)need) {
            d = 255 - 4 * lane - j;
            break;
          }
          above += c[j];
        }
        *s_sel = prefix | ((unsigned long long)d << shift);
        *s_need = need - (int)above;
      }
    }
    __syncthreads();
    prefix = *s_sel;
    need = *s_need;
  }
  return prefix;
}

template <int M>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(
    const float* __restrict__ logits, long long rows, const unsigned long long* __restrict__ keys, int G,
    float temperature, int top_k, float top_p, const float* __restrict__ u, const int* __restrict__ draft,
    int* __restrict__ token_out, int* __restrict__ topk_out, int* __restrict__ emitted_out, int* __restrict__ n_out,
    unsigned* __restrict__ counter) {
  constexpr int kWavesS = kSampleThreads / kWave;
  constexpr int kPer = kHeadGrid / kSampleThreads;   // workgroup lists per thread
  static_assert(kPer == 4, "four lists per lane: a wave's maxima fit its four rounds");
  __shared__ unsigned long long s_l[kHeadGrid][kListKeys];   // the lists (maxima first)
  __shared__ unsigned long long s_a[kHeadGrid];               // the maxima (for the exact fallback)
  __shared__ unsigned long long s_c[kCandMax];
  __shared__ unsigned long long s_top[kMaxTopK];
  __shared__ uint32_t s_w[kWavesS][kPer];
  __shared__ unsigned s_hist[2][256];
  __shared__ unsigned long long s_sel, s_t;
  __shared__ int s_need, s_nwg, s_nc, s_ntop, s_nfull;
  __shared__ int s_wg[kCandWg];    // candidate workgroups
  __shared__ int s_fwg[kCandWg];   // those whose lists are full
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int my_draft = m < M - 1 ? draft[m] : -1;
  const long long ntiles = (rows + 15) >> 4;
  const int tpg = (int)((ntiles + G - 1) / G);   // tiles per head workgroup (host: <= 8)
  const int k = (int)(top_k < rows ? top_k : rows);
  const float* lg = logits + (size_t)m * rows;
  // the lists of workgroups tid + q * 512 (zeros past G): four descending keys each
  const int jw = (k + kWavesS - 1) / kWavesS;   // <= 4
  unsigned long long kl[kPer][kListKeys];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = tid + q * kSampleThreads;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(keys + ((size_t)m * G + min(i, G - 1)) * kListKeys);
    const u32x4_t lo = ld16(src), hi = ld16(src + 1);
    const bool in = i < G;
    kl[q][0] = in ? (unsigned long long)lo[1] << 32 | lo[0] : 0ull;
    kl[q][1] = in ? (unsigned long long)lo[3] << 32 | lo[2] : 0ull;
    kl[q][2] = in ? (unsigned long long)hi[1] << 32 | hi[0] : 0ull;
    kl[q][3] = in ? (unsigned long long)hi[3] << 32 | hi[2] : 0ull;
    s_a[i] = kl[q][0];
#pragma unroll
    for (int j = 0; j < kListKeys; ++j) s_l[i][j] = kl[q][j];
  }
  if (tid == 0) {
    s_nwg = 0;
    s_nc = 0;
    s_ntop = 0;
    s_nfull = 0;
  }
  // 1. each wave's jw largest distinct upper words of its maxima (a round clears every copy)
  uint32_t kh[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) kh[q] = (uint32_t)(kl[q][0] >> 32);
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    if (r < jw) {
      uint32_t mx = max(max(kh[0], kh[1]), max(kh[2], kh[3]));
      mx = wave_max_u32(mx, lane);
#pragma unroll
      for (int q = 0; q < kPer; ++q) kh[q] = kh[q] == mx ? 0u : kh[q];
      if (lane == 0) s_w[wave][r] = mx;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // the waves' values sit in lanes 4w + r < 32
    static_assert(kWavesS * 4 <= 32, "one lane group of 32 holds the waves' values");
    const int w = lane >> 2, r = lane & 3;
    const uint32_t v = wave_sort_desc<32>(w < kWavesS && r < jw ? s_w[w][r] : 0u, lane);
    const uint32_t kth = (uint32_t)__builtin_amdgcn_readlane((int)v, k - 1);
    if (lane == 0) s_t = G > k ? (unsigned long long)kth << 32 : 0ull;
  }
  __syncthreads();
  unsigned long long t = s_t;
  // 2. the candidate workgroups (maximum >= t) and those among them whose lists are full
  auto discover = [&]() {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int b = tid + q * kSampleThreads;
      if (b < G && kl[q][0] >= t) {
        const int at = atomicAdd(&s_nwg, 1);
        if (at < kCandWg) {
          s_wg[at] = b;
          if (kl[q][kListKeys - 1] != 0ull && kl[q][kListKeys - 1] >= t) s_fwg[atomicAdd(&s_nfull, 1)] = b;
        }
      }
    }
  };
  discover();
  __syncthreads();
  if (s_nwg > kCandWg) {
    // the waves' maxima were too uneven: the exact k-th largest, reached by exactly k workgroups
    t = block_kth_largest(s_a, G, k, s_hist, &s_sel, &s_need);
    if (tid == 0) {
      s_nwg = 0;
      s_nfull = 0;
    }
    __syncthreads();
    discover();
    __syncthreads();
  }
  // the listed keys >= t of the candidates whose lists are not full, one per thread
  const int nwg = s_nwg;
  if (tid < nwg * kListKeys) {
    const int b = s_wg[tid / kListKeys];
    const unsigned long long key = s_l[b][tid % kListKeys], last = s_l[b][kListKeys - 1];
    if (!(last != 0ull && last >= t) && key != 0ull && key >= t) s_c[atomicAdd(&s_nc, 1)] = key;
  }
  // the rows of the full lists' workgroups that reach t
  const int nfl = s_nfull, per = tpg * 16;
  if (nfl > 0 && (rows & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0) {
    // four rows per load: slot i = quarter i % 4 of tile i / 4 of those workgroups' tiles (16-byte
    // aligned: the logits are, and every position's start at a multiple of 4 rows; a quarter is
    // whole rows or none, since rows is a multiple of 4)
    constexpr int kPerQ = kCandMax / 4 / kSampleThreads;
    long long r0[kPerQ];
    f32x4_t v[kPerQ];
#pragma unroll
    for (int j = 0; j < kPerQ; ++j) {
      const int i = tid + j * kSampleThreads, ti = i >> 2;
      const long long tile = ti < nfl * tpg ? head_tile0(s_fwg[ti / tpg], G) + (long long)(ti % tpg) * G : ntiles;
      r0[j] = tile < ntiles && tile * 16 + 4 * (i & 3) < rows ? tile * 16 + 4 * (i & 3) : -1;
      v[j] = r0[j] >= 0 ? *reinterpret_cast<const f32x4_t*>(lg + r0[j]) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int j = 0; j < kPerQ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned long long key = rank_key(sel_key(v[j][e]), (int)(r0[j] + e));
        if (r0[j] >= 0 && key >= t) s_c[atomicAdd(&s_nc, 1)] = key;
      }
  } else if (nfl > 0) {
    constexpr int kPerC = kCandMax / kSampleThreads;
    long long row[kPerC];
    float v[kPerC];
#pragma unroll
    for (int j = 0; j < kPerC; ++j) {
      const int i = tid + j * kSampleThreads;
      const long long tile = i < nfl * per ? head_tile0(s_fwg[i / per], G) + (long long)((i % per) >> 4) * G : ntiles;
      row[j] = tile < ntiles && tile * 16 + (i & 15) < rows ? tile * 16 + (i & 15) : -1;
      v[j] = row[j] >= 0 ? lg[row[j]] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kPerC; ++j) {
      const unsigned long long key = rank_key(sel_key(v[j]), (int)row[j]);
      if (row[j] >= 0 && key >= t) s_c[atomicAdd(&s_nc, 1)] = key;
    }
  }
  __syncthreads();
  const int nc = s_nc;   // >= k
  const unsigned long long* top = s_c;
  if (nc > kWave) {
    const unsigned long long tk = block_kth_largest(s_c, nc, k, s_hist, &s_sel, &s_need);
    for (int i = tid; i < nc; i += kSampleThreads)
      if (s_c[i] >= tk) s_top[atomicAdd(&s_ntop, 1)] = s_c[i];
    __syncthreads();
    top = s_top;
  }
  // 3. wave 0: the k keys in order (bitonic sort across the lanes, descending), then the sample
  if (wave != 0) return;
  const int n = nc > kWave ? k : nc;
  const unsigned long long key = sort_candidates(lane < n ? top[lane] : 0ull, n, lane);
  const int row = (int)(0xffffffffu - (uint32_t)key);
  const float v = key_to_float((uint32_t)(key >> 32));
  const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  // probabilities relative to the largest: exp((v - v0) / temperature), their running sums
  const float p = lane < k ? expf(__fdiv_rn(v - v0, temperature)) : 0.0f;
  const float c = wave_inclusive_sum(p);
  const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), k - 1));
  // the shortest prefix whose share reaches top_p, then the first token of it whose running sum
  // exceeds u times the prefix's sum
  const unsigned long long reach = __ballot(lane < k && c >= top_p * total);
  const int keep = reach ? __builtin_ctzll(reach) + 1 : k;
  const float sk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), keep - 1));
  const unsigned long long over = __ballot(lane < keep && c > u[m] * sk);
  const int pick = over ? __builtin_ctzll(over) : keep - 1;
  const int token = __builtin_amdgcn_readlane(row, pick);
  if (topk_out && lane < top_k) topk_out[(size_t)m * top_k + lane] = lane < k ? row : -1;
  // 4. the window: emitted[i] is token i for every i up to the first rejected draft a (accepted
  // drafts equal their tokens) and -1 after it. Each position stores its token there and, once
  // that store is acknowledged, arrives with its acceptance bit: counter += 256 + (bit << m). The
  // last to arrive has every bit, stores -1 past a (after every other position's token store) and
  // n = a + 1, and clears the counter for the next call.
  if (lane == 0) {
    token_out[m] = token;
    st_coherent(emitted_out + m, token);
    wait_mem();
    const unsigned add = 256u + ((m < M - 1 && my_draft == token ? 1u : 0u) << m);
    const unsigned now = __hip_atomic_fetch_add(counter, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
    if ((now >> 8) == (unsigned)M) {
      st_coherent(counter, 0u);
      int a = 0;
      while (a < M - 1 && ((now >> a) & 1u)) ++a;
      for (int i = a + 1; i < M; ++i) st_coherent(emitted_out + i, -1);
      *n_out = a + 1;
    }
  }
}

// --------------------------------------------------------------------------- bf16 GEMV
template <int M>
__global__ __launch_bounds__(kBlock) void gemv_bf16_kernel(const uint16_t* __restrict__ w, long long rows, int cols,
                                                           const uint16_t* __restrict__ x, float* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int nch = cols >> 3;  // chunks of 8 bf16
  const long long nwaves = (long long)gridDim.x * kWavesPerBlock;
  // the 8 four-row groups of each 128-byte line of logits go to workgroups of one XCD (b, b + 8,
  // .. b + 56: consecutive workgroups run on different XCDs) when the grid is a multiple of 64
  const int b = blockIdx.x, xcd = b % 8, k = b / 8;
  const long long slot = gridDim.x % 64 ? b : 64 * (k / 8) + 8 * xcd + k % 8;
  long long row = slot * kWavesPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;

  u32x4_t xr[M][kCpl];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int c = lane + kWave * t;
      xr[m][t] = c < nch ? ld16(x + (size_t)m * cols + c * 8) : u32x4_t{0, 0, 0, 0};
    }
  auto load = [&](long long rr, u32x4_t (&wv)[kCpl]) {
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int c = lane + kWave * t;
      wv[t] = c < nch ? ld16_weights(w + rr * cols + c * 8) : u32x4_t{0, 0, 0, 0};
    }
  };
  u32x4_t cur[kCpl], nxt[kCpl];
  load(row, cur);
  for (; row < rows; row += nwaves) {
    if (row + nwaves < rows) load(row + nwaves, nxt);
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int t = 0; t < kCpl; ++t)
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = dot2(as_bf16x2(cur[t][d]), as_bf16x2(xr[m][t][d]), acc[m]);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v = group_sum<kWave>(acc[m]);
      if (lane == 0) out[(size_t)m * rows + row] = v;
    }
#pragma unroll
    for (int t = 0; t < kCpl; ++t) cur[t] = nxt[t];
  }
}

// 16 workgroups per CU; each wave loops over the rest (4096 .. 8192 workgroups measured best on
// MI355X for the bf16 head, ~3% ahead of 2048 and ~10% ahead of one unit per wave)
constexpr int kGemvGrid = 4096;
int grid_for(long long units) {
  long long blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  return (int)(blocks < kGemvGrid ? blocks : kGemvGrid);
}

int check_head(const qws_lmhead* h, unsigned fmt) {
  if (!h || !h->w) return QWS_ERR_ARG;
  if (h->format != fmt) return QWS_ERR_FORMAT;
  if ((fmt == QWS_FMT_FP8_E4M3FN_ROWSCALE_T16 || fmt == QWS_FMT_FP8_E4M3FN_ROWSCALE) && !h->row_scale)
    return QWS_ERR_ARG;
  if (h->rows < 1 || h->rows > (1ll << 31) || h->cols < 32 || h->cols > kMaxCols || h->cols % 32) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(h->w)) return QWS_ERR_ALIGN;
  return QWS_OK;
}

}  // namespace

extern "C" int lmhead_bf16_desc(const void* w_bf16, long long rows, long long cols, qws_lmhead* desc_out) {
  if (!w_bf16 || !desc_out) return QWS_ERR_ARG;
  qws_lmhead d{QWS_FMT_BF16, rows, cols, w_bf16, nullptr};
  int st = check_head(&d, QWS_FMT_BF16);
  if (st == QWS_OK) *desc_out = d;
  return st;
}

extern "C" int lmhead_quantize_fp8(const void* w_bf16, long long rows, long long cols, unsigned char* codes_out,
                                   float* row_scale_out, qws_lmhead* desc_out, qws_stream_t stream) {
  if (!w_bf16 || !codes_out || !row_scale_out || !desc_out) return QWS_ERR_ARG;
  if (rows < 1 || rows > (1ll << 31) || cols < 32 || cols > kMaxCols || cols % 32) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(w_bf16) || !qws_host::aligned16(codes_out)) return QWS_ERR_ALIGN;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3(grid_for(rows)), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(w_bf16), rows, (int)cols, codes_out, row_scale_out);
  int st = qws_host::check_launch();
  if (st == QWS_OK) *desc_out = qws_lmhead{QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, rows, cols, codes_out, row_scale_out};
  return st;
}

extern "C" int lmhead_fp8_tile_major(const qws_lmhead* src, unsigned char* codes_out, size_t codes_bytes,
                                     qws_lmhead* desc_out, qws_stream_t stream) {
  if (!desc_out || !codes_out) return QWS_ERR_ARG;
  int st = check_head(src, QWS_FMT_FP8_E4M3FN_ROWSCALE);
  if (st != QWS_OK) return st;
  const size_t need = (size_t)((src->rows + 15) / 16 * 16) * (size_t)src->cols;
  if (codes_bytes < need) return QWS_ERR_WORKSPACE;
  if (!qws_host::aligned16(codes_out)) return QWS_ERR_ALIGN;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src->w), b = reinterpret_cast<uintptr_t>(codes_out);
  const size_t in_bytes = (size_t)src->rows * (size_t)src->cols;
  if (a < b + need && b < a + in_bytes) return QWS_ERR_ARG;
  const long long n = (long long)(need / 16);
  const long long want = (n + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(tile_major_fp8_kernel, dim3((unsigned)(want < 65536 ? want : 65536)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(src->w), src->rows, (int)src->cols,
                     codes_out, n);
  st = qws_host::check_launch();
  if (st == QWS_OK) *desc_out = qws_lmhead{QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, src->rows, src->cols, codes_out, src->row_scale};
  return st;
}

namespace {
// One launch of head_fp8_kernel: M tokens; with `keys`, each workgroup's largest key per token too
// (its four largest with `list4`).
int launch_head_fp8(const qws_lmhead* head, const void* x_bf16, int M, float* logits_out, unsigned long long* keys,
                    hipStream_t s, bool list4 = false) {
  const uint8_t* q = static_cast<const uint8_t*>(head->w);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const int cols = (int)head->cols;
  const long long ntiles = (head->rows + 15) / 16;
  dim3 grid((unsigned)(ntiles < kHeadGrid ? ntiles : kHeadGrid)), block(kHeadWaves * kWave);
#define QWS_HEAD(MM, VV)                                                                                    \
  hipLaunchKernelGGL((head_fp8_kernel<MM, VV>), grid, block, 0, s, q, head->row_scale, head->rows, cols, x, \
                     logits_out, keys)
#define QWS_HEAD_M(VV)                  \
  switch (M) {                          \
    case 1: QWS_HEAD(1, VV); break;     \
    case 2: QWS_HEAD(2, VV); break;     \
    case 3: QWS_HEAD(3, VV); break;     \
    default: QWS_HEAD(4, VV); break;    \
  }
  if (keys && list4) {
    QWS_HEAD_M(kKeys4)
  } else if (keys) {
    QWS_HEAD_M(kKeys)
  } else {
    QWS_HEAD_M(kGemv)
  }
#undef QWS_HEAD_M
#undef QWS_HEAD
  return qws_host::check_launch();
}
}  // namespace

extern "C" size_t lmhead_fp8_codes_bytes(long long rows, long long cols) {
  if (rows < 1 || rows > (1ll << 31) || cols < 32 || cols > kMaxCols || cols % 32) return 0;
  return (size_t)((rows + 15) / 16 * 16) * (size_t)cols;
}

extern "C" int lmhead_gemv_fp8(const qws_lmhead* head, const void* x_bf16, int M, float* logits_out,
                               qws_stream_t stream) {
  int st = check_head(head, QWS_FMT_FP8_E4M3FN_ROWSCALE_T16);
  if (st != QWS_OK) return st;
  if (!x_bf16 || !logits_out) return QWS_ERR_ARG;
  if (M < 1 || M > 4) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(x_bf16)) return QWS_ERR_ALIGN;
  return launch_head_fp8(head, x_bf16, M, logits_out, nullptr, static_cast<hipStream_t>(stream));
}

// Verification workspace: per-workgroup keys, [M][kHeadGrid] u64 for the greedy epilogue and
// [M][kHeadGrid][4] for the sampled one, then 256 B for the sampling kernel's arrival counter.
size_t verify_keys_bytes(int M) { return qws_host::align256((size_t)kHeadGrid * M * kListKeys * 8); }

extern "C" size_t lmhead_verify_workspace_bytes(int M) {
  if (M < 1 || M > 4) return 0;
  return verify_keys_bytes(M) + 256;
}

namespace {
// Argument checks of the greedy verification (everything but the workspace).
int check_verify_greedy(const qws_lmhead* head, const void* x_bf16, int M, const int* draft, const int* target_out,
                        const int* emitted_out, const int* n_out) {
  int st = check_head(head, QWS_FMT_FP8_E4M3FN_ROWSCALE_T16);
  if (st != QWS_OK) return st;
  if (!x_bf16 || !target_out || !emitted_out || !n_out || (M > 1 && !draft)) return QWS_ERR_ARG;
  if (M < 1 || M > 4) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(x_bf16)) return QWS_ERR_ALIGN;
  return QWS_OK;
}

// The two launches of the greedy verification, with the head workgroups' keys in `keys`
// (kHeadGrid x M words; written by the first launch before the second reads them).
int launch_verify_greedy(const qws_lmhead* head, const void* x_bf16, int M, const int* draft, float* logits_out,
                         int* target_out, int* emitted_out, int* n_out, unsigned long long* keys, hipStream_t s) {
  int st = launch_head_fp8(head, x_bf16, M, logits_out, keys, s);
  if (st != QWS_OK) return st;
  const long long ntiles = (head->rows + 15) / 16;
  const int G = (int)(ntiles < kHeadGrid ? ntiles : kHeadGrid);
#define QWS_FINISH(MM)                                                                                         \
  hipLaunchKernelGGL(greedy_finish_kernel<MM>, dim3(1), dim3(kFinishThreads), 0, s, keys, G, draft, target_out, \
                     emitted_out, n_out)
  switch (M) {
    case 1: QWS_FINISH(1); break;
    case 2: QWS_FINISH(2); break;
    case 3: QWS_FINISH(3); break;
    default: QWS_FINISH(4); break;
  }
#undef QWS_FINISH
  return qws_host::check_launch();
}
}  // namespace

extern "C" int lmhead_verify_greedy_fp8(const qws_lmhead* head, const void* x_bf16, int M, const int* draft,
                                        float* logits_out, int* target_out, int* emitted_out, int* n_out,
                                        void* workspace, size_t workspace_bytes, qws_stream_t stream) {
  int st = check_verify_greedy(head, x_bf16, M, draft, target_out, emitted_out, n_out);
  if (st != QWS_OK) return st;
  if (!workspace || workspace_bytes < lmhead_verify_workspace_bytes(M)) return QWS_ERR_WORKSPACE;
  if (!qws_host::aligned16(workspace)) return QWS_ERR_ALIGN;
  return launch_verify_greedy(head, x_bf16, M, draft, logits_out, target_out, emitted_out, n_out,
                              static_cast<unsigned long long*>(workspace), static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
// Greedy verification without a caller's workspace, for callers that cannot allocate. The keys go
// to `scratch`, a device array of this library (one per GPU, kept until the process ends). In host
// code `scratch` names a host-side stand-in, not device memory: its device address is looked up
// once per device with hipGetSymbolAddress and only that address is used.
namespace {
constexpr size_t kScratchBytes = (size_t)kHeadGrid * 4 * 8;   // keys of a 4-position window
static_assert(kScratchBytes == 65536, "scratch: one 64-bit key per (head workgroup, position)");
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[64];   // per device: the device address of `scratch`, 0 until looked up

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return qws_host::set_device_error(e);
  if (dev < 0 || dev >= 64) return QWS_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return qws_host::set_device_error(e);
    if (!p) return QWS_ERR_DEVICE;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return QWS_OK;
}
}  // namespace

extern "C" int lmhead_verify_greedy_fp8_noalloc(const qws_lmhead* head, const void* x_bf16, int M, const int* draft,
                                                float* logits_out, int* target_out, int* emitted_out, int* n_out,
                                                qws_stream_t stream) {
  int st = check_verify_greedy(head, x_bf16, M, draft, target_out, emitted_out, n_out);
  if (st != QWS_OK) return st;
  if ((size_t)kHeadGrid * (size_t)M * 8 > kScratchBytes)
    return qws_host::set_error_text(QWS_ERR_WORKSPACE, "window larger than the library's verification scratch");
  void* keys = nullptr;
  st = scratch_address(&keys);
  if (st != QWS_OK) return st;
  return launch_verify_greedy(head, x_bf16, M, draft, logits_out, target_out, emitted_out, n_out,
                              static_cast<unsigned long long*>(keys), static_cast<hipStream_t>(stream));
}

extern "C" int lmhead_verify_sample_fp8(const qws_lmhead* head, const void* x_bf16, int M, const int* draft,
                                        float temperature, int top_k, float top_p, const float* u,
                                        float* logits_out, int* token_out, int* topk_out, int* emitted_out,
                                        int* n_out, void* workspace, size_t workspace_bytes, qws_stream_t stream) {
  int st = check_head(head, QWS_FMT_FP8_E4M3FN_ROWSCALE_T16);
  if (st != QWS_OK) return st;
  if (!x_bf16 || !u || !logits_out || !token_out || !emitted_out || !n_out || (M > 1 && !draft)) return QWS_ERR_ARG;
  if (!(temperature > 0.0f) || !(temperature < 3.0e38f) || !(top_p > 0.0f) || !(top_p <= 1.0f)) return QWS_ERR_ARG;
  if (M < 1 || M > 4 || top_k < 1 || top_k > kMaxTopK) return QWS_ERR_SHAPE;
  const long long ntiles = (head->rows + 15) / 16;
  const int G = (int)(ntiles < kHeadGrid ? ntiles : kHeadGrid);
  if ((ntiles + G - 1) / G > kMaxTilesPerGroup) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(x_bf16)) return QWS_ERR_ALIGN;
  if (!workspace || workspace_bytes < lmhead_verify_workspace_bytes(M)) return QWS_ERR_WORKSPACE;
  if (!qws_host::aligned16(workspace)) return QWS_ERR_ALIGN;
  unsigned long long* keys = static_cast<unsigned long long*>(workspace);
  char* tail = static_cast<char*>(workspace) + verify_keys_bytes(M);
  unsigned* counter = reinterpret_cast<unsigned*>(tail);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_head_fp8(head, x_bf16, M, logits_out, keys, s, true);
  if (st != QWS_OK) return st;
#define QWS_SAMPLE(MM)                                                                                             \
  hipLaunchKernelGGL(sample_kernel<MM>, dim3(MM), dim3(kSampleThreads), 0, s, logits_out, head->rows, keys, G,      \
                     temperature, top_k, top_p, u, draft, token_out, topk_out, emitted_out, n_out, counter)
  switch (M) {
    case 1: QWS_SAMPLE(1); break;
    case 2: QWS_SAMPLE(2); break;
    case 3: QWS_SAMPLE(3); break;
    default: QWS_SAMPLE(4); break;
  }
#undef QWS_SAMPLE
  return qws_host::check_launch();
}

extern "C" int lmhead_gemv_bf16(const qws_lmhead* head, const void* x_bf16, int M, float* logits_out,
                                qws_stream_t stream) {
  int st = check_head(head, QWS_FMT_BF16);
  if (st != QWS_OK) return st;
  if (!x_bf16 || !logits_out) return QWS_ERR_ARG;
  if (M < 1 || M > 4) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(x_bf16)) return QWS_ERR_ALIGN;
  const uint16_t* w = static_cast<const uint16_t*>(head->w);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const int cols = (int)head->cols;
  dim3 grid(grid_for(head->rows)), block(kBlock);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (M) {
    case 1: hipLaunchKernelGGL(gemv_bf16_kernel<1>, grid, block, 0, s, w, head->rows, cols, x, logits_out); break;
    case 2: hipLaunchKernelGGL(gemv_bf16_kernel<2>, grid, block, 0, s, w, head->rows, cols, x, logits_out); break;
    case 3: hipLaunchKernelGGL(gemv_bf16_kernel<3>, grid, block, 0, s, w, head->rows, cols, x, logits_out); break;
    default: hipLaunchKernelGGL(gemv_bf16_kernel<4>, grid, block, 0, s, w, head->rows, cols, x, logits_out); break;
  }
  return qws_host::check_launch();
}

