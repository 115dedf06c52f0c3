// The FP8 LM-head GEMV of libqws on the matrix cores (gfx950), with its verification epilogues.
// Compiled twice: into the library as a template over (M, mode), and at run time by hipRTC with
// the head's rows and cols fixed (QWS_SPEC_ROWS / QWS_SPEC_COLS), which lets the compiler fold
// every shape-dependent bound (see rtc.hip). One source, so both give the same logits bit for bit.
#pragma once

#include "qws_common.hpp"

namespace qws_head {

using namespace qws;

constexpr int kMaxCols = 2560;

// Non-temporal 16-byte load of head weights (each byte is read once per call).
__device__ __forceinline__ u32x4_t ld16_weights(const void* p) {
  return __builtin_nontemporal_load((const QWS_GLOBAL u32x4_t*)p);
}

// The head's rows in tiles of 16 on the matrix cores: D (16 rows x 16 columns) += A (16 rows x 32
// codes, E4M3 -> bf16, exact) x B (32 columns of x x 16 tokens; tokens M .. 15 are zero), fp32
// accumulation. The codes are stored tile-major (tile t of 16 rows at byte 16 t cols; inside it,
// chunk c of tile row i at byte 16 (16c + i)) so that the 64 lanes of a wave load 1 KB of
// consecutive bytes per instruction: chunk c of tile row i is what lane
// (g = c % 4, i) needs for k-block c / 4. A row-major head read this way moves 16 rows x 64 B per
// instruction and measured ~25% slower on MI355X.
// A workgroup takes one tile at a time; its kHeadWaves waves split the tile's columns, the next
// tile's codes load while the current one is multiplied, and the waves' partial sums meet in LDS.
// Every token's column is computed the same way whatever M is, so a window of M tokens gives each
// token the logits it would get alone, bit for bit.
constexpr int kHeadWaves = 8;
constexpr int kKbw = kMaxCols / 64 / kHeadWaves;  // k-blocks (64 columns) per wave
constexpr int kXsStride = kMaxCols + 64;          // LDS stride of one token's x (bf16 elements)
constexpr int kHeadGrid = 2048;   // workgroups (at most one per tile)

// The first tile of workgroup b (then every G-th after it). Tiles 2j and 2j+1 fill the two halves
// of each 128-byte line of logits (and of row scales); consecutive workgroups run on different
// XCDs, so with tile b each such line was written half by one XCD's L2 and half by another's. Here
// the pair goes to workgroups b and b + 8, which share an XCD, when G is a multiple of 16
// (otherwise tile b): 0.5 us faster at M = 1, 1.2 us at M = 4 on the full head.
__device__ __forceinline__ long long head_tile0(int b, int G) {
  if (G % 16) return b;
  const int x = b % 8, k = b / 8;
  return 16 * (k >> 1) + 2 * x + (k & 1);
}

// kMode: kGemv (logits), kKeys (logits optional, and each workgroup's largest (logit, lower row)
// key per token, for greedy_finish_kernel), kKeys4 (logits, and each workgroup's four largest keys
// per token in descending order, zero where it has fewer rows, for sample_kernel).
enum HeadMode { kGemv = 0, kKeys = 1, kKeys4 = 2 };
constexpr int kListKeys = 4;   // keys per workgroup and token in kKeys4
constexpr int kListTiles = 8;  // sample_kernel: tiles per workgroup at most (rows <= kHeadGrid x 16 x 8)

// The four largest of two descending lists of four: the pairwise maxima of one list against the
// other reversed hold them (as a bitonic sequence), which two compare rounds put in order.
__device__ __forceinline__ void cas_desc(unsigned long long& a, unsigned long long& b) {
  const unsigned long long hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}
__device__ __forceinline__ void merge_top4(unsigned long long (&a)[kListKeys], const unsigned long long (&b)[kListKeys]) {
#pragma unroll
  for (int j = 0; j < kListKeys; ++j) a[j] = a[j] > b[kListKeys - 1 - j] ? a[j] : b[kListKeys - 1 - j];
  cas_desc(a[0], a[2]);
  cas_desc(a[1], a[3]);
  cas_desc(a[0], a[1]);
  cas_desc(a[2], a[3]);
}

template <int M, int kMode>
__global__ __launch_bounds__(kHeadWaves * kWave) void head_fp8_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ scale, long long rows, int cols,
    const uint16_t* __restrict__ x, float* __restrict__ out, unsigned long long* __restrict__ keys) {
#ifdef QWS_SPEC_COLS
  // compiled at run time for one head: the shape is a constant (the arguments carry the same values)
  rows = QWS_SPEC_ROWS;
  cols = QWS_SPEC_COLS;
#endif
  __shared__ __align__(16) uint16_t xs[M * kXsStride];
  __shared__ __align__(16) float red[2][kHeadWaves][M][16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1), g = lane >> 4, i = lane & 15;
  const long long ntiles = (rows + 15) >> 4;   // the grid never exceeds it
  const int ncs = cols >> 4;                   // 16-byte chunks per row
  const int kb0 = wave * kKbw;
  // this wave's codes of a tile: k-blocks kb0 .. kb0 + kKbw - 1, 1 KB each (chunks past the row
  // end are not loaded and add zeros)
  auto load = [&](long long tl, u32x4_t (&w)[kKbw]) {
    const uint8_t* p = q + tl * 16 * (long long)cols + lane * 16;
#pragma unroll
    for (int t = 0; t < kKbw; ++t)
      w[t] = 4 * (kb0 + t) + g < ncs ? ld16_weights(p + (kb0 + t) * 1024) : u32x4_t{0u, 0u, 0u, 0u};
  };
  long long tile = head_tile0(blockIdx.x, gridDim.x);
  u32x4_t cur[kKbw], nxt[kKbw];
  load(tile, cur);
  // epilogue thread: tile row er of token em
  const int er = tid & 15, em = tid >> 4;
  const bool ep = tid < 16 * M;
  float sc = ep ? scale[min(tile * 16 + er, rows - 1)] : 0.0f;
  unsigned long long best = 0ull;   // below every key
  // kKeys4, descending. (Ranked tile by tile: staging the values and ranking them after the last
  // tile measured 2 us slower, since a workgroup's tail delays the next one on its compute unit.)
  unsigned long long top4[kListKeys] = {0ull, 0ull, 0ull, 0ull};
  // x (bf16) into LDS, zero past the row end
  for (int e = tid; e < M * (kXsStride / 8); e += kHeadWaves * kWave) {
    const int m = e / (kXsStride / 8), c = (e % (kXsStride / 8)) * 8;
    *reinterpret_cast<u32x4_t*>(xs + m * kXsStride + c) =
        c < cols ? ld16(x + (size_t)m * cols + c) : u32x4_t{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  int buf = 0;
  for (; tile < ntiles; tile += gridDim.x) {
    const long long tn = tile + gridDim.x;
    if (tn < ntiles) load(tn, nxt);
    const float scn = ep && tn < ntiles ? scale[min(tn * 16 + er, rows - 1)] : 0.0f;
    f32x4_t d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = d0;
#pragma unroll
    for (int t = 0; t < kKbw; ++t) {
      // lane (g, i) holds codes 16c .. 16c+15 of tile row i (c = 4 kb + g): the first 8 go with
      // x columns 16c .. 16c+7 in one product, the last 8 with 16c+8 .. 16c+15 in the other
      u32x4_t xa = {0u, 0u, 0u, 0u}, xb = xa;
      if (i < M) {
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xs + i * kXsStride + 64 * (kb0 + t) + 16 * g);
        xa = xp[0];
        xb = xp[1];
      }
      const u32x4_t w = cur[t];
      const u32x4_t alo = {__builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<false>(w[0])),
                           __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<true>(w[0])),
                           __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<false>(w[1])),
                           __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<true>(w[1]))};
      const u32x4_t ahi = {__builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<false>(w[2])),
                           __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<true>(w[2])),
                           __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<false>(w[3])),
                           __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<true>(w[3]))};
      d0 = mfma_16x16x32(alo, xa, d0);
      d1 = mfma_16x16x32(ahi, xb, d1);
    }
    // lane (g, i < M) holds token i's partial sums of tile rows 4g .. 4g+3
    if (i < M) *reinterpret_cast<f32x4_t*>(&red[buf][wave][i][4 * g]) = d0 + d1;
    __syncthreads();   // red[buf] is rewritten two tiles later, after the next barrier
    if (ep) {
      float v = red[buf][0][em][er];
#pragma unroll
      for (int w = 1; w < kHeadWaves; ++w) v += red[buf][w][em][er];
      v *= sc;
      const long long row = tile * 16 + er;
      if (row < rows) {
        if (kMode != kKeys || out) out[(size_t)em * rows + row] = v;
        if constexpr (kMode == kKeys) {
          const unsigned long long k = rank_key(sel_key(v), (int)row);
          best = k > best ? k : best;
        }
        if constexpr (kMode == kKeys4) {
          // insert into the descending list (the smallest falls off)
          unsigned long long k = rank_key(sel_key(v), (int)row);
#pragma unroll
          for (int j = 0; j < kListKeys; ++j) {
            const unsigned long long hi = top4[j] > k ? top4[j] : k;
            k = top4[j] > k ? k : top4[j];
            top4[j] = hi;
          }
        }
      }
    }
    sc = scn;
    buf ^= 1;
#pragma unroll
    for (int t = 0; t < kKbw; ++t) cur[t] = nxt[t];
  }
  if constexpr (kMode == kKeys) {
    // the workgroup's largest key per token (epilogue threads of token m: the 16-lane groups of
    // wave 0), token-major, for greedy_finish_kernel / sample_kernel
    if (ep) {
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const unsigned long long k = __shfl_xor(best, o, kWave);
        best = k > best ? k : best;
      }
      if (er == 0) keys[(size_t)em * gridDim.x + blockIdx.x] = best;
    }
  }
  if constexpr (kMode == kKeys4) {
    // the workgroup's four largest keys per token: the 16 lists of token m's epilogue threads
    // merged pairwise; [token][workgroup][4], for sample_kernel
    if (ep) {
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        unsigned long long other[kListKeys];
#pragma unroll
        for (int j = 0; j < kListKeys; ++j) other[j] = __shfl_xor(top4[j], o, kWave);
        merge_top4(top4, other);
      }
      if (er == 0) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(keys + ((size_t)em * gridDim.x + blockIdx.x) * kListKeys);
        dst[0] = u32x4_t{(uint32_t)top4[0], (uint32_t)(top4[0] >> 32), (uint32_t)top4[1], (uint32_t)(top4[1] >> 32)};
        dst[1] = u32x4_t{(uint32_t)top4[2], (uint32_t)(top4[2] >> 32), (uint32_t)top4[3], (uint32_t)(top4[3] >> 32)};
      }
    }
  }
}

}  // namespace qws_head
