// Vocabulary LM head on gfx950: online per-row FP8 (E4M3) quantisation of a bf16 head, and the
// head GEMV in FP8 and in bf16, for M <= 4 token vectors, float32 logits.
// The head is 157,184 x 2,560 and every token reads all of it: ~805 MB in bf16, half in FP8
// (runbyai.xyz/posts/593 paragraph 3; Netics, "Online FP8 quantization halves the LM head weight
// reads"). At M = 1 the GEMV is a pure HBM stream, so the kernels are built around keeping many
// 128-bit loads in flight per lane, and the weights are read with non-temporal loads (measured on
// MI355X over the 402 MB FP8 head: 63.6 us against 71.4 us with ordinary loads, whose lines are
// kept in the caches that a read-once stream never revisits):
//  - FP8: half a wave (32 lanes) per row, 5 x 16 B per lane; x (bf16) stays in VGPRs for the whole
//    grid-stride loop, the next row pair's loads are issued before the current pair is reduced.
//    E4M3 -> bf16 is exact and one VALU op per pair; bf16 dot2 accumulates in fp32; the row scale
//    multiplies the reduced sum once.
//  - bf16: one wave per row, 5 x 16 B per lane, same structure.
#include "qws_common.hpp"

namespace {

using namespace qws;

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kCpl = 5;          // chunks per lane; cols <= 2560 for both variants
constexpr int kMaxCols = 2560;

// Non-temporal 16-byte load of head weights (each byte is read once per call).
__device__ __forceinline__ u32x4_t ld16_weights(const void* p) {
  return __builtin_nontemporal_load((const QWS_GLOBAL u32x4_t*)p);
}

__device__ __forceinline__ float group_max64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// --------------------------------------------------------------------------- quantise
// One wave per row: absmax, s = fl32(absmax / 448), codes = E4M3_RNE(fl32(w / s)).
__global__ __launch_bounds__(kBlock) void quantize_fp8_kernel(const uint16_t* __restrict__ w, long long rows,
                                                              int cols, uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int lane = threadIdx.x % kWave;
  const long long nwaves = (long long)gridDim.x * kWavesPerBlock;
  const int nch = cols >> 3;  // chunks of 8 bf16
  for (long long row = (long long)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; row < rows; row += nwaves) {
    const uint16_t* src = w + row * cols;
    u32x4_t v[kCpl];
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int c = lane + t * kWave;
      v[t] = c < nch ? ld16(src + c * 8) : u32x4_t{0, 0, 0, 0};
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
    uint8_t* dst = codes + row * cols;
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int c = lane + t * kWave;
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
        *reinterpret_cast<u32x2_t*>(dst + c * 8) = out;
      }
    }
    if (lane == 0) scales[row] = s;
  }
}

// --------------------------------------------------------------------------- FP8 GEMV
// This lane's share of x: chunks j + 32 t (16 bf16 each) of every token.
template <int M>
__device__ __forceinline__ void fp8_load_x(const uint16_t* __restrict__ x, int cols, int j, u32x4_t (&xr)[M][kCpl][2]) {
  const int nch = cols >> 4;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int c = j + 32 * t;
      xr[m][t][0] = c < nch ? ld16(x + (size_t)m * cols + c * 16) : u32x4_t{0, 0, 0, 0};
      xr[m][t][1] = c < nch ? ld16(x + (size_t)m * cols + c * 16 + 8) : u32x4_t{0, 0, 0, 0};
    }
}
// This lane's partial dot products of one row (its 5 chunks of 16 codes) with the M tokens.
template <int M>
__device__ __forceinline__ void fp8_row_dots(const u32x4_t (&w)[kCpl], const u32x4_t (&xr)[M][kCpl][2], float (&acc)[M]) {
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int t = 0; t < kCpl; ++t) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x2_t lo = fp8x2_to_bf16x2<false>(w[t][d]);
      const bf16x2_t hi = fp8x2_to_bf16x2<true>(w[t][d]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        // codes 4d..4d+3 of the chunk pair with bf16 elements 4d..4d+3: x dwords 2d, 2d+1
        acc[m] = dot2(lo, as_bf16x2(xr[m][t][d >> 1][(2 * d) & 3]), acc[m]);
        acc[m] = dot2(hi, as_bf16x2(xr[m][t][d >> 1][(2 * d + 1) & 3]), acc[m]);
      }
    }
  }
}

template <int M>
__global__ __launch_bounds__(kBlock) void gemv_fp8_kernel(const uint8_t* __restrict__ q, const float* __restrict__ scale,
                                                          long long rows, int cols, const uint16_t* __restrict__ x,
                                                          float* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int half = lane >> 5, j = lane & 31;
  const int nch = cols >> 4;  // chunks of 16 codes
  const long long npairs = (rows + 1) >> 1;
  const long long nwaves = (long long)gridDim.x * kWavesPerBlock;
  long long p = (long long)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (p >= npairs) return;

  u32x4_t xr[M][kCpl][2];
  fp8_load_x<M>(x, cols, j, xr);

  auto load = [&](long long pp, u32x4_t (&wq)[kCpl]) {
    const long long row = 2 * pp + half;
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int c = j + 32 * t;
      wq[t] = (row < rows && c < nch) ? ld16_weights(q + row * cols + c * 16) : u32x4_t{0, 0, 0, 0};
    }
  };
  u32x4_t cur[kCpl], nxt[kCpl];
  load(p, cur);
  for (; p < npairs; p += nwaves) {
    if (p + nwaves < npairs) load(p + nwaves, nxt);
    float acc[M];
    fp8_row_dots<M>(cur, xr, acc);
    const long long row = 2 * p + half;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v = group_sum<32>(acc[m]);
      if (j == 0 && row < rows) out[(size_t)m * rows + row] = scale[row] * v;
    }
#pragma unroll
    for (int t = 0; t < kCpl; ++t) cur[t] = nxt[t];
  }
}

// --------------------------------------------------------------------------- greedy verification
// The FP8 GEMV of a verification window (M positions) with the epilogue fused: each wave keeps,
// per position, the largest (logit, lower row) key of its rows; a workgroup stores the maximum of
// its waves; the last workgroup to arrive (two-level arrival) reduces them to each position's
// target token and forms the accepted prefix of the M - 1 draft tokens.
template <int M>
__global__ __launch_bounds__(kBlock) void verify_fp8_kernel(const uint8_t* __restrict__ q, const float* __restrict__ scale,
                                                            long long rows, int cols, const uint16_t* __restrict__ x,
                                                            float* __restrict__ out, const int* __restrict__ draft,
                                                            int* __restrict__ target_out, int* __restrict__ emitted_out,
                                                            int* __restrict__ n_out, unsigned long long* __restrict__ keys,
                                                            unsigned* __restrict__ counters) {
  __shared__ unsigned long long s_best[kWavesPerBlock][M];
  __shared__ bool s_last;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int half = lane >> 5, j = lane & 31;
  const int nch = cols >> 4;
  const long long npairs = (rows + 1) >> 1;
  const long long nwaves = (long long)gridDim.x * kWavesPerBlock;
  long long p = (long long)blockIdx.x * kWavesPerBlock + wave;
  unsigned long long best[M];
#pragma unroll
  for (int m = 0; m < M; ++m) best[m] = 0ull;   // below every key

  if (p < npairs) {   // no early return: every workgroup arrives below
    u32x4_t xr[M][kCpl][2];
    fp8_load_x<M>(x, cols, j, xr);
    auto load = [&](long long pp, u32x4_t (&wq)[kCpl]) {
      const long long row = 2 * pp + half;
#pragma unroll
      for (int t = 0; t < kCpl; ++t) {
        const int c = j + 32 * t;
        wq[t] = (row < rows && c < nch) ? ld16_weights(q + row * cols + c * 16) : u32x4_t{0, 0, 0, 0};
      }
    };
    u32x4_t cur[kCpl], nxt[kCpl];
    load(p, cur);
    for (; p < npairs; p += nwaves) {
      if (p + nwaves < npairs) load(p + nwaves, nxt);
      float acc[M];
      fp8_row_dots<M>(cur, xr, acc);
      const long long row = 2 * p + half;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = scale[row < rows ? row : rows - 1] * group_sum<32>(acc[m]);
        if (out && j == 0 && row < rows) out[(size_t)m * rows + row] = v;
        const unsigned long long k = row < rows ? rank_key(sel_key(v), (int)row) : 0ull;
        best[m] = k > best[m] ? k : best[m];
      }
#pragma unroll
      for (int t = 0; t < kCpl; ++t) cur[t] = nxt[t];
    }
  }
  // the two half-waves' rows, then the waves of the workgroup
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const unsigned long long o = __shfl_xor(best[m], 32, kWave);
    best[m] = o > best[m] ? o : best[m];
    if (lane == 0) s_best[wave][m] = best[m];
  }
  __syncthreads();
  if (threadIdx.x < M) {
    unsigned long long k = 0ull;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) k = s_best[w][threadIdx.x] > k ? s_best[w][threadIdx.x] : k;
    st_coherent(keys + (size_t)blockIdx.x * M + threadIdx.x, k);
  }
  if (!arrive_last_grid(counters, &s_last)) return;

  // last workgroup: every workgroup's keys (device-coherent loads), then the window
#pragma unroll
  for (int m = 0; m < M; ++m) best[m] = 0ull;
  for (unsigned g = threadIdx.x; g < gridDim.x; g += kBlock)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const unsigned long long k = ld_coherent(keys + (size_t)g * M + m);
      best[m] = k > best[m] ? k : best[m];
    }
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long k = __shfl_xor(best[m], o, kWave);
      best[m] = k > best[m] ? k : best[m];
    }
    if (lane == 0) s_best[wave][m] = best[m];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int target[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      unsigned long long k = 0ull;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) k = s_best[w][m] > k ? s_best[w][m] : k;
      target[m] = (int)(0xffffffffu - (uint32_t)k);
      target_out[m] = target[m];
    }
    // draft i is accepted while it equals the target of position i; then the target of the first
    // position not accepted
    int a = 0;
    while (a < M - 1 && draft[a] == target[a]) ++a;
#pragma unroll
    for (int i = 0; i < M; ++i) emitted_out[i] = i < a ? draft[i] : (i == a ? target[a] : -1);
    *n_out = a + 1;
  }
}

// --------------------------------------------------------------------------- bf16 GEMV
template <int M>
__global__ __launch_bounds__(kBlock) void gemv_bf16_kernel(const uint16_t* __restrict__ w, long long rows, int cols,
                                                           const uint16_t* __restrict__ x, float* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int nch = cols >> 3;  // chunks of 8 bf16
  const long long nwaves = (long long)gridDim.x * kWavesPerBlock;
  long long row = (long long)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
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
// MI355X for the 157,184-row head, ~3% ahead of 2048 and ~10% ahead of one unit per wave)
constexpr int kHeadGrid = 4096;
int grid_for(long long units) {
  long long blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  return (int)(blocks < kHeadGrid ? blocks : kHeadGrid);
}

int check_head(const qws_lmhead* h, unsigned fmt) {
  if (!h || !h->w) return QWS_ERR_ARG;
  if (h->format != fmt) return QWS_ERR_FORMAT;
  if (fmt == QWS_FMT_FP8_E4M3FN_ROWSCALE && !h->row_scale) return QWS_ERR_ARG;
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
  if (st == QWS_OK) *desc_out = qws_lmhead{QWS_FMT_FP8_E4M3FN_ROWSCALE, rows, cols, codes_out, row_scale_out};
  return st;
}

extern "C" int lmhead_gemv_fp8(const qws_lmhead* head, const void* x_bf16, int M, float* logits_out,
                               qws_stream_t stream) {
  int st = check_head(head, QWS_FMT_FP8_E4M3FN_ROWSCALE);
  if (st != QWS_OK) return st;
  if (!x_bf16 || !logits_out) return QWS_ERR_ARG;
  if (M < 1 || M > 4) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(x_bf16)) return QWS_ERR_ALIGN;
  const uint8_t* q = static_cast<const uint8_t*>(head->w);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const int cols = (int)head->cols;
  dim3 grid(grid_for((head->rows + 1) / 2)), block(kBlock);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (M) {
    case 1: hipLaunchKernelGGL(gemv_fp8_kernel<1>, grid, block, 0, s, q, head->row_scale, head->rows, cols, x, logits_out); break;
    case 2: hipLaunchKernelGGL(gemv_fp8_kernel<2>, grid, block, 0, s, q, head->row_scale, head->rows, cols, x, logits_out); break;
    case 3: hipLaunchKernelGGL(gemv_fp8_kernel<3>, grid, block, 0, s, q, head->row_scale, head->rows, cols, x, logits_out); break;
    default: hipLaunchKernelGGL(gemv_fp8_kernel<4>, grid, block, 0, s, q, head->row_scale, head->rows, cols, x, logits_out); break;
  }
  return qws_host::check_launch();
}

extern "C" size_t lmhead_verify_workspace_bytes(int M) {
  if (M < 1 || M > 4) return 0;
  return qws_host::align256((size_t)kHeadGrid * M * 8) + (size_t)(kArriveGroups + 1) * kCounterStride * 4;
}

extern "C" int lmhead_verify_greedy_fp8(const qws_lmhead* head, const void* x_bf16, int M, const int* draft,
                                        float* logits_out, int* target_out, int* emitted_out, int* n_out,
                                        void* workspace, size_t workspace_bytes, qws_stream_t stream) {
  int st = check_head(head, QWS_FMT_FP8_E4M3FN_ROWSCALE);
  if (st != QWS_OK) return st;
  if (!x_bf16 || !target_out || !emitted_out || !n_out || (M > 1 && !draft)) return QWS_ERR_ARG;
  if (M < 1 || M > 4) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(x_bf16)) return QWS_ERR_ALIGN;
  if (!workspace || workspace_bytes < lmhead_verify_workspace_bytes(M)) return QWS_ERR_WORKSPACE;
  if (!qws_host::aligned16(workspace)) return QWS_ERR_ALIGN;
  const uint8_t* q = static_cast<const uint8_t*>(head->w);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const int cols = (int)head->cols;
  unsigned long long* keys = static_cast<unsigned long long*>(workspace);
  unsigned* counters = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) +
                                                   qws_host::align256((size_t)kHeadGrid * M * 8));
  dim3 grid(grid_for((head->rows + 1) / 2)), block(kBlock);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define QWS_VERIFY(MM)                                                                                            \
  hipLaunchKernelGGL(verify_fp8_kernel<MM>, grid, block, 0, s, q, head->row_scale, head->rows, cols, x, logits_out, \
                     draft, target_out, emitted_out, n_out, keys, counters)
  switch (M) {
    case 1: QWS_VERIFY(1); break;
    case 2: QWS_VERIFY(2); break;
    case 3: QWS_VERIFY(3); break;
    default: QWS_VERIFY(4); break;
  }
#undef QWS_VERIFY
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
