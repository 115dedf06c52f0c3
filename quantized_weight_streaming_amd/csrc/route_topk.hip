// MoE router on gfx950: router GEMV over E experts, then top-K and the softmax over the selected
// logits, in ONE launch. Each wave streams one router row (H bf16) with 128-bit loads and dots it
// with the M <= 4 token vectors; the last workgroup to finish (atomic arrival counter) runs the
// selection, one wave per token, on the logits the others left in L2/HBM.
// Routing: eight of 512 routed experts plus a shared one (runbyai.xyz/posts/593 paragraph 2).
#include "qws_common.hpp"

namespace {

using namespace qws;

constexpr int kRouteWaves = 2;          // waves (router rows) per workgroup
constexpr int kRouteCpl = 5;            // 16-byte chunks per lane: H <= 64 * 5 * 8 = 2560
constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / kWave;

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// Top-K of one token's E logits by one wave, then the renormalised softmax gate weights.
// 64-bit key = (ordered logit << 32) | (~index): the maximum is the largest logit, and among
// equal logits the lowest index.
__device__ void select_topk(const float* __restrict__ lg, int E, int K, int* __restrict__ idx_out,
                            float* __restrict__ w_out) {
  const int lane = threadIdx.x % kWave;
  unsigned long long key[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    int e = lane + i * kWave;
    key[i] = e < E ? ((unsigned long long)sel_key(ld_coherent(lg + e)) << 32) | (0xffffffffu - (unsigned)e) : 0ull;
  }
  float sel_v[8];
  int sel_i[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (r < K) {
      unsigned long long best = 0ull;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (key[i] == best) key[i] = 0ull;  // keys are unique (distinct indices): one lane matches
      sel_i[r] = (int)(0xffffffffu - (unsigned)(best & 0xffffffffu));
      sel_v[r] = key_to_float((uint32_t)(best >> 32));
    }
  }
  if (lane == 0) {
    const float vmax = sel_v[0];
    float z[8], s = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r < K) {
        z[r] = expf(sel_v[r] - vmax);
        s += z[r];
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r < K) {
        idx_out[r] = sel_i[r];
        w_out[r] = z[r] / s;
      }
    }
  }
}

template <int M>
__global__ __launch_bounds__(kRouteWaves * kWave) void route_topk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    long long bias_stride, int H, int E, int K, float* __restrict__ logits, int* __restrict__ topk_idx,
    float* __restrict__ topk_w, unsigned* __restrict__ counter) {
  __shared__ bool last_flag;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int e = blockIdx.x * kRouteWaves + wave;
  const int nch = H / 8;  // 16-byte chunks of 8 bf16

  if (e < E) {
    u32x4_t w[kRouteCpl];
    const uint16_t* row = wr + (size_t)e * H;
#pragma unroll
    for (int t = 0; t < kRouteCpl; ++t) {
      int c = lane + t * kWave;
      w[t] = c < nch ? ld16(row + c * 8) : u32x4_t{0, 0, 0, 0};
    }
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      acc[m] = 0.0f;
#pragma unroll
      for (int t = 0; t < kRouteCpl; ++t) {
        int c = lane + t * kWave;
        if (c < nch) {
          u32x4_t xv = ld16(x + (size_t)m * H + c * 8);
#pragma unroll
          for (int d = 0; d < 4; ++d) acc[m] = dot2(as_bf16x2(w[t][d]), as_bf16x2(xv[d]), acc[m]);
        }
      }
      acc[m] = wave_sum(acc[m]);   // the fused layer kernel reduces the same way
    }
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float b = bias ? bias[(size_t)m * bias_stride + e] : 0.0f;
        st_coherent(logits + (size_t)m * E + e, acc[m] + b);
      }
    }
  }

  if (!arrive_last_grid(counter, &last_flag)) return;
  for (int m = wave; m < M; m += kRouteWaves)
    select_topk(logits + (size_t)m * E, E, K, topk_idx + m * K, topk_w + m * K);
}

}  // namespace

constexpr size_t kCounterBytes = (kArriveGroups + 1) * kCounterStride * sizeof(unsigned);

extern "C" size_t moe_route_workspace_bytes(int M, int E) {
  if (M < 1 || M > 4 || E < 1 || E > kMaxE) return 0;
  return qws_host::align256((size_t)M * E * sizeof(float)) + kCounterBytes;
}

extern "C" int moe_route_topk(const void* x_bf16, int M, int H, const void* w_router_bf16, int E,
                              const float* bias, long long bias_row_stride, int K, int* topk_idx,
                              float* topk_w, float* logits_out, void* workspace, size_t workspace_bytes,
                              qws_stream_t stream) {
  if (!x_bf16 || !w_router_bf16 || !topk_idx || !topk_w) return QWS_ERR_ARG;
  if (M < 1 || M > 4 || H < 8 || H > kRouteCpl * kWave * 8 || H % 8 || E < 1 || E > kMaxE) return QWS_ERR_SHAPE;
  if (K < 1 || K > 8 || K > E) return QWS_ERR_SHAPE;
  if (bias && !(bias_row_stride == 0 || bias_row_stride == E)) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(x_bf16) || !qws_host::aligned16(w_router_bf16)) return QWS_ERR_ALIGN;
  if (!workspace) return QWS_ERR_WORKSPACE;
  if (workspace_bytes < moe_route_workspace_bytes(M, E)) return QWS_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(ws);
  unsigned* counter = reinterpret_cast<unsigned*>(ws + qws_host::align256((size_t)M * E * sizeof(float)));
  dim3 grid((E + kRouteWaves - 1) / kRouteWaves), block(kRouteWaves * kWave);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const uint16_t* w = static_cast<const uint16_t*>(w_router_bf16);
  switch (M) {
    case 1: hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, x, w, bias, bias_row_stride, H, E, K, logits, topk_idx, topk_w, counter); break;
    case 2: hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, x, w, bias, bias_row_stride, H, E, K, logits, topk_idx, topk_w, counter); break;
    case 3: hipLaunchKernelGGL(route_topk_kernel<3>, grid, block, 0, s, x, w, bias, bias_row_stride, H, E, K, logits, topk_idx, topk_w, counter); break;
    default: hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, x, w, bias, bias_row_stride, H, E, K, logits, topk_idx, topk_w, counter); break;
  }
  return qws_host::check_launch();
}
