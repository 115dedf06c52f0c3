// Routed-expert FFN in MXFP4 on gfx950, for a window of M <= 4 tokens.
//
// Each routed expert selected by any token of the window is read from HBM once, for all tokens
// that selected it (the expert union of a verification pass: runbyai.xyz/posts/593 paragraph 5).
// Two launches:
//   gate_up_swiglu: grid (I / 16, slots). A 16-lane group owns one gate or up row and streams its
//                   1,280 nibble bytes as 5 x 128-bit loads per lane; the partner group owns the
//                   matching up/gate row, so the SwiGLU happens in registers after a 16-lane
//                   reduction. x sits in LDS as bf16; e2m1 -> bf16 (block scale applied) in one
//                   VALU op per pair, then bf16 dot2 with fp32 accumulation.
//   down_combine:   grid (H / 64, slots). An 8-lane group owns one down row of one expert (384
//                   bytes); the float32 activations sit in LDS; e2m1 -> fp32 and fp32 FMA. Each
//                   workgroup writes its gate-weighted partial rows; the last workgroup of a row
//                   block (arrival counter) sums the slots in slot order -- a fixed order, so the
//                   result is deterministic -- and writes y in fp32 and/or bf16.
// Slots: 0 .. n_u-1 are the distinct valid routed ids in ascending order, then the shared expert.
#include "qws_common.hpp"

namespace {

using namespace qws;

constexpr int kMaxM = 4;
constexpr int kMaxK = 8;
constexpr int kMaxSlots = kMaxM * kMaxK + 1;
constexpr int kBlock = 256;
constexpr int kGuRows = 2;              // rows per 16-lane group in gate_up
constexpr int kGuCpl = 5;               // 16-byte chunks per lane: H <= 16 * 5 * 32 = 2560
constexpr int kGuActPerBlock = 8 * kGuRows;
constexpr int kDnRows = 2;              // rows per 8-lane group in down
constexpr int kDnCpl = 4;               // chunks per lane: I <= 8 * 4 * 32 = 1024
constexpr int kDnRowsPerBlock = 32 * kDnRows;
constexpr int kHMax = 2560;
constexpr int kIMax = 1024;

struct UnionInfo {
  int n;              // slots in use
  int n_routed_slots; // distinct valid routed ids
  unsigned bad;       // bit m set: token m holds an id outside [0, n_routed)
  int id[kMaxSlots];
  unsigned mask[kMaxSlots];  // bit m set: token m uses the slot
};

// Built by wave 0 (threads 0..63) of every workgroup from the device-resident routing.
__device__ void build_union(const int* __restrict__ idx, int M, int K, int n_routed, int has_shared,
                            UnionInfo* un) {
  const int lane = threadIdx.x;
  const int n = M * K;
  const int e = lane < n ? idx[lane] : -1;
  const bool valid = lane < n && e >= 0 && e < n_routed;
  bool first = valid;
  unsigned mask = 0;
  for (int i = 0; i < n; ++i) {
    int ei = __shfl(e, i, kWave);
    if (ei == e) {
      if (i < lane) first = false;
      mask |= 1u << (i / K);
    }
  }
  const unsigned long long firsts = __ballot(first);
  int rank = 0;
  for (int i = 0; i < n; ++i) {
    int ei = __shfl(e, i, kWave);
    if (((firsts >> i) & 1ull) && ei < e) ++rank;
  }
  if (first) {
    un->id[rank] = e;
    un->mask[rank] = mask;
  }
  const unsigned long long bad = __ballot(lane < n && !valid);
  if (lane == 0) {
    unsigned bt = 0;
    for (int i = 0; i < n; ++i)
      if ((bad >> i) & 1ull) bt |= 1u << (i / K);
    const int nr = __popcll(firsts);
    un->n_routed_slots = nr;
    un->bad = bt;
    if (has_shared) {
      un->id[nr] = n_routed;
      un->mask[nr] = (1u << M) - 1u;
    }
    un->n = nr + (has_shared ? 1 : 0);
  }
}

template <int M>
__global__ __launch_bounds__(kBlock) void gate_up_swiglu_kernel(
    const uint8_t* __restrict__ gq, const uint8_t* __restrict__ gs, int n_routed, int has_shared, int H,
    int I, const uint16_t* __restrict__ x, const int* __restrict__ idx, int K, float* __restrict__ act) {
  __shared__ UnionInfo un;
  __shared__ __attribute__((aligned(16))) uint16_t xs[M * kHMax];
  const int tid = threadIdx.x;
  if (tid < kWave) build_union(idx, M, K, n_routed, has_shared, &un);
  __syncthreads();
  const int slot = blockIdx.y;
  if (slot >= un.n) return;
  const int e = un.id[slot];
  const unsigned mask = un.mask[slot];

  const int g = tid >> 4, j = tid & 15;
  const int is_up = g & 1;
  const int i0 = blockIdx.x * kGuActPerBlock + (g >> 1) * kGuRows;
  const int nch = H >> 5;
  const size_t row_bytes = (size_t)(H >> 1);
  const size_t exp_rows = 2 * (size_t)I;

  // 1. issue every weight load of this lane first
  u32x4_t wq[kGuRows][kGuCpl];
  uint32_t wsc[kGuRows][kGuCpl];
#pragma unroll
  for (int r = 0; r < kGuRows; ++r) {
    const int i = i0 + r;
    const size_t row = (size_t)e * exp_rows + (size_t)(i + is_up * I);
#pragma unroll
    for (int t = 0; t < kGuCpl; ++t) {
      const int c = j + 16 * t;
      if (i < I && c < nch) {
        wq[r][t] = ld16(gq + row * row_bytes + (size_t)c * 16);
        wsc[r][t] = gs[row * nch + c];
      } else {
        wq[r][t] = u32x4_t{0, 0, 0, 0};
        wsc[r][t] = 127;
      }
    }
  }
  // 2. stage the token vectors in LDS
  for (int v = tid; v < M * H / 8; v += kBlock)
    *reinterpret_cast<u32x4_t*>(xs + v * 8) = ld16(x + (size_t)v * 8);
  __syncthreads();

  // 3. dequantise (e2m1 x 2^s -> bf16, exact) and dot with every token that uses this expert
  float acc[kGuRows][M];
#pragma unroll
  for (int r = 0; r < kGuRows; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
#pragma unroll
  for (int t = 0; t < kGuCpl; ++t) {
    const int c = j + 16 * t;
    if (c < nch) {
      u32x4_t xv[M][4];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xv[m][q] = *reinterpret_cast<const u32x4_t*>(xs + m * H + c * 32 + q * 8);
#pragma unroll
      for (int r = 0; r < kGuRows; ++r) {
        const float sc = e8m0_to_f32(wsc[r][t]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = wq[r][t][d];
          const bf16x2_t p0 = fp4x2_to_bf16x2<0>(wd, sc);
          const bf16x2_t p1 = fp4x2_to_bf16x2<1>(wd, sc);
          const bf16x2_t p2 = fp4x2_to_bf16x2<2>(wd, sc);
          const bf16x2_t p3 = fp4x2_to_bf16x2<3>(wd, sc);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            if ((mask >> m) & 1u) {
              float a = acc[r][m];
              a = dot2(p0, as_bf16x2(xv[m][d][0]), a);
              a = dot2(p1, as_bf16x2(xv[m][d][1]), a);
              a = dot2(p2, as_bf16x2(xv[m][d][2]), a);
              a = dot2(p3, as_bf16x2(xv[m][d][3]), a);
              acc[r][m] = a;
            }
          }
        }
      }
    }
  }
  // 4. reduce over the 16 lanes, meet the partner row, SwiGLU, store fp32 activations
#pragma unroll
  for (int r = 0; r < kGuRows; ++r) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float h = group_sum<16>(acc[r][m]);
      const float partner = __shfl_xor(h, 16, kWave);
      const int i = i0 + r;
      if (!is_up && j == r && i < I && ((mask >> m) & 1u))
        act[((size_t)slot * M + m) * I + i] = silu(h) * partner;
    }
  }
}

template <int M>
__global__ __launch_bounds__(kBlock) void down_combine_kernel(
    const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds, int n_routed, int has_shared, int H,
    int I, const int* __restrict__ idx, const float* __restrict__ tw, int K, const float* __restrict__ act,
    float* __restrict__ partial, unsigned* __restrict__ counters, float* __restrict__ y32,
    uint16_t* __restrict__ y16) {
  __shared__ UnionInfo un;
  __shared__ float wt[M];
  __shared__ __attribute__((aligned(16))) float as[M * kIMax];
  __shared__ bool last_flag;
  const int tid = threadIdx.x;
  if (tid < kWave) build_union(idx, M, K, n_routed, has_shared, &un);
  __syncthreads();
  const int slot = blockIdx.y;
  const int row0 = blockIdx.x * kDnRowsPerBlock;
  if (un.n == 0) {  // every token routed only to invalid ids and there is no shared expert
    if (slot == 0)
      for (int p = tid; p < M * kDnRowsPerBlock; p += kBlock) {
        const int m = p / kDnRowsPerBlock, row = row0 + p % kDnRowsPerBlock;
        if (row < H) {
          if (y32) y32[(size_t)m * H + row] = __uint_as_float(0x7fc00000u);
          if (y16) y16[(size_t)m * H + row] = 0x7fc0;
        }
      }
    return;
  }
  if (slot >= un.n) return;
  const int e = un.id[slot];
  const unsigned mask = un.mask[slot];
  const bool shared_slot = has_shared && slot == un.n_routed_slots;
  if (tid < M) {
    float s = 0.0f;
    if (shared_slot) {
      s = 1.0f;
    } else {
      for (int k = 0; k < K; ++k)
        if (idx[tid * K + k] == e) s += tw[tid * K + k];
    }
    wt[tid] = s;
  }

  const int g = tid >> 3, j = tid & 7;
  const int nch = I >> 5;
  const size_t row_bytes = (size_t)(I >> 1);

  u32x4_t wq[kDnRows][kDnCpl];
  uint32_t wsc[kDnRows][kDnCpl];
#pragma unroll
  for (int r = 0; r < kDnRows; ++r) {
    const int row = row0 + r * 32 + g;
    const size_t grow = (size_t)e * H + row;
#pragma unroll
    for (int t = 0; t < kDnCpl; ++t) {
      const int c = j + 8 * t;
      if (row < H && c < nch) {
        wq[r][t] = ld16(dq + grow * row_bytes + (size_t)c * 16);
        wsc[r][t] = ds[grow * nch + c];
      } else {
        wq[r][t] = u32x4_t{0, 0, 0, 0};
        wsc[r][t] = 127;
      }
    }
  }
  {
    const float* src = act + (size_t)slot * M * I;
    for (int v = tid; v < M * I / 4; v += kBlock) {
      const int m = (v * 4) / I;
      if ((mask >> m) & 1u) *reinterpret_cast<u32x4_t*>(as + v * 4) = ld16(src + (size_t)v * 4);
    }
  }
  __syncthreads();

  float acc[kDnRows][M];
#pragma unroll
  for (int r = 0; r < kDnRows; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
#pragma unroll
  for (int t = 0; t < kDnCpl; ++t) {
    const int c = j + 8 * t;
    if (c < nch) {
      float wf[kDnRows][32];
#pragma unroll
      for (int r = 0; r < kDnRows; ++r) {
        const float sc = e8m0_to_f32(wsc[r][t]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = wq[r][t][d];
          const f32x2_t p0 = fp4x2_to_f32x2<0>(wd, sc);
          const f32x2_t p1 = fp4x2_to_f32x2<1>(wd, sc);
          const f32x2_t p2 = fp4x2_to_f32x2<2>(wd, sc);
          const f32x2_t p3 = fp4x2_to_f32x2<3>(wd, sc);
          wf[r][8 * d + 0] = p0.x; wf[r][8 * d + 1] = p0.y;
          wf[r][8 * d + 2] = p1.x; wf[r][8 * d + 3] = p1.y;
          wf[r][8 * d + 4] = p2.x; wf[r][8 * d + 5] = p2.y;
          wf[r][8 * d + 6] = p3.x; wf[r][8 * d + 7] = p3.y;
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if ((mask >> m) & 1u) {
          const float* ap = as + m * I + c * 32;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float4 a4 = *reinterpret_cast<const float4*>(ap + q * 4);
#pragma unroll
            for (int r = 0; r < kDnRows; ++r) {
              float s = acc[r][m];
              s = fmaf(wf[r][4 * q + 0], a4.x, s);
              s = fmaf(wf[r][4 * q + 1], a4.y, s);
              s = fmaf(wf[r][4 * q + 2], a4.z, s);
              s = fmaf(wf[r][4 * q + 3], a4.w, s);
              acc[r][m] = s;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kDnRows; ++r) {
    const int row = row0 + r * 32 + g;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v = group_sum<8>(acc[r][m]);
      if (j == 0 && row < H && ((mask >> m) & 1u)) st_coherent(partial + ((size_t)slot * M + m) * H + row, wt[m] * v);
    }
  }

  if (!arrive_last(counters + blockIdx.x, (unsigned)un.n, &last_flag)) return;
  for (int p = tid; p < M * kDnRowsPerBlock; p += kBlock) {
    const int m = p / kDnRowsPerBlock, row = row0 + p % kDnRowsPerBlock;
    if (row >= H) continue;
    float s = 0.0f;
    for (int u = 0; u < un.n; ++u)
      if ((un.mask[u] >> m) & 1u) s += ld_coherent(partial + ((size_t)u * M + m) * H + row);
    if ((un.bad >> m) & 1u) s = __uint_as_float(0x7fc00000u);
    if (y32) y32[(size_t)m * H + row] = s;
    if (y16) y16[(size_t)m * H + row] = f32_to_bf16_rne(s);
  }
}

struct Workspace {
  float* act;
  float* partial;
  unsigned* counters;
};

size_t workspace_layout(int M, int K, int H, int I, char* base, Workspace* w) {
  const size_t slots = (size_t)M * K + 1;
  const size_t a = qws_host::align256(slots * M * I * sizeof(float));
  const size_t p = qws_host::align256(slots * M * H * sizeof(float));
  const size_t c = qws_host::align256((size_t)((H + kDnRowsPerBlock - 1) / kDnRowsPerBlock) * sizeof(unsigned));
  if (w) {
    w->act = reinterpret_cast<float*>(base);
    w->partial = reinterpret_cast<float*>(base + a);
    w->counters = reinterpret_cast<unsigned*>(base + a + p);
  }
  return a + p + c;
}

template <int M>
void launch(const qws_mxfp4_experts* w, const uint16_t* x, const int* idx, const float* tw, int K,
            uint16_t* y16, float* y32, const Workspace& ws, hipStream_t s) {
  const int H = w->hidden, I = w->inter;
  const int slots = M * K + (w->has_shared ? 1 : 0);
  dim3 g1((I + kGuActPerBlock - 1) / kGuActPerBlock, slots), g2((H + kDnRowsPerBlock - 1) / kDnRowsPerBlock, slots);
  hipLaunchKernelGGL(gate_up_swiglu_kernel<M>, g1, dim3(kBlock), 0, s, w->gate_up_q, w->gate_up_s, w->n_routed,
                     w->has_shared, H, I, x, idx, K, ws.act);
  hipLaunchKernelGGL(down_combine_kernel<M>, g2, dim3(kBlock), 0, s, w->down_q, w->down_s, w->n_routed,
                     w->has_shared, H, I, idx, tw, K, ws.act, ws.partial, ws.counters, y32, y16);
}

}  // namespace

extern "C" size_t moe_expert_workspace_bytes(int M, int K, int hidden, int inter) {
  if (M < 1 || M > kMaxM || K < 1 || K > kMaxK || hidden < 32 || hidden > kHMax || inter < 32 || inter > kIMax)
    return 0;
  return workspace_layout(M, K, hidden, inter, nullptr, nullptr);
}

extern "C" int moe_expert_gemv_mxfp4(const qws_mxfp4_experts* w, const void* x_bf16, int M, const int* topk_idx,
                                     const float* topk_w, int K, void* y_bf16, float* y_f32, void* workspace,
                                     size_t workspace_bytes, qws_stream_t stream) {
  if (!w || !x_bf16 || !topk_idx || !topk_w || (!y_bf16 && !y_f32)) return QWS_ERR_ARG;
  if (w->format != QWS_FMT_MXFP4_E2M1_E8M0_B32) return QWS_ERR_FORMAT;
  if (!w->gate_up_q || !w->gate_up_s || !w->down_q || !w->down_s) return QWS_ERR_ARG;
  if (w->has_shared != 0 && w->has_shared != 1) return QWS_ERR_ARG;
  if (w->n_routed < 1 || w->n_routed > 1024) return QWS_ERR_SHAPE;
  if (w->hidden < 32 || w->hidden > kHMax || w->hidden % 32) return QWS_ERR_SHAPE;
  if (w->inter < 32 || w->inter > kIMax || w->inter % 32) return QWS_ERR_SHAPE;
  if (M < 1 || M > kMaxM || K < 1 || K > kMaxK) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(x_bf16) || !qws_host::aligned16(w->gate_up_q) || !qws_host::aligned16(w->down_q))
    return QWS_ERR_ALIGN;
  if (!workspace || workspace_bytes < moe_expert_workspace_bytes(M, K, w->hidden, w->inter)) return QWS_ERR_WORKSPACE;
  if (!qws_host::aligned16(workspace)) return QWS_ERR_ALIGN;

  Workspace ws;
  workspace_layout(M, K, w->hidden, w->inter, static_cast<char*>(workspace), &ws);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint16_t* y16 = static_cast<uint16_t*>(y_bf16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (M) {
    case 1: launch<1>(w, x, topk_idx, topk_w, K, y16, y_f32, ws, s); break;
    case 2: launch<2>(w, x, topk_idx, topk_w, K, y16, y_f32, ws, s); break;
    case 3: launch<3>(w, x, topk_idx, topk_w, K, y16, y_f32, ws, s); break;
    default: launch<4>(w, x, topk_idx, topk_w, K, y16, y_f32, ws, s); break;
  }
  return qws_host::check_launch();
}
