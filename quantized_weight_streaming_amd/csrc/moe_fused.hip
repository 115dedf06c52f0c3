// Host side of the fused MoE layer(s) (moe_fused_kernel.hpp holds the device code and its design
// notes): the task-major pack, workspace layout, launch configuration and the C entry points.
#include "moe_fused_kernel.hpp"

namespace {

using namespace qws;
using namespace qws_moe;

// ------------------------------------------------------------------------------ task-major pack
// One thread per 16-byte piece (expert e, block j, piece p, wave w, lane l) of the task records;
// it gathers the piece's bytes from the canonical bank (the layout is stated where
// moe_pack_mxfp4 is declared). Bytes past H stay zero.
__global__ void pack_tasks_kernel(const uint8_t* __restrict__ gq, const uint8_t* __restrict__ gs,
                                  const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds, long long n_pieces,
                                  int H, int I, uint8_t* __restrict__ out) {
  const int J = I / kBlk, nch = H / 32;
  const long long gu_row = H / 2, gu_srow = nch, dn_row = I / 2, dn_srow = J;
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < n_pieces;
       x += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(x % kWave), w = (int)((x / kWave) % kWaves), p = (int)((x / kThreads) % kPieces);
    const long long task = x / ((long long)kPieces * kThreads);
    const long long e = task / J;
    const int j = (int)(task - e * J);
    const int g = lane >> 4, i = lane & 15, rg = w >> 2, ks = w & 3;
    // gate/up row of this lane and its chunk for step t
    const long long grow = e * 2 * I + (rg >= 2 ? I : 0) + (long long)kBlk * j + 16 * (rg & 1) + i;
    auto gu_chunk = [&](int t) { return kGuCpk * ks + 4 * t + g; };
    // 4-byte word d (bytes 4d .. 4d+3) of down row 16 (w + 16 q) + i in block j (0 past H)
    auto down_word = [&](int q, int d) -> uint32_t {
      const int row = 16 * (w + kWaves * q) + i;
      if (q >= kDnTpw || row >= H) return 0u;
      const uint8_t* src = dq + (e * H + row) * dn_row + 16 * j + 4 * d;
      return (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16) | ((uint32_t)src[3] << 24);
    };
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    if (p == 0) {
      // tiles 8, 9: lane group g holds half g >> 1 (bytes 8 (g >> 1) ..) of tile 8 + (g & 1)
      v[0] = down_word(8 + (g & 1), 2 * (g >> 1));
      v[1] = down_word(8 + (g & 1), 2 * (g >> 1) + 1);
      uint8_t tail[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int t = 0; t < kGuCpl; ++t) {
        const int c = gu_chunk(t);
        tail[t] = c < nch ? gs[grow * gu_srow + c] : 0;
      }
      for (int Q = 0; Q < 3; ++Q) {
        const int q = 4 * Q + g;       // down scale of tile q, row i
        const int row = 16 * (w + kWaves * q) + i;
        tail[5 + Q] = (q < kDnTpw && row < H) ? ds[(e * H + row) * dn_srow + j] : 0;
      }
      for (int b = 0; b < 8; ++b) v[2 + (b >> 2)] |= (uint32_t)tail[b] << (8 * (b & 3));
    } else if (p <= kGuCpl) {
      const int c = gu_chunk(p - 1);
      if (c < nch) {
        const uint8_t* src = gq + grow * gu_row + 16 * c;
        for (int b = 0; b < 16; ++b) v[b >> 2] |= (uint32_t)src[b] << (8 * (b & 3));
      }
    } else {
      // row i of tile 4 (p - 6) + g, all 16 bytes
      for (int d = 0; d < 4; ++d) v[d] = down_word(4 * (p - kGuCpl - 1) + g, d);
    }
    *reinterpret_cast<u32x4_t*>(out + x * 16) = u32x4_t{v[0], v[1], v[2], v[3]};
  }
}

// ------------------------------------------------------------------------------ host side
int g_grid[64];       // workgroups per launch, per device (one per CU)
unsigned long long* g_trace[64];  // per device: trace buffer registered by qws_debug_trace_buffer
size_t g_trace_bytes[64];
float* g_act[64];                 // per device: activation buffer registered by qws_debug_w4a8_act_buffer
size_t g_act_bytes[64];
constexpr size_t kMaxDynLds = 160 * 1024 - 16 * 1024;

size_t lds_bytes(int M, int E, int H, int P, int J, int nrw) {
  // scratch: selection keys, then a task's gate/up sums and activation parts, then the combine's
  // per-wave row sums
  // (per token: E candidates, 64 slots written by the lanes without a candidate, and the count;
  // several tokens: then their keys [M][E] u32)
  const size_t sel = (size_t)M * (E + kWave + 1) * 8 + (M > 1 ? (size_t)M * E * 4 : 0), gu = (size_t)4 * M * 64 * 4 + M * 4 * 32 * 2;
  const size_t comb = (size_t)kWaves * M * kLine * 4;
  const size_t scratch = sel > comb ? (sel > gu ? sel : gu) : (comb > gu ? comb : gu);
  const size_t x8 = (size_t)2 * M * H + (((size_t)2 * M * (H / 32) + 15) & ~(size_t)15);   // FP8 parts of x, scales
  return (size_t)M * H * 2 + (size_t)nrw * H * 2 + x8 + scratch;
}

// n words rounded up to whole 128-byte lines
constexpr int line_words(int n) { return (n + kLine - 1) / kLine * kLine; }

size_t ws_layout(int M, int K, int E, int H, int I, char* base, Work* w) {
  const size_t sync = qws_host::align256(kSyncCounters * kSyncStride * 8);
  const size_t misc = 256;   // launch counter, error count
  // sized for the largest grid and per-workgroup strides (kWaves router rows, kMaxRows owned
  // rows); the partial sums for every (pair, block) line of H rows
  (void)E;
  const size_t lg = qws_host::align256((size_t)kMaxE * kLine * 8);
  const size_t yt = qws_host::align256((size_t)kMaxGrid * line_words(M * kMaxRows / 2) * 8);   // one copy
  const size_t dn = qws_host::align256((size_t)kReplicas * kMaxGrid * kLine * 8);
  const size_t part = qws_host::align256((size_t)M * (K + 1) * (I / kBlk) * H * 8);
  if (w) {
    w->trace = nullptr;
    w->sync = reinterpret_cast<unsigned long long*>(base);
    w->launches = reinterpret_cast<unsigned long long*>(base + sync);
    w->errors = reinterpret_cast<unsigned*>(base + sync + 128);
    w->abort = reinterpret_cast<unsigned long long*>(base + sync + 192);
    w->launch1 = 0;
    w->logits = reinterpret_cast<unsigned long long*>(base + sync + misc);
    w->ytag = reinterpret_cast<unsigned long long*>(base + sync + misc + lg);
    w->done = reinterpret_cast<unsigned long long*>(base + sync + misc + lg + yt);
    w->partial = reinterpret_cast<unsigned long long*>(base + sync + misc + lg + yt + dn);
    w->ytag_more = reinterpret_cast<unsigned long long*>(base + sync + misc + lg + yt + dn + part);
    // the odd layers' logits of a chained sequence: one token's copies fill half of the logits area
    // (kReplicas x kMaxE words of kMaxE x kLine), the other half takes them; several tokens need a
    // second area, after the rest (the other buffers keep their places either way)
    w->logits_odd = M == 1 ? w->logits + (size_t)kReplicas * kMaxE
                           : reinterpret_cast<unsigned long long*>(base + sync + misc + lg + yt + dn + part + (kReplicas - 1) * yt);
  }
  static_assert(2 * kReplicas * kMaxE <= kMaxE * kLine, "both one-token logits buffers fit the logits area");
  return sync + misc + lg + yt + dn + part + (kReplicas - 1) * yt + (M == 1 ? 0 : lg);
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
  if (x.format != QWS_FMT_MXFP4_E2M1_E8M0_B32_TASKMAJOR) return QWS_ERR_FORMAT;
  if (!x.gate_up_q) return QWS_ERR_ARG;
  if (x.n_routed != E || x.hidden != H || x.inter != I || x.has_shared != has_shared) return QWS_ERR_SHAPE;
  if (d.bias && !(d.bias_row_stride == 0 || d.bias_row_stride == E)) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(d.x_bf16) || !qws_host::aligned16(d.w_router_bf16) || !qws_host::aligned16(x.gate_up_q))
    return QWS_ERR_ALIGN;
  return QWS_OK;
}

template <int M, bool A8, bool CH>
int launch(const Layer& first, const qws_moe_layer* rest, int n, const Shape& sh, const Work& w, int G, size_t lds,
           hipStream_t s) {
  static bool configured[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (!configured[dev]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_layers_kernel<M, A8, CH>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxDynLds);
    if (e != hipSuccess) return qws_host::set_device_error(e);
    configured[dev] = true;
  }
  // the in-kernel hand-offs need every workgroup resident at once: one per compute unit
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_layers_kernel<M, A8, CH>, kThreads, lds);
  if (e != hipSuccess) return qws_host::set_device_error(e);
  if (per_cu < 1) return QWS_ERR_SHAPE;
  hipLaunchKernelGGL((moe_layers_kernel<M, A8, CH>), dim3(G), dim3(kThreads), lds, s, first, rest, n, sh, w);
  return qws_host::check_launch();
}

template <int M, bool A8>
int launch_kind(const Layer& first, const qws_moe_layer* rest, int n, const Shape& sh, const Work& w, int G,
                size_t lds, hipStream_t s) {
  return sh.chained ? launch<M, A8, true>(first, rest, n, sh, w, G, lds, s)
                    : launch<M, A8, false>(first, rest, n, sh, w, G, lds, s);
}

// The run-time-compiled kernel for this launch's M, precision and layer shape, launched with the
// same arguments as the template build's.
int launch_rtc(const Layer& first, const qws_moe_layer* rest, int n, const Shape& sh, const Work& w, int G,
               size_t lds, hipStream_t s, int M, bool a8, const char* cache_dir) {
  void* fn = nullptr;
  int st = qws_host::moe_rtc_function(M, a8, sh.chained != 0, sh.K, sh.E, sh.H, sh.I, sh.has_shared, cache_dir, &fn);
  if (st != QWS_OK) return st;
  int per_cu = 0;
  hipError_t e = hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, static_cast<hipFunction_t>(fn), kThreads,
                                                                      lds);
  if (e != hipSuccess) return qws_host::set_device_error(e);
  if (per_cu < 1) return QWS_ERR_SHAPE;
  Layer a0 = first;
  const qws_moe_layer* a1 = rest;
  int a2 = n;
  Shape a3 = sh;
  Work a4 = w;
  void* args[] = {&a0, &a1, &a2, &a3, &a4};
  e = hipModuleLaunchKernel(static_cast<hipFunction_t>(fn), G, 1, 1, kThreads, 1, 1, (unsigned)lds, s, args, nullptr);
  return e == hipSuccess ? QWS_OK : qws_host::set_device_error(e);
}

int run_layers(const qws_moe_layer* host, const qws_moe_layer* dev_copy, int n_layers, int M, int K,
               void* workspace, size_t workspace_bytes, qws_stream_t stream, bool a8, bool rtc = false,
               const char* rtc_dir = nullptr) {
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
  // rows per owner: even, so that a thread writes a bf16 pair of one token
  const int R_all = ((H + G - 1) / G + 1) & ~1;   // every workgroup owns rows
  if (G > kMaxGrid || G < J || nrw > kCopyWaves || R_all > kMaxRows) return QWS_ERR_SHAPE;
  const int P = M * (K + 1);
  const size_t lds = lds_bytes(M, E, H, P, J, nrw);
  if (lds > kMaxDynLds) return QWS_ERR_SHAPE;
  // Chained: layer l+1 reads y of layer l. Then the layers need no barrier, provided every
  // workgroup computes router rows, so that no workgroup can fall a layer behind the others (each
  // layer waits for every workgroup's logits); the logits alternate between two buffers, so that
  // a workgroup that owns no rows may still read layer l's while the others write layer l+1's.
  bool chained = n_layers > 1 && E >= G;
  for (int l = 0; chained && l + 1 < n_layers; ++l)
    chained = host[l].y_bf16 != nullptr && host[l + 1].x_bf16 == host[l].y_bf16;
  // An owner takes one whole 128-byte line of every partial-sum vector (kLine rows, when the grid
  // has owners for all of them): it reads no line another owner also reads.
  const int R = (size_t)G * kLine >= (size_t)H ? kLine : R_all;
  Work w;
  ws_layout(M, K, E, H, I, static_cast<char*>(workspace), &w);
  {
    int dev = 0;
    (void)hipGetDevice(&dev);
    const size_t need = (size_t)n_layers * G * kTracePoints * 8;
    w.trace = (dev >= 0 && dev < 64 && g_trace[dev] && g_trace_bytes[dev] >= need) ? g_trace[dev] : nullptr;
    const size_t na = (size_t)(E + 1) * M * I, need_act = na * 5 + na / kBlk;
    w.act = (a8 && n_layers == 1 && dev >= 0 && dev < 64 && g_act[dev] && g_act_bytes[dev] >= need_act) ? g_act[dev]
                                                                                                       : nullptr;
  }
  // x_fresh: no layer's x overlaps an output of any layer of this launch (all x were written before it)
  bool x_fresh = !chained;
  {
    auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
      const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
      return a && b && pa < pb + nb && pb < pa + na;
    };
    for (int l = 1; x_fresh && l < n_layers; ++l) {
      const size_t nx = (size_t)M * H * 2;
      for (int o = 0; x_fresh && o < n_layers; ++o) {
        const qws_moe_layer& d = host[o];
        if (overlap(host[l].x_bf16, nx, d.y_bf16, (size_t)M * H * 2) ||
            overlap(host[l].x_bf16, nx, d.y_f32, (size_t)M * H * 4) ||
            overlap(host[l].x_bf16, nx, d.topk_idx, (size_t)M * K * 4) ||
            overlap(host[l].x_bf16, nx, d.topk_w, (size_t)M * K * 4) ||
            overlap(host[l].x_bf16, nx, d.logits_out, (size_t)M * E * 4))
          x_fresh = false;
      }
    }
  }
  const Shape sh{E, K, H, I, hs, R, P, chained ? 1 : 0, nrw, 1.0f / (float)R, line_words(M * R / 2),
                 x_fresh ? 1 : 0, J};
  const Layer first = to_layer(host[0]);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (rtc) return launch_rtc(first, dev_copy, n_layers, sh, w, G, lds, s, M, a8, rtc_dir);
  if (a8) {
    switch (M) {
      case 1: return launch_kind<1, true>(first, dev_copy, n_layers, sh, w, G, lds, s);
      case 2: return launch_kind<2, true>(first, dev_copy, n_layers, sh, w, G, lds, s);
      case 3: return launch_kind<3, true>(first, dev_copy, n_layers, sh, w, G, lds, s);
      default: return launch_kind<4, true>(first, dev_copy, n_layers, sh, w, G, lds, s);
    }
  }
  switch (M) {
    case 1: return launch_kind<1, false>(first, dev_copy, n_layers, sh, w, G, lds, s);
    case 2: return launch_kind<2, false>(first, dev_copy, n_layers, sh, w, G, lds, s);
    case 3: return launch_kind<3, false>(first, dev_copy, n_layers, sh, w, G, lds, s);
    default: return launch_kind<4, false>(first, dev_copy, n_layers, sh, w, G, lds, s);
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
  return run_layers(layer, nullptr, 1, M, K, workspace, workspace_bytes, stream, false);
}

extern "C" int moe_layers_mxfp4(const qws_moe_layer* layers_host, const qws_moe_layer* layers_device, int n_layers,
                                int M, int K, void* workspace, size_t workspace_bytes, qws_stream_t stream) {
  return run_layers(layers_host, layers_device, n_layers, M, K, workspace, workspace_bytes, stream, false);
}

extern "C" int moe_layer_w4a8(const qws_moe_layer* layer, int M, int K, void* workspace, size_t workspace_bytes,
                              qws_stream_t stream) {
  return run_layers(layer, nullptr, 1, M, K, workspace, workspace_bytes, stream, true);
}

extern "C" int moe_layers_w4a8(const qws_moe_layer* layers_host, const qws_moe_layer* layers_device, int n_layers,
                               int M, int K, void* workspace, size_t workspace_bytes, qws_stream_t stream) {
  return run_layers(layers_host, layers_device, n_layers, M, K, workspace, workspace_bytes, stream, true);
}

extern "C" int moe_layers_rtc(const qws_moe_layer* layers_host, const qws_moe_layer* layers_device, int n_layers,
                              int M, int K, int w4a8, void* workspace, size_t workspace_bytes, const char* cache_dir,
                              qws_stream_t stream) {
  if (w4a8 != 0 && w4a8 != 1) return QWS_ERR_ARG;
  return run_layers(layers_host, layers_device, n_layers, M, K, workspace, workspace_bytes, stream, w4a8 != 0, true,
                    cache_dir);
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

extern "C" size_t moe_pack_mxfp4_bytes(int n_experts, int hidden, int inter) {
  if (n_experts < 1 || n_experts > kMaxE + 1) return 0;
  if (hidden < 32 || hidden > kHMax || hidden % 32 || inter < 32 || inter > kIMax || inter % 32) return 0;
  return (size_t)n_experts * (inter / kBlk) * kTaskBytes;
}

extern "C" int moe_pack_mxfp4(const qws_mxfp4_experts* src, unsigned char* out, size_t out_bytes,
                              qws_mxfp4_experts* desc_out, qws_stream_t stream) {
  if (!src || !out || !desc_out) return QWS_ERR_ARG;
  if (src->format != QWS_FMT_MXFP4_E2M1_E8M0_B32) return QWS_ERR_FORMAT;
  if (!src->gate_up_q || !src->gate_up_s || !src->down_q || !src->down_s) return QWS_ERR_ARG;
  if (src->has_shared != 0 && src->has_shared != 1) return QWS_ERR_ARG;
  if (src->n_routed < 1 || src->n_routed > kMaxE) return QWS_ERR_SHAPE;
  const int n = src->n_routed + src->has_shared, H = src->hidden, I = src->inter;
  const size_t need = moe_pack_mxfp4_bytes(n, H, I);
  if (need == 0) return QWS_ERR_SHAPE;
  if (out_bytes < need) return QWS_ERR_WORKSPACE;
  if (!qws_host::aligned16(out)) return QWS_ERR_ALIGN;
  const long long pieces = (long long)(need / 16);
  const long long want = (pieces + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_tasks_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), src->gate_up_q,
                     src->gate_up_s, src->down_q, src->down_s, pieces, H, I, out);
  const int st = qws_host::check_launch();
  if (st == QWS_OK) {
    *desc_out = *src;
    desc_out->format = QWS_FMT_MXFP4_E2M1_E8M0_B32_TASKMAJOR;
    desc_out->gate_up_q = out;
    desc_out->gate_up_s = nullptr;
    desc_out->down_q = nullptr;
    desc_out->down_s = nullptr;
  }
  return st;
}

extern "C" int qws_debug_w4a8_act_buffer(void* buf, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return qws_host::set_device_error(e);
  if (dev < 0 || dev >= 64) return QWS_ERR_DEVICE;
  if (buf && !qws_host::aligned16(buf)) return QWS_ERR_ALIGN;
  g_act[dev] = static_cast<float*>(buf);
  g_act_bytes[dev] = buf ? bytes : 0;
  return QWS_OK;
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
