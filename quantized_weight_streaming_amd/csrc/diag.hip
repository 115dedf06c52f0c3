// Diagnostics and status plumbing of libqws: startup self-check of the device format routines,
// debug dequantisation through the exact routines the GEMVs use, a streaming-read bandwidth
// probe, and status strings.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "qws_common.hpp"

namespace {

using namespace qws;

thread_local char g_err[512];

// --------------------------------------------------------------------------- host tables
// e2m1: bit 3 sign, bits 2:1 exponent (bias 1), bit 0 mantissa; exponent 0 is subnormal.
float host_e2m1(int c) {
  const int e = (c >> 1) & 3, m = c & 1;
  const float mag = e == 0 ? 0.5f * m : ldexpf(1.0f + 0.5f * m, e - 1);
  return (c & 8) ? -mag : mag;
}
// E4M3 (OCP "FN"): bias 7, S.1111.111 NaN, no infinities.
float host_e4m3(int c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const float mag = e == 0 ? ldexpf(m / 8.0f, -6) : ldexpf(1.0f + m / 8.0f, e - 7);
  return (c & 0x80) ? -mag : mag;
}
// Round-to-nearest-even, saturating E4M3 encode of a finite float (for the self-check only).
int host_e4m3_encode(float v) {
  const int sign = signbit(v) ? 0x80 : 0;
  const double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) return sign | (int)nearbyint(a * 512.0);
  int ex;
  const double f = frexp(a, &ex);  // a = f * 2^ex, f in [0.5, 1)
  const int m = (int)nearbyint(16.0 * f - 8.0);
  return sign | (((ex - 1 + 7) << 3) + m);
}

constexpr int kScaleBytes[] = {2, 100, 119, 121, 123, 127, 140, 252};
constexpr int kNScales = sizeof(kScaleBytes) / sizeof(kScaleBytes[0]);
constexpr float kEncodeInputs[] = {0.0f, -0.0f, 1.0f, -1.0f, 1.0625f, 1.1875f, 1.07f, 0.0009765625f, 0.0029296875f,
                                   0.0146484375f, 0.001f, 3.0e-4f, 0.0155f, 447.9f, 448.0f, 448.0001f, 460.0f,
                                   240.5f, 17.3f, -0.3333f, 96.0f, 100.0f, 104.0f, -2.75f};
constexpr int kNEnc = sizeof(kEncodeInputs) / sizeof(kEncodeInputs[0]);

struct CheckOut {
  float fp4_f32[kNScales][16];
  float fp4_bf16[kNScales][16];
  float fp8[256];
  int enc[kNEnc];
};

__global__ void selfcheck_kernel(const int* __restrict__ scale_bytes, const float* __restrict__ enc_in,
                                 CheckOut* __restrict__ out) {
  const int t = threadIdx.x;
  if (t < kNScales * 16) {
    const int si = t / 16, c = t % 16;
    const float sc = e8m0_to_f32((uint32_t)scale_bytes[si]);
    // code c in the low nibble of byte 2 (element 0 of that pair), code 15-c in the high nibble
    const uint32_t w = (uint32_t)(c | ((15 - c) << 4)) << 16;
    const f32x2_t a = fp4x2_to_f32x2<2>(w, sc);
    const bf16x2_t b = fp4x2_to_bf16x2<2>(w, sc);
    out->fp4_f32[si][c] = a.x;
    out->fp4_bf16[si][c] = (float)b.x;
    // the high nibble must decode to code 15-c: fold a mismatch into a NaN of the low result
    const float want_hi = fp4x2_to_f32x2<0>((uint32_t)(15 - c), sc).x;
    if (__float_as_uint(a.y) != __float_as_uint(want_hi)) out->fp4_f32[si][c] = NAN;
    if (__float_as_uint((float)b.y) != __float_as_uint(want_hi)) out->fp4_bf16[si][c] = NAN;
  }
  if (t < 128) {
    // codes 2t (low byte of the high half-word) and 2t+1
    const uint32_t w = (uint32_t)(2 * t) << 16 | (uint32_t)(2 * t + 1) << 24;
    const bf16x2_t v = fp8x2_to_bf16x2<true>(w);
    out->fp8[2 * t] = (float)v.x;
    out->fp8[2 * t + 1] = (float)v.y;
  }
  if (t < kNEnc) {
    out->enc[t] = (int)(f32x2_to_e4m3x2<false>(enc_in[t], 0.0f, 0u) & 0xffu);
  }
}

bool same_bits(float a, float b) {
  if (isnan(a) || isnan(b)) return isnan(a) && isnan(b);
  uint32_t ua, ub;
  memcpy(&ua, &a, 4);
  memcpy(&ub, &b, 4);
  return ua == ub;
}

// --------------------------------------------------------------------------- debug dequant
template <int PATH>
__global__ void dequant_mxfp4_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, long long rows,
                                     int cols, float* __restrict__ out) {
  const int nch = cols >> 5;
  const long long n = rows * nch;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const long long r = i / nch;
    const int c = (int)(i % nch);
    const u32x4_t w = ld16(q + r * (cols >> 1) + (size_t)c * 16);
    const float sc = e8m0_to_f32(s[r * nch + c]);
    float v[32];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (PATH == 0) {
        const f32x2_t p0 = fp4x2_to_f32x2<0>(w[d], sc), p1 = fp4x2_to_f32x2<1>(w[d], sc);
        const f32x2_t p2 = fp4x2_to_f32x2<2>(w[d], sc), p3 = fp4x2_to_f32x2<3>(w[d], sc);
        v[8 * d + 0] = p0.x; v[8 * d + 1] = p0.y; v[8 * d + 2] = p1.x; v[8 * d + 3] = p1.y;
        v[8 * d + 4] = p2.x; v[8 * d + 5] = p2.y; v[8 * d + 6] = p3.x; v[8 * d + 7] = p3.y;
      } else {
        const bf16x2_t p0 = fp4x2_to_bf16x2<0>(w[d], sc), p1 = fp4x2_to_bf16x2<1>(w[d], sc);
        const bf16x2_t p2 = fp4x2_to_bf16x2<2>(w[d], sc), p3 = fp4x2_to_bf16x2<3>(w[d], sc);
        v[8 * d + 0] = (float)p0.x; v[8 * d + 1] = (float)p0.y; v[8 * d + 2] = (float)p1.x; v[8 * d + 3] = (float)p1.y;
        v[8 * d + 4] = (float)p2.x; v[8 * d + 5] = (float)p2.y; v[8 * d + 6] = (float)p3.x; v[8 * d + 7] = (float)p3.y;
      }
    }
    float4* o = reinterpret_cast<float4*>(out + r * cols + (size_t)c * 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

__global__ void dequant_fp8_kernel(const uint8_t* __restrict__ q, const float* __restrict__ scale, long long rows,
                                   int cols, float* __restrict__ out) {
  const int nch = cols >> 4;
  const long long n = rows * nch;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const long long r = i / nch;
    const int c = (int)(i % nch);
    // tile-major codes: tile r / 16 at byte 16 (r / 16) cols, chunk c of tile row r % 16 at 16 (16c + r % 16)
    const u32x4_t w = ld16(q + (r >> 4) * 16 * (long long)cols + (16ll * c + (r & 15)) * 16);
    const float sc = scale[r];
    float4* o = reinterpret_cast<float4*>(out + r * cols + (size_t)c * 16);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x2_t lo = fp8x2_to_bf16x2<false>(w[d]);
      const bf16x2_t hi = fp8x2_to_bf16x2<true>(w[d]);
      o[d] = make_float4(__fmul_rn((float)lo.x, sc), __fmul_rn((float)lo.y, sc), __fmul_rn((float)hi.x, sc),
                         __fmul_rn((float)hi.y, sc));
    }
  }
}

// --------------------------------------------------------------------------- read probe
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4_t* __restrict__ buf, size_t n16,
                                                         unsigned* __restrict__ sink) {
  __shared__ unsigned part[4];
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t a = buf[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Non-temporal read probe: workgroup b reads share b (contiguous, 1/gridDim of the buffer), each
// wave 4 consecutive KB per step with non-temporal loads. Measured on MI355X this is the access
// shape that streams fastest (~7.0 TB/s over 4 GiB, against ~5.9 TB/s for the grid-strided
// ordinary loads above).
__global__ __launch_bounds__(256) void probe_read_nt_kernel(const u32x4_t* __restrict__ buf, size_t n16,
                                                            unsigned* __restrict__ sink) {
  __shared__ unsigned part[4];
  constexpr int kU = 4;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t acc = 0;
  for (size_t base = b0 + (size_t)wave * kU * kWave; base < b1; base += (size_t)4 * kU * kWave) {
    u32x4_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t i = base + (size_t)u * kWave + lane;
      v[u] = i < b1 ? __builtin_nontemporal_load((const QWS_GLOBAL u32x4_t*)(buf + i)) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// --------------------------------------------------------------------------- copy probe
// A plain copy of known size: the reference point that turns the HBM traffic counters of other
// kernels into bytes (read and write both equal `bytes` here).
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                         size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

namespace qws_host {
int set_device_error(hipError_t e) {
  snprintf(g_err, sizeof(g_err), "%s", hipGetErrorString(e));
  return QWS_ERR_DEVICE;
}
int set_error_text(int status, const char* text) {
  snprintf(g_err, sizeof(g_err), "%s", text ? text : "");
  return status;
}
}  // namespace qws_host

extern "C" const char* qws_strerror(int status) {
  static thread_local char buf[640];
  const char* base = "unknown status";
  switch (status) {
    case QWS_OK: base = "ok"; break;
    case QWS_ERR_ARG: base = "invalid argument (NULL pointer, bad enum value or no output)"; break;
    case QWS_ERR_SHAPE: base = "size outside the supported range"; break;
    case QWS_ERR_ALIGN: base = "pointer not 16-byte aligned"; break;
    case QWS_ERR_FORMAT: base = "descriptor format tag does not match this entry point"; break;
    case QWS_ERR_WORKSPACE: base = "workspace missing or too small"; break;
    case QWS_ERR_DEVICE: base = "HIP runtime error"; break;
    case QWS_ERR_SELFCHECK: base = "device format self-check failed"; break;
    case QWS_ERR_COMPILE: base = "run-time compilation failed"; break;
  }
  if (status == QWS_ERR_DEVICE || status == QWS_ERR_SELFCHECK || status == QWS_ERR_COMPILE) {
    snprintf(buf, sizeof(buf), "%s: %s", base, g_err);
    return buf;
  }
  return base;
}

extern "C" int qws_abi_version(void) { return QWS_ABI_VERSION; }

extern "C" int qws_selfcheck(qws_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  CheckOut* d_out = nullptr;
  int* d_scales = nullptr;
  float* d_enc = nullptr;
  hipError_t e = hipMalloc(&d_out, sizeof(CheckOut));
  if (e == hipSuccess) e = hipMalloc(&d_scales, sizeof(kScaleBytes));
  if (e == hipSuccess) e = hipMalloc(&d_enc, sizeof(kEncodeInputs));
  CheckOut h;
  if (e == hipSuccess) e = hipMemcpyAsync(d_scales, kScaleBytes, sizeof(kScaleBytes), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(d_enc, kEncodeInputs, sizeof(kEncodeInputs), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(selfcheck_kernel, dim3(1), dim3(256), 0, s, d_scales, d_enc, d_out);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipMemcpyAsync(&h, d_out, sizeof(CheckOut), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(d_out);
  (void)hipFree(d_scales);
  (void)hipFree(d_enc);
  if (e != hipSuccess) return qws_host::set_device_error(e);

  int bad = 0;
  char first[256] = "";
  for (int si = 0; si < kNScales; ++si)
    for (int c = 0; c < 16; ++c) {
      const float want = host_e2m1(c) * ldexpf(1.0f, kScaleBytes[si] - 127);
      if (!same_bits(h.fp4_f32[si][c], want) || !same_bits(h.fp4_bf16[si][c], want)) {
        if (!bad++) snprintf(first, sizeof(first), "e2m1 code %d scale byte %d: got %g / %g want %g", c, kScaleBytes[si],
                             h.fp4_f32[si][c], h.fp4_bf16[si][c], want);
      }
    }
  for (int c = 0; c < 256; ++c)
    if (!same_bits(h.fp8[c], host_e4m3(c))) {
      if (!bad++) snprintf(first, sizeof(first), "e4m3 code 0x%02x: got %g want %g", c, h.fp8[c], host_e4m3(c));
    }
  for (int i = 0; i < kNEnc; ++i)
    if (h.enc[i] != host_e4m3_encode(kEncodeInputs[i])) {
      if (!bad++) snprintf(first, sizeof(first), "e4m3 encode %.9g: got 0x%02x want 0x%02x", kEncodeInputs[i], h.enc[i],
                           host_e4m3_encode(kEncodeInputs[i]));
    }
  if (bad) {
    snprintf(g_err, sizeof(g_err), "%d mismatches; first: %s", bad, first);
    return QWS_ERR_SELFCHECK;
  }
  return QWS_OK;
}

extern "C" int qws_debug_dequant_mxfp4(const unsigned char* q, const unsigned char* s, long long rows, int cols,
                                       int path, float* out, qws_stream_t stream) {
  if (!q || !s || !out) return QWS_ERR_ARG;
  if (path != 0 && path != 1) return QWS_ERR_ARG;
  if (rows < 1 || cols < 32 || cols > 65536 || cols % 32) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(q) || !qws_host::aligned16(out)) return QWS_ERR_ALIGN;
  const long long n = rows * (cols / 32);
  const int blocks = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (path == 0)
    hipLaunchKernelGGL(dequant_mxfp4_kernel<0>, dim3(blocks), dim3(256), 0, st, q, s, rows, cols, out);
  else
    hipLaunchKernelGGL(dequant_mxfp4_kernel<1>, dim3(blocks), dim3(256), 0, st, q, s, rows, cols, out);
  return qws_host::check_launch();
}

extern "C" int qws_debug_dequant_fp8(const qws_lmhead* head, float* out, qws_stream_t stream) {
  if (!head || !head->w || !out) return QWS_ERR_ARG;
  if (head->format != QWS_FMT_FP8_E4M3FN_ROWSCALE_T16) return QWS_ERR_FORMAT;
  if (!head->row_scale) return QWS_ERR_ARG;
  if (head->rows < 1 || head->cols < 32 || head->cols > 65536 || head->cols % 32) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(head->w) || !qws_host::aligned16(out)) return QWS_ERR_ALIGN;
  const long long n = head->rows * (head->cols / 16);
  const int blocks = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  hipLaunchKernelGGL(dequant_fp8_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(head->w), head->row_scale, head->rows, (int)head->cols, out);
  return qws_host::check_launch();
}

extern "C" int qws_probe_read(const void* buf, size_t bytes, unsigned* sink, int blocks, qws_stream_t stream) {
  if (!buf || !sink) return QWS_ERR_ARG;
  if (bytes == 0 || bytes % 16 || blocks < 1 || blocks > 65536) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(buf)) return QWS_ERR_ALIGN;
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return qws_host::check_launch();
}

extern "C" int qws_probe_read_nt(const void* buf, size_t bytes, unsigned* sink, int blocks, qws_stream_t stream) {
  if (!buf || !sink) return QWS_ERR_ARG;
  if (bytes == 0 || bytes % 16 || blocks < 1 || blocks > 65536) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(buf)) return QWS_ERR_ALIGN;
  hipLaunchKernelGGL(probe_read_nt_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return qws_host::check_launch();
}

extern "C" int qws_probe_copy(const void* src, void* dst, size_t bytes, int blocks, qws_stream_t stream) {
  if (!src || !dst) return QWS_ERR_ARG;
  if (bytes == 0 || bytes % 16 || blocks < 1 || blocks > 65536) return QWS_ERR_SHAPE;
  if (!qws_host::aligned16(src) || !qws_host::aligned16(dst)) return QWS_ERR_ALIGN;
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return QWS_ERR_ARG;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), bytes / 16);
  return qws_host::check_launch();
}
