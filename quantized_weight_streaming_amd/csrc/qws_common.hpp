// Shared device helpers and host-side plumbing of libqws (gfx950 only).
#pragma once

#ifndef __HIPCC_RTC__   // hipRTC (rtc.hip) compiles the device part alone, with its own runtime headers
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qws.h"
#else
typedef __hip_internal::uint8_t uint8_t;
typedef __hip_internal::uint16_t uint16_t;
typedef __hip_internal::uint32_t uint32_t;
typedef __hip_internal::int32_t int32_t;
typedef __hip_internal::uint64_t uint64_t;
#endif

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace qws {

constexpr int kWave = 64;

// ------------------------------------------------------------------------------ loads
// Every pointer these helpers take is device (global) memory. The casts state that address space
// explicitly: a pointer read from a descriptor in memory is otherwise generic, and generic
// accesses become flat instructions (no scalar base + 32-bit offset form, and they also count
// against the LDS wait counter).
#define QWS_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *(const QWS_GLOBAL u32x4_t*)p; }
template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
  return *(const QWS_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ void stg(T* p, T v) {
  *(QWS_GLOBAL T*)p = v;
}

// ------------------------------------------------------------------------------ formats
// E8M0 byte -> the float32 scale 2^(s-127). Bytes 1..254 are normal float32 exponents; byte 0 is
// 2^-127 (a float32 subnormal); byte 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t bits = s == 0 ? 0x00400000u : (s == 255 ? 0x7fc00000u : (s << 23));
  return __uint_as_float(bits);
}

// E8M0 byte 1 .. 254 -> 2^(s-127) in one shift (the scales a bank may hold); byte 0 gives 0.0,
// which the task-major records use as padding next to zero codes.
__device__ __forceinline__ float e8m0_normal_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

// Two e2m1 nibbles of byte `B` of `w`, times `scale`, as bf16x2 / float2 (element order: low
// nibble first). gfx950 converts in one VALU op.
template <int B>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, B);
}
template <int B>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, B);
}
// Two E4M3 codes of 16-bit half `H` of `w` as bf16x2 (exact: E4M3 values are bf16 values).
template <bool H>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, H);
}
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

// Two floats -> two E4M3 codes, round to nearest even and saturating at +-448, written into 16-bit
// half H of `old` (element a in the lower byte). Clamping first makes the result independent of
// how the conversion treats overflow; RNE(clamp(v)) equals saturating RNE because 448 is a code.
template <bool H>
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b, uint32_t old) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, H);
}

// acc + a.x*b.x + a.y*b.y with bf16 inputs (products exact in fp32).
__device__ __forceinline__ float dot2(bf16x2_t a, bf16x2_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

// ------------------------------------------------------------------------------ matrix cores
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// D = A (16 x 32) * B (32 x 16) + C, bf16 inputs (products exact in fp32), fp32 accumulation, one
// wave. Lane l holds A row l % 16 at k = 8 (l / 16) .. +7, B column l % 16 at the same k (8 bf16
// each, lower k in the lower half-word), and D column l % 16 at rows 4 (l / 16) .. +3.
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
// The 8 e2m1 codes of word `w` times `scale` as 8 bf16 (an MFMA operand; exact).
__device__ __forceinline__ u32x4_t fp4x8_to_bf16x8(uint32_t w, float scale) {
  return u32x4_t{__builtin_bit_cast(uint32_t, fp4x2_to_bf16x2<0>(w, scale)),
                 __builtin_bit_cast(uint32_t, fp4x2_to_bf16x2<1>(w, scale)),
                 __builtin_bit_cast(uint32_t, fp4x2_to_bf16x2<2>(w, scale)),
                 __builtin_bit_cast(uint32_t, fp4x2_to_bf16x2<3>(w, scale))};
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------------------------ reductions
// Sum over aligned groups of W lanes (W a power of two <= 64); every lane gets its group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
  return v;
}

// DPP (data-parallel primitive) lane moves: cross-lane operands without an LDS round trip.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}
// v + (the DPP-moved v), with lanes outside ROWS adding 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
// Sum over each aligned group of 16 lanes; every lane of the group gets it (quad swaps, then
// half-row and row mirrors).
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  v = dpp_add<0x140>(v);
  return v;
}
// Sum over each aligned group of 8 lanes; every lane of the group gets it.
__device__ __forceinline__ float row8_sum(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  return v;
}
// After row8_sum: each lane gets the sum of its 16-lane row (adds the other half-row's sum).
__device__ __forceinline__ float row16_sum_of_row8(float v) { return dpp_add<0x140>(v); }
// Wave-uniform sum of 64 lanes: 16-lane sums, then row 15 -> next row and lane 31 -> rows 2, 3
// broadcasts; lane 63 ends with the total. The order of additions is fixed.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v = dpp_add<0x142, 0xA>(v);
  v = dpp_add<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Wave-uniform max of a uint32 across 64 lanes.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<0xB1>(v));
  v = max(v, dpp<0x4E>(v));
  v = max(v, dpp<0x141>(v));
  v = max(v, dpp<0x140>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// The value of lane (lane ^ S) for a constant S, without the LDS: DPP for S = 1, 2 (quad
// permutes), 4 (the half-row mirror, then the quad reversal: lane 8a + 4c + d reads 8a + 4(1-c) + d)
// and 8 (rotation by 8 inside a row of 16), the lane-group swaps for S = 16 and 32. Every source
// lane of these DPP moves exists, so no lane keeps an old value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
  if constexpr (S == 1) return dpp_mov<0xB1>(v);
  else if constexpr (S == 2) return dpp_mov<0x4E>(v);
  else if constexpr (S == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(v));
  else if constexpr (S == 8) return dpp_mov<0x128>(v);
  else if constexpr (S == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);   // {(r0, r0, r2, r2), (r1, r1, r3, r3)}
    return (lane & 16) ? p[0] : p[1];
  } else {
    static_assert(S == 32, "strides 1 .. 32");
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // {(r0, r1, r0, r1), (r2, r3, r2, r3)}
    return (lane & 32) ? p[0] : p[1];
  }
}
template <int S>
__device__ __forceinline__ unsigned long long xor_lane64(unsigned long long v, int lane) {
  return (unsigned long long)xor_lane<S>((uint32_t)v, lane) | ((unsigned long long)xor_lane<S>((uint32_t)(v >> 32), lane) << 32);
}

template <int S>
__device__ __forceinline__ uint32_t xor_lane_any(uint32_t v, int lane) { return xor_lane<S>(v, lane); }
template <int S>
__device__ __forceinline__ unsigned long long xor_lane_any(unsigned long long v, int lane) {
  return xor_lane64<S>(v, lane);
}

// The largest of one 32-bit value per lane, in every lane: quad swaps, then the mirrors inside
// half-rows and rows (each lane then holds the maximum of its 8, then 16), then the lane-group swaps.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v, int lane) {
  v = max(v, dpp_mov<0xB1>(v));
  v = max(v, dpp_mov<0x4E>(v));
  v = max(v, dpp_mov<0x141>(v));
  v = max(v, dpp_mov<0x140>(v));
  v = max(v, xor_lane<16>(v, lane));
  return max(v, xor_lane<32>(v, lane));
}

// One compare-exchange stage of a bitonic network at a constant stride S: lanes whose keep_max
// holds take the larger of their key and lane (lane ^ S)'s, the others the smaller (one compare:
// the partner's key is taken when "it is larger" agrees with keep_max). Keys of 32 or 64 bits.
template <int S, typename T>
__device__ __forceinline__ T bitonic_step(T key, bool keep_max, int lane) {
  const T o = xor_lane_any<S>(key, lane);
  return (o > key) == keep_max ? o : key;
}
template <int S, typename T>
__device__ __forceinline__ T bitonic_merge_desc(T key, int size, int lane) {
  // the strides S, S/2, .. 1 of merging blocks of `size` (descending where lane & size is 0)
  key = bitonic_step<S>(key, ((lane & S) == 0) == ((lane & size) == 0), lane);
  if constexpr (S > 1) key = bitonic_merge_desc<S / 2>(key, size, lane);
  return key;
}

// Bitonic sort of one key per lane inside aligned groups of N lanes (N = 16, 32 or 64): lanes
// 0 .. N-1 end descending (lane 0 the largest); with N < 64 the other groups end sorted too, in
// either direction.
template <int N = 64, typename T = unsigned long long>
__device__ __forceinline__ T wave_sort_desc(T key, int lane) {
  static_assert(N == 16 || N == 32 || N == 64, "groups of 16, 32 or 64 lanes");
  key = bitonic_merge_desc<1>(key, 2, lane);
  key = bitonic_merge_desc<2>(key, 4, lane);
  key = bitonic_merge_desc<4>(key, 8, lane);
  key = bitonic_merge_desc<8>(key, 16, lane);
  if constexpr (N >= 32) key = bitonic_merge_desc<16>(key, 32, lane);
  if constexpr (N == 64) key = bitonic_merge_desc<32>(key, 64, lane);   // lane & 64 is 0: descending throughout
  return key;
}

// Keys, one per lane (0 past the first n <= 64), sorted descending in lanes 0 .. n-1 by the
// smallest lane group of 16, 32 or 64 that holds them (n is wave-uniform).
__device__ __forceinline__ unsigned long long sort_candidates(unsigned long long c, int n, int lane) {
  if (n <= 16) return wave_sort_desc<16>(c, lane);
  if (n <= 32) return wave_sort_desc<32>(c, lane);
  return wave_sort_desc<64>(c, lane);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// ------------------------------------------------------------------------------ selection keys
// Order-preserving float -> uint32 (larger float, larger key; -0 == +0; NaN ranks as -inf).
// Every number maps to >= 0x007fffff, so 0 can mark an absent entry.
__device__ __forceinline__ uint32_t sel_key(float f) {
  f = f != f ? -__builtin_inff() : f + 0.0f;   // -0 + 0 = +0 (round to nearest)
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);   // negative: ~u, else u | sign bit
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Total order of a selection: larger key first, then lower index (the maximum is the winner).
__device__ __forceinline__ unsigned long long rank_key(uint32_t key, int i) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}

// ------------------------------------------------------------------------------ sync
// Cross-workgroup hand-off inside one kernel, without an agent-scope fence. On gfx950 such a
// fence writes back the whole L2 of the XCD and invalidates it, and every wave that executes one
// serialises device-wide (~14 ns each), so a grid of hundreds of workgroups pays tens of
// microseconds. Instead, data that another workgroup reads in the same kernel is written with a
// device-coherent store (global_store ... sc1: written through to the coherence point that all
// XCDs share) and read with a device-coherent load (global_load ... sc1: never served by a stale
// L2/L1 copy). A writer waits for its stores to be acknowledged (s_waitcnt) before it signals on
// a counter, and a reader only issues its loads after it has observed the signal.
template <typename T>
__device__ __forceinline__ void st_coherent(T* p, T v) {
  __hip_atomic_store((QWS_GLOBAL T*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coherent(const T* p) {
  return __hip_atomic_load((QWS_GLOBAL T*)const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Arrive on `counter`, shared by `expected` workgroups that each call this once per launch;
// returns true (in every thread) in the last one to arrive, which also resets the counter to zero
// for the next launch. Every thread must have finished its st_coherent() stores beforehand and
// every thread of the workgroup must call this.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected, bool* lds_flag) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == expected;
    if (last) st_coherent(counter, 0u);
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag;
}

// Two-level arrival for large grids: same-address atomics serialise (~10 ns each), so workgroups
// first arrive on one of kArriveGroups counters (blockIdx % kArriveGroups) and the last of each
// group arrives on counters[kArriveGroups]. Returns true in the single last workgroup of the grid.
// Needs kArriveGroups + 1 counters, each on its own 128-byte line (stride kCounterStride).
constexpr int kArriveGroups = 16;
constexpr int kCounterStride = 32;  // unsigned words: 128 bytes
__device__ __forceinline__ bool arrive_last_grid(unsigned* counters, bool* lds_flag) {
  const unsigned g = blockIdx.x % kArriveGroups;
  const unsigned groups = gridDim.x < (unsigned)kArriveGroups ? gridDim.x : (unsigned)kArriveGroups;
  const unsigned in_group = (gridDim.x - g + kArriveGroups - 1) / kArriveGroups;
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    bool last = false;
    unsigned prev = __hip_atomic_fetch_add(counters + g * kCounterStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == in_group) {
      st_coherent(counters + g * kCounterStride, 0u);
      prev = __hip_atomic_fetch_add(counters + kArriveGroups * kCounterStride, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
      last = prev + 1 == groups;
      if (last) st_coherent(counters + kArriveGroups * kCounterStride, 0u);
    }
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag;
}

}  // namespace qws

// ------------------------------------------------------------------------------ host side
#ifndef __HIPCC_RTC__
namespace qws_host {

int set_device_error(hipError_t e);  // records the message, returns QWS_ERR_DEVICE
int set_error_text(int status, const char* text);  // records `text` for qws_strerror, returns status
int head_fp8_rtc_function(int M, long long rows, long long cols, const char* cache_dir, void** fn_out);
int moe_rtc_function(int M, bool a8, bool chained, int K, int E, int H, int I, int has_shared, const char* cache_dir,
                     void** fn_out);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

inline int check_launch() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? QWS_OK : set_device_error(e);
}

}  // namespace qws_host
#endif
