// Shared device types and helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace phi {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// LDS destination of the direct global -> LDS loads (buffer_load_dwordx4
// with lds: each lane's 16 bytes land at the wave-uniform LDS address +
// 16 * lane).  Every kernel issues them in the buffer (MUBUF) form: the
// compiler treats the global (FLAT) form as an LDS access in flight as well,
// which turns the per-read lgkmcnt waits of later LDS reads into
// lgkmcnt(0).  An offset argument of the buffer builtin is passed as a named
// variable: with an inline expression there, the host pass of this compiler
// silently dropped the kernel's launch stub (an undefined symbol at load).
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Cache-policy operand of global loads: non-temporal (streamed data).
constexpr int kCacheNT = 2;

// s_waitcnt with only vmcnt constrained (vmcnt bits [3:0] and [15:14]).
#define PHI_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// only.  __syncthreads() would also wait for every outstanding global load,
// draining DMA stages that are meant to stay in flight; a stage about to be
// read is waited for explicitly (vmcnt) before this barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Lane pairs (l, l ^ 32) and (l, l ^ 16) combined without an LDS round trip:
// v_permlane32_swap / v_permlane16_swap of a value with itself leave, in the
// two result registers of lane l, the values of lanes l and l ^ 32 (l ^ 16);
// which register holds which depends on the half, so only symmetric
// combinations are formed.  Both lanes of a pair get the same sum, operand
// order included.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <class T> struct vec4;
template <> struct vec4<float> {
  static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};
template <> struct vec4<f16> {
  static __device__ __forceinline__ f32x4 load(const f16* p) {
    f16x4 h = *reinterpret_cast<const f16x4*>(p);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  }
  static __device__ __forceinline__ void store(f16* p, f32x4 v) {
    *reinterpret_cast<f16x4*>(p) = f16x4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
  }
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }

template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }

// Workgroup index -> logical tile index, so that consecutive logical tiles
// run on the same XCD (workgroups are dispatched round-robin over the 8 XCDs,
// each with its own L2).  `grid` is a multiple of 8; indices >= n_tiles idle.
__device__ __forceinline__ int xcd_swizzle(int bid, int grid) {
  return (bid & 7) * (grid >> 3) + (bid >> 3);
}

}  // namespace phi
