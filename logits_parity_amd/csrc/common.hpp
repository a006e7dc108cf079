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

// Address spaces of the direct global -> LDS loads (global_load_lds_dwordx4:
// each lane's 16 bytes land at the wave-uniform LDS address + 16 * lane).
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

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
