// Device helpers shared by the gfx950 kernels of the gen-tower step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DEVI __device__ __forceinline__

DEVI float to_f(float x) { return x; }
DEVI float to_f(bf16 x) { return static_cast<float>(x); }
template <typename T> DEVI T from_f(float x);
template <> DEVI float from_f<float>(float x) { return x; }
template <> DEVI bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }  // RNE (v_cvt_pk_bf16_f32)

DEVI float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEVI float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Map hardware id -> logical id so that each XCD receives one contiguous range of
// logical ids: neighbouring logical tiles (which share operands) share an L2.
DEVI int xcd_remap(int id, int n) {
  const int q = n >> 3;
  if (id >= (q << 3)) return id;
  return (id & 7) * q + (id >> 3);
}

// silu(x) = x sigmoid(x).  The reciprocal is v_rcp_f32 (1 ulp) rather than an IEEE division,
// whose scale / fma / fixup sequence costs several times as many instructions; the result is
// rounded to bf16 by every caller.  1 + e^-x >= 1, so no denormal reaches the reciprocal;
// x = -inf gives NaN as the division would (-inf * 0).
DEVI float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
