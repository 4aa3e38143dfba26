// Internal helpers shared by the libddtree kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ddtree.h"

namespace ddt {

// ---------------------------------------------------------------- errors
void set_hip_error(hipError_t e);
int launch_status();  // DDT_OK, or DDT_E_HIP after recording the last launch error

// ---------------------------------------------------------------- types
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// 8 consecutive elements -> float (16 B aligned for bf16, 32 B for fp32)
__device__ __forceinline__ void load8(const uint16_t *p, float *f) {
  uint4 u = *reinterpret_cast<const uint4 *>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float *p, float *f) {
  float4 a = reinterpret_cast<const float4 *>(p)[0];
  float4 b = reinterpret_cast<const float4 *>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ float load1(const uint16_t *p) { return bf16f(*p); }
__device__ __forceinline__ float load1(const float *p) { return *p; }

// ---------------------------------------------------------------- plan access
// A sequence's node range, clamped so that a corrupt tree_off can never
// send a kernel outside the per-node arrays.  A single tree is nodes
// 0..n_total-1 and costs no load (the device plan flags a tree_off that
// says otherwise).
struct Seq {
  int o, n;
};
__device__ __forceinline__ Seq seq_of(const ddt_plan &P, int b) {
  if (P.B == 1) {
    const int n = P.n_total < P.n_max ? P.n_total : P.n_max;
    return {0, n < 0 ? 0 : n};
  }
  int o = P.tree_off[b], e = P.tree_off[b + 1];
  o = o < 0 ? 0 : (o > P.n_total ? P.n_total : o);
  e = e < o ? o : (e > P.n_total ? P.n_total : e);
  int n = e - o;
  if (n > P.n_max) n = P.n_max;
  return {o, n};
}

// ---------------------------------------------------------------- lane reductions
// DPP moves inside a row of 16 lanes.  quad_perm [1,0,3,2] = 0xB1,
// [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.  Each step
// adds two operands that are the same pair on both partner lanes, so every
// lane of a group ends with bitwise the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int G>  // sum over aligned groups of G lanes, G in {1,2,4,8,16}
__device__ __forceinline__ float group_sum(float v) {
  if (G >= 2) v += dpp<0xB1>(v);
  if (G >= 4) v += dpp<0x4E>(v);
  if (G >= 8) v += dpp<0x141>(v);
  if (G >= 16) v += dpp<0x140>(v);
  return v;
}

// ---------------------------------------------------------------- global views
// A pointer read from device memory (a field of a layer record) has the
// generic address space, so its loads are flat loads, and a wait can only
// drain flat loads all at once.  Through a global view they are global loads,
// which a wait can take one by one (the others stay in flight).
#define DDT_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const DDT_GLOBAL T *as_global(const T *p) {
  return (const DDT_GLOBAL T *)p;
}
template <typename T>
__device__ __forceinline__ DDT_GLOBAL T *as_global_w(T *p) {
  return (DDT_GLOBAL T *)p;
}
typedef unsigned ddt_u32x4 __attribute__((ext_vector_type(4)));
typedef float ddt_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load8(const DDT_GLOBAL uint16_t *p, float *f) {
  const ddt_u32x4 u = *(const DDT_GLOBAL ddt_u32x4 *)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const DDT_GLOBAL float *p, float *f) {
  const ddt_f32x4 a = ((const DDT_GLOBAL ddt_f32x4 *)p)[0];
  const ddt_f32x4 b = ((const DDT_GLOBAL ddt_f32x4 *)p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[4 + i] = b[i];
  }
}
__device__ __forceinline__ float load1(const DDT_GLOBAL uint16_t *p) { return bf16f(*p); }
__device__ __forceinline__ float load1(const DDT_GLOBAL float *p) { return *p; }
__device__ __forceinline__ void st8f(DDT_GLOBAL float *p, const float (&f)[8]) {
  ((DDT_GLOBAL ddt_f32x4 *)p)[0] = ddt_f32x4{f[0], f[1], f[2], f[3]};
  ((DDT_GLOBAL ddt_f32x4 *)p)[1] = ddt_f32x4{f[4], f[5], f[6], f[7]};
}

__device__ __forceinline__ void ld8f(const float *p, float (&f)[8]) {
  float4 a0 = reinterpret_cast<const float4 *>(p)[0];
  float4 a1 = reinterpret_cast<const float4 *>(p)[1];
  f[0] = a0.x; f[1] = a0.y; f[2] = a0.z; f[3] = a0.w;
  f[4] = a1.x; f[5] = a1.y; f[6] = a1.z; f[7] = a1.w;
}
__device__ __forceinline__ void st8f(float *p, const float (&f)[8]) {
  reinterpret_cast<float4 *>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4 *>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

}  // namespace ddt
