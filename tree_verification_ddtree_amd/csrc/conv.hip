// a2: tree-aware causal depthwise conv1d.
//
// The pages name a tree-mode conv among the kernels for tree-aware SSM
// state rollback (lucebox-hub README, "02 · DFlash DDtree", "Implemented
// here": ssm_conv_tree).  Each node convolves the W-token window that ends
// at it on the sequence committed-prefix ++ root path; the plan's window
// table names those tokens, so every output is an independent gather of W
// rows plus W taps: one thread per (node, 8 channels), 16-byte loads.
#include "common.h"

namespace ddt {

template <typename T, int W>
__global__ __launch_bounds__(256) void conv_kernel(ddt_plan P, const T *__restrict__ x,
                                                   const T *__restrict__ prefix,
                                                   const T *__restrict__ w, int C, int act,
                                                   float *__restrict__ y) {
  const int b = blockIdx.z, i = blockIdx.y;
  const Seq s = seq_of(P, b);
  if (i >= s.n) return;
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c0 >= C) return;
  constexpr int W1 = W - 1;
  const int g = s.o + i;
  float acc[8], v[8], tap[W][8];
  // taps w[c][0..W-1] of the 8 channels: one contiguous run of 8*W elements
  constexpr int NB = 8 * W * (int)sizeof(T);
  if constexpr (NB % 16 == 0) {
    T raw[8 * W];
    const uint4 *src = reinterpret_cast<const uint4 *>(w + (size_t)c0 * W);
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) reinterpret_cast<uint4 *>(raw)[i] = src[i];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int t = 0; t < W; ++t) tap[t][e] = load1(raw + e * W + t);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int t = 0; t < W; ++t) tap[t][e] = load1(w + (size_t)(c0 + e) * W + t);
  }
  load8(x + (size_t)g * C + c0, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = tap[W - 1][e] * v[e];
#pragma unroll
  for (int j = 1; j <= W1; ++j) {
    int src = P.win[(size_t)g * W1 + (j - 1)];
    const T *row;
    if (src >= 0) {
      src = src < s.n ? src : 0;
      row = x + (size_t)(s.o + src) * C;
    } else {
      int sl = -src - 1;
      sl = sl < W1 ? sl : W1 - 1;
      row = prefix + ((size_t)b * W1 + sl) * C;
    }
    load8(row + c0, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(tap[W - 1 - j][e], v[e], acc[e]);
  }
  if (act == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] / (1.0f + __expf(-acc[e]));
  }
  float4 *out = reinterpret_cast<float4 *>(y + (size_t)g * C + c0);
  out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

int check_plan(const ddt_plan *P);

}  // namespace ddt

using namespace ddt;

extern "C" int ddt_tree_conv(const ddt_plan *P, const void *x, const void *prefix, const void *w,
                             int32_t C, int32_t act, int32_t dtype, float *y, void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!x || !w || !y || (P->W > 1 && !prefix)) return DDT_E_ARG;
  if (act != 0 && act != 1) return DDT_E_ARG;
  if (C < 8 || C % 8) return DDT_E_SHAPE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  dim3 grid((C / 8 + 255) / 256, P->n_max, P->B);
  hipStream_t st = (hipStream_t)stream;
#define DDT_CONV(WW)                                                                              \
  do {                                                                                            \
    if (dtype == DDT_BF16)                                                                        \
      hipLaunchKernelGGL((conv_kernel<uint16_t, WW>), grid, dim3(256), 0, st, *P,                 \
                         (const uint16_t *)x, (const uint16_t *)prefix, (const uint16_t *)w, C,   \
                         act, y);                                                                 \
    else                                                                                          \
      hipLaunchKernelGGL((conv_kernel<float, WW>), grid, dim3(256), 0, st, *P, (const float *)x,  \
                         (const float *)prefix, (const float *)w, C, act, y);                     \
  } while (0)
  switch (P->W) {
    case 1: DDT_CONV(1); break;
    case 2: DDT_CONV(2); break;
    case 3: DDT_CONV(3); break;
    case 4: DDT_CONV(4); break;
    case 5: DDT_CONV(5); break;
    case 6: DDT_CONV(6); break;
    case 7: DDT_CONV(7); break;
    default: DDT_CONV(8); break;
  }
#undef DDT_CONV
  return launch_status();
}
