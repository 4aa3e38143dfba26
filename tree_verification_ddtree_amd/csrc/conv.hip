// Tree-aware causal depthwise conv1d.
//
// The pages name a tree-mode conv among the kernels for tree-aware SSM
// state rollback (lucebox-hub README, "02 · DFlash DDtree", "Implemented
// here": ssm_conv_tree).  Each node convolves the W-token window that ends
// at it on the sequence committed-prefix ++ root path; the plan's window
// table names those tokens, so every output is a gather of W rows plus W
// taps.  The gather is served from LDS so that the kernel needs a single
// round of global loads.
#include "common.h"

namespace ddt {

// A workgroup owns CS = 64 channels of every node of one tree: thread
// (node group ng, chunk cc) handles 8 channels of nodes ng, ng + 32.  All
// global reads (x rows, prefix rows, taps, window entries) are independent
// and issued together; the window gather then reads the x slice from LDS.
constexpr int CS = 64;

// The plan's sizes and the pointers come first among the arguments, so that
// they arrive preloaded in scalar registers (see fused_kernel).
template <typename T, int W>
__global__ __launch_bounds__(256) void conv_kernel(int plan_B, int plan_n_total, int plan_n_max,
                                                   const T *__restrict__ x, const T *__restrict__ prefix,
                                                   const T *__restrict__ w, float *__restrict__ y, int C, int act,
                                                   ddt_plan P) {
  P.B = plan_B;
  P.n_total = plan_n_total;
  P.n_max = plan_n_max;
  asm volatile("" ::"s"(C), "s"(act), "s"(P.win));  // fetched now, in one round
  constexpr int W1 = W - 1;
  __shared__ float4 xs4[DDT_MAX_NODES * CS / 4];  // [node][CS] fp32
  float *xs = reinterpret_cast<float *>(xs4);
  const int b = blockIdx.y;
  const Seq s = seq_of(P, b);
  const int cc = threadIdx.x & 7, ng = threadIdx.x >> 3;
  const int cl = cc * 8, c0 = blockIdx.x * CS + cl;
  float tap[W][8], pre[W1 > 0 ? W1 : 1][8], xv[2][8];
  int win[2][W1 > 0 ? W1 : 1];
  // ---- one round of independent loads
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
#pragma unroll
  for (int j = 0; j < W1; ++j) load8(prefix + ((size_t)b * W1 + j) * C + c0, pre[j]);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = min(ng + 32 * r, s.n - 1);
    if (i >= 0) {
      load8(x + (size_t)(s.o + i) * C + c0, xv[r]);
#pragma unroll
      for (int j = 0; j < W1; ++j) win[r][j] = P.win[(size_t)(s.o + i) * W1 + j];
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = ng + 32 * r;
    if (i < s.n) {
      float4 *d = reinterpret_cast<float4 *>(xs + i * CS + cl);
      d[0] = make_float4(xv[r][0], xv[r][1], xv[r][2], xv[r][3]);
      d[1] = make_float4(xv[r][4], xv[r][5], xv[r][6], xv[r][7]);
    }
  }
  __syncthreads();
  // ---- y_i = act(sum_t w[c][W-1-t] tok_t(i))
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = ng + 32 * r;
    if (i >= s.n) continue;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = tap[W - 1][e] * xv[r][e];
#pragma unroll
    for (int j = 1; j <= W1; ++j) {
      const int src = win[r][j - 1];
      float v[8];
      if (src >= 0) {
        ld8f(xs + (src < s.n ? src : 0) * CS + cl, v);
      } else {
        const int sl = min(-src - 1, W1 - 1);
#pragma unroll
        for (int jj = 0; jj < W1; ++jj)
          if (jj == sl)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = pre[jj][e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(tap[W - 1 - j][e], v[e], acc[e]);
    }
    if (act == 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] / (1.0f + __expf(-acc[e]));
    }
    st8f(y + (size_t)(s.o + i) * C + c0, acc);
  }
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
  if (C < CS || C % CS) return DDT_E_SHAPE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  dim3 grid(C / CS, P->B);
  hipStream_t st = (hipStream_t)stream;
#define DDT_CONV(WW)                                                                              \
  do {                                                                                            \
    if (dtype == DDT_BF16)                                                                        \
      hipLaunchKernelGGL((conv_kernel<uint16_t, WW>), grid, dim3(256), 0, st, P->B, P->n_total,   \
                         P->n_max, (const uint16_t *)x, (const uint16_t *)prefix, (const uint16_t *)w, \
                         y, C, act, *P);                                                          \
    else                                                                                          \
      hipLaunchKernelGGL((conv_kernel<float, WW>), grid, dim3(256), 0, st, P->B, P->n_total,      \
                         P->n_max, (const float *)x, (const float *)prefix, (const float *)w, y, C,   \
                         act, *P);                                                                \
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
