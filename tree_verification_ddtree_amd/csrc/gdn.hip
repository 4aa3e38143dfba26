// Tree gated delta-net with optional state persistence.
//
// The pages name tree-aware gated delta-net kernels, one of which persists
// per-node state so the accepted node's state can be restored (lucebox-hub
// README, "02 · DFlash DDtree", "Implemented here": gated_delta_net_tree,
// gated_delta_net_tree_persist).  The recurrence is the gated delta rule
// (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", 2024), applied per node
// from its parent's state.  It is evaluated here in WY form (gdn_wy.h):
// instead of walking the tree node after node with a d_k-wide reduction per
// step, a workgroup gets every dot product it needs from one small
// matrix-core product (exact bf16 products, fp32 accumulation), forms each
// node's coefficients once, and then solves a scalar triangular system per
// row, level by level, producing the outputs on the way.  One workgroup owns
// 16 rows of one value head; its committed rows are read from HBM once.
//
// Besides the outputs the kernel can store every node's state (persist) and
// every node's u (16 floats per node and row tile), from which the commit
// rebuilds the accepted node's state with one rank-L update.
#include "gdn_wy.h"

namespace ddt {

// The plan's sizes and the first pointers come first among the arguments,
// so that they arrive preloaded in scalar registers (see fused_kernel).
// With bf16 inputs the kernel is held to 168 registers, so three workgroups
// share a compute unit: a batch of sequences has many more workgroups than
// units, and each one is latency bound (8 sequences, 2048 workgroups: 23.9
// -> 20.1 us per layer; one sequence, 256 workgroups: unchanged at 5.4 us).
template <typename T, int DK>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 3 : 1) void gdn_kernel(int plan_B, int plan_n_total, int plan_n_max,
                                                     const float *__restrict__ S_c, const T *__restrict__ q,
                                                     const T *__restrict__ k, const T *__restrict__ v,
                                                     const T *__restrict__ alpha, const T *__restrict__ beta,
                                                     ddt_plan P, int Hk, int Hv, int dv, float scale,
                                                     float *__restrict__ out,
                                                     float *__restrict__ node_states,
                                                     float *__restrict__ node_u) {
  P.B = plan_B;
  P.n_total = plan_n_total;
  P.n_max = plan_n_max;
  // every other argument fetched now, in one round
  asm volatile("" ::"s"(P.anc), "s"(Hk), "s"(Hv), "s"(dv), "s"(scale), "s"(out), "s"(node_states),
               "s"(node_u));
  constexpr int LPR = DK / 8;  // lanes per state row when storing states
  extern __shared__ float4 lds4[];
  const GdnLds L(P.n_max);
  GdnView V(reinterpret_cast<char *>(lds4), L, P.n_max);
  const int b = blockIdx.z, h = blockIdx.y, row0 = blockIdx.x * GDN_R;
  const int tid = threadIdx.x;
  const Seq s = seq_of(P, b);
  const int n = s.n;
  if (n == 0) return;
  const int g = h / (Hv / Hk);
  const float *Srows = S_c + (((size_t)b * Hv + h) * dv + row0) * DK;
  auto gid = [&](int j) { return s.o + j; };
  auto anc_of = [&](int j) { return (P.anc[s.o + j] & ((2ull << j) - 1)) | (1ull << j); };
  gdn_front<T, DK>(V, n, gid, anc_of, q, k, v, alpha, beta, Srows, Hk, Hv, dv, g, h, row0);
  __syncthreads();
  const int nlev = gdn_nlev(n, (tid & 63) < n ? V.anc[tid & 63] : 0ull);
  gdn_scalar<true>(V, n, nlev, scale);
  __syncthreads();
  for (int idx = tid; idx < n * 4; idx += blockDim.x) {
    const int i = idx >> 2, c = (idx & 3) * 4;
    *reinterpret_cast<float4 *>(out + ((size_t)(s.o + i) * Hv + h) * dv + row0 + c) =
        *reinterpret_cast<const float4 *>(V.O + i * GDN_RS + c);
    if (node_u)
      *reinterpret_cast<float4 *>(node_u + ((size_t)(s.o + i) * Hv + h) * dv + row0 + c) =
          *reinterpret_cast<const float4 *>(V.U + i * GDN_RS + c);
  }
  if (node_states && tid < GDN_R * LPR) {
    const int lr = tid / LPR, c0 = (tid % LPR) * 8;
    auto krow = [&](int a) { return k + ((size_t)(s.o + a) * Hk + g) * DK; };
    for (int i = 0; i < n; ++i) {
      float st[8];
      gdn_state(V, i, lr, c0, Srows + lr * DK, krow, st);
      st8f(node_states + (((size_t)(s.o + i) * Hv + h) * dv + row0 + lr) * DK + c0, st);
    }
  }
}

int check_plan(const ddt_plan *P);

template <typename T>
static void launch_gdn(int dk, dim3 grid, size_t lds, hipStream_t st, const ddt_plan &P,
                       const void *q, const void *k, const void *v, const void *al,
                       const void *be, const float *S, int Hk, int Hv, int dv, float scale,
                       float *out, float *ns, float *nu) {
#define DDT_GDN(D)                                                                              \
  do {                                                                                          \
    (void)hipFuncSetAttribute((const void *)gdn_kernel<T, D>,                                   \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);            \
    hipLaunchKernelGGL((gdn_kernel<T, D>), grid, dim3(256), lds, st, P.B, P.n_total, P.n_max, S,      \
                       (const T *)q, (const T *)k, (const T *)v, (const T *)al, (const T *)be, P, Hk,  \
                       Hv, dv, scale, out, ns, nu);                                                    \
  } while (0)
  switch (dk) {
    case 16: DDT_GDN(16); break;
    case 32: DDT_GDN(32); break;
    case 64: DDT_GDN(64); break;
    default: DDT_GDN(128); break;
  }
#undef DDT_GDN
}

}  // namespace ddt

using namespace ddt;

extern "C" int ddt_tree_gdn(const ddt_plan *P, const void *q, const void *k, const void *v,
                            const void *alpha, const void *beta, const float *S_c, int32_t Hk,
                            int32_t Hv, int32_t dk, int32_t dv, float scale, int32_t dtype,
                            float *out, float *node_states, float *node_u, void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!q || !k || !v || !alpha || !beta || !S_c || !out) return DDT_E_ARG;
  if (Hk < 1 || Hv < 1 || Hv % Hk) return DDT_E_SHAPE;
  if (dk != 16 && dk != 32 && dk != 64 && dk != 128) return DDT_E_SHAPE;
  if (dv < GDN_R || dv % GDN_R) return DDT_E_SHAPE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  const size_t lds = GdnLds(P->n_max).total;
  dim3 grid(dv / GDN_R, Hv, P->B);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == DDT_BF16)
    launch_gdn<uint16_t>(dk, grid, lds, st, *P, q, k, v, alpha, beta, S_c, Hk, Hv, dv, scale, out,
                         node_states, node_u);
  else
    launch_gdn<float>(dk, grid, lds, st, *P, q, k, v, alpha, beta, S_c, Hk, Hv, dv, scale, out,
                      node_states, node_u);
  return launch_status();
}
