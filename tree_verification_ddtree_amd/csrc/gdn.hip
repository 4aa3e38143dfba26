// a3: tree gated delta-net with optional state persistence.
//
// The pages name tree-aware gated delta-net kernels, one of which persists
// per-node state so the accepted node's state can be restored (lucebox-hub
// README, "02 · DFlash DDtree", "Implemented here": gated_delta_net_tree,
// gated_delta_net_tree_persist).  The recurrence is the gated delta rule
// (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", 2024), applied per node
// from its parent's state.  It is evaluated here in WY form (gdn_wy.h):
// instead of walking the tree node after node with a 128-wide reduction per
// step, a workgroup forms every node's products with its R committed rows
// and the key products along ancestor paths in parallel, then solves a
// small triangular system per row level by level.  One workgroup owns R
// rows of one value head; DK/8 lanes own one row, 8 columns each.  The
// committed state is read once (2 MB per layer at 32 heads x 128 x 128).
#include "gdn_wy.h"

namespace ddt {

template <typename T, int DK>
__global__ __launch_bounds__(256, 1) void gdn_kernel(ddt_plan P, const T *__restrict__ q,
                                                     const T *__restrict__ k,
                                                     const T *__restrict__ v,
                                                     const T *__restrict__ alpha,
                                                     const T *__restrict__ beta,
                                                     const float *__restrict__ S_c, int Hk,
                                                     int Hv, int dv, int R, float scale,
                                                     float *__restrict__ out,
                                                     float *__restrict__ node_states) {
  constexpr int LPR = DK / 8;
  extern __shared__ float4 lds4[];
  const GdnLds L(P.n_max, R, DK);
  GdnView V(reinterpret_cast<char *>(lds4), L, P.n_max, R);
  const int b = blockIdx.z, h = blockIdx.y, tile = blockIdx.x;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int lr = tid / LPR, cg = tid % LPR, row0 = tile * R;
  const Seq s = seq_of(P, b);
  const int n = s.n;
  if (n == 0) return;
  const int g = h / (Hv / Hk);
  for (int j = tid; j < n; j += nth) {
    V.gid[j] = s.o + j;
    const unsigned long long a = (P.anc[s.o + j] & ((2ull << j) - 1)) | (1ull << j);
    V.anc[j] = a;
    V.dep[j] = __popcll(a) - 1;
  }
  float sc[8];
  ld8f(S_c + (((size_t)b * Hv + h) * dv + row0 + lr) * DK + cg * 8, sc);
  __syncthreads();
  gdn_stage<T, DK>(V, n, q, k, v, alpha, beta, Hk, Hv, dv, g, h, row0);
  const int nlev = gdn_levels(V, n);
  __syncthreads();
  gdn_products<LPR, DK>(V, n, sc, lr, cg, true);
  __syncthreads();
  gdn_solve(V, nlev, nth);
  gdn_outputs(V, n, scale, nth);
  if (node_states) {
    for (int i = 0; i < n; ++i) {
      float st[8];
      gdn_state<DK>(V, i, sc, lr, cg, st);
      st8f(node_states + (((size_t)(s.o + i) * Hv + h) * dv + row0 + lr) * DK + cg * 8, st);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < n * R; idx += nth)
    out[((size_t)(s.o + idx / R) * Hv + h) * dv + row0 + idx % R] = V.O[idx];
}

int check_plan(const ddt_plan *P);

template <typename T>
static void launch_gdn(int dk, dim3 grid, dim3 block, size_t lds, hipStream_t st, const ddt_plan &P,
                       const void *q, const void *k, const void *v, const void *al,
                       const void *be, const float *S, int Hk, int Hv, int dv, int R, float scale,
                       float *out, float *ns) {
#define DDT_GDN(D)                                                                              \
  do {                                                                                          \
    (void)hipFuncSetAttribute((const void *)gdn_kernel<T, D>,                                   \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);            \
    hipLaunchKernelGGL((gdn_kernel<T, D>), grid, block, lds, st, P, (const T *)q, (const T *)k, \
                       (const T *)v, (const T *)al, (const T *)be, S, Hk, Hv, dv, R, scale,    \
                       out, ns);                                                                \
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
                            float *out, float *node_states, void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!q || !k || !v || !alpha || !beta || !S_c || !out) return DDT_E_ARG;
  if (Hk < 1 || Hv < 1 || Hv % Hk) return DDT_E_SHAPE;
  if (dk != 16 && dk != 32 && dk != 64 && dk != 128) return DDT_E_SHAPE;
  const int lpr = dk / 8;
  if (dv < 1) return DDT_E_SHAPE;
  const int R = gdn_rows(dk, dv);
  if (dv % R) return DDT_E_SHAPE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  const size_t lds = GdnLds(P->n_max, R, dk).total;
  dim3 grid(dv / R, Hv, P->B), block(R * lpr);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == DDT_BF16)
    launch_gdn<uint16_t>(dk, grid, block, lds, st, *P, q, k, v, alpha, beta, S_c, Hk, Hv, dv, R,
                         scale, out, node_states);
  else
    launch_gdn<float>(dk, grid, block, lds, st, *P, q, k, v, alpha, beta, S_c, Hk, Hv, dv, R,
                      scale, out, node_states);
  return launch_status();
}
