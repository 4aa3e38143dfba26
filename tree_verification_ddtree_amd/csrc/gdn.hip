// a3: tree gated delta-net with optional state persistence.
//
// The pages name tree-aware gated delta-net kernels, one of which persists
// per-node state so the accepted node's state can be restored (lucebox-hub
// README, "02 · DFlash DDtree", "Implemented here": gated_delta_net_tree,
// gated_delta_net_tree_persist).  The rule is the gated delta rule (Yang,
// Kautz, Hatamizadeh, "Gated Delta Networks", 2024):
//   S_n = a_n S_p (I - b_n k_n k_n^T) + b_n v_n k_n^T,   o_n = scale S_n q_n,
// applied per node from its parent's state.  Row r of S evolves on its own:
//   s_n = a s_p + u k,  u = b (v_r - a (s_p . k)),
//   o_r = scale (a (s_p . q) + u (k . q)),
// so a workgroup owns R rows of one value head and walks the whole tree.
//
// Layout: DK/8 consecutive lanes own one row, 8 columns each.  All node
// inputs of the head (k, q, the tile's v, alpha, beta, plan entries) are
// staged in LDS in one parallel pass, and k.q of every node is formed once,
// so the sequential walk over the nodes touches only LDS and registers.
// Dot products finish with DPP sums inside the lane group.  The states of
// nodes that still have children to visit live in LDS slots chosen by the
// plan (at most floor(log2 n)+1 per row); when a node's parent is the node
// visited just before (the common case in a preorder) its state is taken
// straight from registers.  Each lane only touches its own 8 columns of its
// own row in the slots, so the walk needs no barrier.  The committed state
// is read once from HBM (2 MB per layer at 32 heads x 128 x 128 fp32).
#include "common.h"

namespace ddt {

template <typename T, int DK>
__global__ __launch_bounds__(256) void gdn_kernel(ddt_plan P, const T *__restrict__ q,
                                                  const T *__restrict__ k,
                                                  const T *__restrict__ v,
                                                  const T *__restrict__ alpha,
                                                  const T *__restrict__ beta,
                                                  const float *__restrict__ S_c, int Hk, int Hv,
                                                  int dv, int R, float scale,
                                                  float *__restrict__ out,
                                                  float *__restrict__ node_states, int nslot) {
  constexpr int LPR = DK / 8;  // lanes per row
  constexpr int CPN = DK / 8;  // 8-element chunks per key / query row
  extern __shared__ float4 lds4[];
  const int nmax = P.n_max;
  float *st = reinterpret_cast<float *>(lds4);              // [nslot][R][DK] live states
  T *kql = reinterpret_cast<T *>(st + (size_t)nslot * R * DK);  // [nmax][2][DK] k, q
  float *vl = reinterpret_cast<float *>(kql + (size_t)nmax * 2 * DK);  // [nmax][R]
  float *al = vl + nmax * R, *bl = al + nmax, *kqd = bl + nmax;       // [nmax] each
  int *ordl = reinterpret_cast<int *>(kqd + nmax), *parl = ordl + nmax, *sll = parl + nmax;

  const int b = blockIdx.z, h = blockIdx.y, tile = blockIdx.x;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int lr = tid / LPR, cg = tid % LPR;
  const int row = tile * R + lr;
  const Seq s = seq_of(P, b);
  const int n = s.n;
  if (n == 0) return;
  const int g = h / (Hv / Hk);
  const int c0 = cg * 8;

  // ---- stage every node's inputs of this head in LDS (one parallel pass)
  for (int idx = tid; idx < n * 2 * CPN; idx += nth) {
    const int node = idx / (2 * CPN), which = (idx / CPN) & 1, cc = idx % CPN;
    const T *src = (which ? q : k) + ((size_t)(s.o + node) * Hk + g) * DK + 8 * cc;
    T *dst = kql + ((size_t)node * 2 + which) * DK + 8 * cc;
    if (sizeof(T) == 2) {
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    } else {
      reinterpret_cast<uint4 *>(dst)[0] = reinterpret_cast<const uint4 *>(src)[0];
      reinterpret_cast<uint4 *>(dst)[1] = reinterpret_cast<const uint4 *>(src)[1];
    }
  }
  for (int idx = tid; idx < n * R; idx += nth)
    vl[idx] = load1(v + ((size_t)(s.o + idx / R) * Hv + h) * dv + tile * R + idx % R);
  for (int idx = tid; idx < n; idx += nth) {
    al[idx] = load1(alpha + (size_t)(s.o + idx) * Hv + h);
    bl[idx] = load1(beta + (size_t)(s.o + idx) * Hv + h);
    int o = P.order[s.o + idx];
    ordl[idx] = (o >= 0 && o < n) ? o : 0;
    parl[idx] = idx == 0 ? -1 : P.parent[s.o + idx];
    int sl = P.slot[s.o + idx];
    sll[idx] = sl < 0 ? 0 : (sl >= nslot ? nslot - 1 : sl);
  }
  float sc[8];
  ld8f(S_c + (((size_t)b * Hv + h) * dv + row) * DK + c0, sc);
  __syncthreads();
  // k . q of every node (one row group per node)
  for (int node = lr; node < n; node += R) {
    float kk[8], qq[8], t = 0.f;
    load8(kql + (size_t)node * 2 * DK + c0, kk);
    load8(kql + ((size_t)node * 2 + 1) * DK + c0, qq);
#pragma unroll
    for (int e = 0; e < 8; ++e) t = fmaf(kk[e], qq[e], t);
    t = group_sum<LPR>(t);
    if (cg == 0) kqd[node] = t;
  }
  __syncthreads();

  // ---- walk the tree in the plan's order; each lane owns 8 columns of a row
  float *mine = st + (size_t)lr * DK + c0;  // this lane's columns in slot 0
  const size_t slot_stride = (size_t)R * DK;
  float sprev[8];
  int prev = -1;
  for (int it = 0; it < n; ++it) {
    const int nd = ordl[it];
    const int par = parl[nd];
    float sp[8];
    if (par < 0 || par >= nd) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sp[e] = sc[e];
    } else if (par == prev) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sp[e] = sprev[e];
    } else {
      ld8f(mine + sll[par] * slot_stride, sp);
    }
    float kk[8], qq[8];
    load8(kql + (size_t)nd * 2 * DK + c0, kk);
    load8(kql + ((size_t)nd * 2 + 1) * DK + c0, qq);
    const float vr = vl[nd * R + lr], a = al[nd], bb = bl[nd], kq = kqd[nd];
    float dq_ = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dq_ = fmaf(sp[e], qq[e], dq_);
    float sn[8];
    const float u = gdn_row_step<LPR>(sp, kk, vr, a, bb, sn);
    dq_ = group_sum<LPR>(dq_);
    st8f(mine + sll[nd] * slot_stride, sn);
    const int gn = s.o + nd;
    if (node_states) st8f(node_states + (((size_t)gn * Hv + h) * dv + row) * DK + c0, sn);
    if (cg == 0) out[((size_t)gn * Hv + h) * dv + row] = scale * fmaf(a, dq_, u * kq);
#pragma unroll
    for (int e = 0; e < 8; ++e) sprev[e] = sn[e];
    prev = nd;
  }
}

static size_t gdn_lds_bytes(int nslot, int R, int dk, int nmax, int tsize) {
  return (size_t)nslot * R * dk * 4 + (size_t)nmax * 2 * dk * tsize + (size_t)nmax * R * 4 +
         (size_t)nmax * 3 * 4 + (size_t)nmax * 3 * 4;
}

int check_plan(const ddt_plan *P);

template <typename T>
static void launch_gdn(int dk, dim3 grid, dim3 block, size_t lds, hipStream_t st, const ddt_plan &P,
                       const void *q, const void *k, const void *v, const void *al,
                       const void *be, const float *S, int Hk, int Hv, int dv, int R, float scale,
                       float *out, float *ns, int nslot) {
#define DDT_GDN(D)                                                                              \
  do {                                                                                          \
    (void)hipFuncSetAttribute((const void *)gdn_kernel<T, D>,                                         \
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                  \
    hipLaunchKernelGGL((gdn_kernel<T, D>), grid, block, lds, st, P, (const T *)q, (const T *)k, \
                       (const T *)v, (const T *)al, (const T *)be, S, Hk, Hv, dv, R, scale,    \
                       out, ns, nslot);                                                         \
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
  const int nslot = ddt_plan_slots(P->n_max);
  const size_t lds = gdn_lds_bytes(nslot, R, dk, P->n_max, dtype == DDT_BF16 ? 2 : 4);
  dim3 grid(dv / R, Hv, P->B), block(R * lpr);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == DDT_BF16)
    launch_gdn<uint16_t>(dk, grid, block, lds, st, *P, q, k, v, alpha, beta, S_c, Hk, Hv, dv, R,
                         scale, out, node_states, nslot);
  else
    launch_gdn<float>(dk, grid, block, lds, st, *P, q, k, v, alpha, beta, S_c, Hk, Hv, dv, R,
                      scale, out, node_states, nslot);
  return launch_status();
}
