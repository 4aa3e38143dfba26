// a6: commit of the accepted path.
//
// After the walk the accepted node's linear-attention state becomes the
// committed state -- the pages' "tree-aware SSM state rollback"
// (lucebox-hub README, "02 · DFlash DDtree", "Implemented here") -- the
// conv prefix advances over the accepted tokens, and their K/V enter the
// cache.  One launch covers every layer: a flat grid whose first blocks
// replay (or select) delta-net state tiles, then conv prefixes, then one
// block per sequence appending K/V for all attention layers and finally
// advancing T.
#include "gdn_wy.h"

namespace ddt {

struct CommitArgs {
  ddt_plan P;
  const int32_t *path, *L;
  int mode;
  const ddt_gdn_layer *gl;
  int n_gdn, Hk, Hv, dk, dv, gdt, C, cdt, tiles, R;
  const ddt_attn_layer *al;
  int n_attn, Hkv, D, kvdt;
  const int32_t *pt;
  int max_pages;
  int32_t *T;
  int nA, nB;  // block counts of the state and prefix parts
};

__device__ __forceinline__ int path_len(const CommitArgs &A, int b, int n) {
  int l = A.L[b];
  return l < 0 ? 0 : (l > n ? n : l);
}
__device__ __forceinline__ int path_node(const CommitArgs &A, int b, int r, int n) {
  int x = A.path[(size_t)b * A.P.n_max + r];
  return (x >= 0 && x < n) ? x : 0;
}

template <typename T, int DK>
__device__ void commit_state_tile(const CommitArgs &A, int unit, char *lds) {
  constexpr int LPR = DK / 8;
  const int tile = unit % A.tiles;
  int rest = unit / A.tiles;
  const int h = rest % A.Hv;
  rest /= A.Hv;
  const int b = rest % A.P.B;
  const int layer = rest / A.P.B;
  const int tid = threadIdx.x;
  const bool lane_on = tid < A.R * LPR;
  const int lr = tid / LPR, cg = tid % LPR, row0 = tile * A.R;
  const Seq s = seq_of(A.P, b);
  const int Lb = path_len(A, b, s.n);
  if (Lb == 0) return;
  const ddt_gdn_layer lay = A.gl[layer];
  float *Sr = lay.S_c + (((size_t)b * A.Hv + h) * A.dv + row0 + lr) * DK + cg * 8;
  if (A.mode == DDT_COMMIT_SELECT) {
    if (!lay.node_states) {
      if (tid == 0) atomicOr((unsigned *)&A.P.status[b], DDT_ST_COMMIT);
      return;
    }
    if (!lane_on) return;
    const int gn = s.o + path_node(A, b, Lb - 1, s.n);
    float s8[8];
    ld8f(lay.node_states + (((size_t)gn * A.Hv + h) * A.dv + row0 + lr) * DK + cg * 8, s8);
    st8f(Sr, s8);
    return;
  }
  // replay: the tree kernel's WY evaluation restricted to the accepted path
  // (a chain), so the state is bitwise the one that kernel would persist
  const GdnLds L(A.P.n_max, A.R, DK);
  GdnView V(lds, L, A.P.n_max, A.R);
  const int g = h / (A.Hv / A.Hk);
  for (int r = tid; r < Lb; r += blockDim.x) {
    V.gid[r] = s.o + path_node(A, b, r, s.n);
    V.anc[r] = (2ull << r) - 1;
    V.lvl[r] = r;
  }
  for (int d = tid; d <= Lb; d += blockDim.x) V.lvs[d] = d;
  float sc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (lane_on) ld8f(Sr, sc);
  __syncthreads();
  gdn_stage<T, DK>(V, Lb, (const T *)lay.q, (const T *)lay.k, (const T *)lay.v,
                   (const T *)lay.alpha, (const T *)lay.beta, A.Hk, A.Hv, A.dv, g, h, row0);
  __syncthreads();
  if (lane_on) gdn_products<LPR, DK>(V, Lb, sc, lr, cg, false);
  __syncthreads();
  if (lane_on) {
    gdn_solve(V, Lb, A.R * LPR);
    float s8[8];
    gdn_state<DK>(V, Lb - 1, sc, lr, cg, s8);
    st8f(Sr, s8);
  }
}

// 16-byte chunk of E elements
template <typename E>
struct Chunk {
  static constexpr int N = 16 / sizeof(E);
};

template <typename E>
__device__ void commit_prefix(const CommitArgs &A, int unit) {
  const int b = unit % A.P.B, layer = unit / A.P.B;
  const ddt_gdn_layer lay = A.gl[layer];
  if (!lay.x || !lay.prefix) return;
  const Seq s = seq_of(A.P, b);
  const int Lb = path_len(A, b, s.n), W1 = A.P.W - 1;
  if (Lb == 0 || W1 == 0) return;
  constexpr int NE = Chunk<E>::N;
  E *pre = (E *)lay.prefix + (size_t)b * W1 * A.C;
  const E *x = (const E *)lay.x;
  for (int c = threadIdx.x * NE; c < A.C; c += blockDim.x * NE) {
    // new slot j = position Lb + j of prefix ++ x[path]; reads run ahead of writes
    for (int j = 0; j < W1; ++j) {
      const int pos = Lb + j;
      const E *src = pos < W1 ? pre + (size_t)pos * A.C + c
                              : x + (size_t)(s.o + path_node(A, b, pos - W1, s.n)) * A.C + c;
      *reinterpret_cast<uint4 *>(pre + (size_t)j * A.C + c) = *reinterpret_cast<const uint4 *>(src);
    }
  }
}

__device__ __forceinline__ bool kv_fits(const CommitArgs &A, int b, int T0, int Lb) {
  return !A.pt || Lb == 0 || (T0 + Lb - 1) / DDT_PAGE < A.max_pages;
}

template <typename E>
__device__ void commit_kv(const CommitArgs &A, int unit) {
  const int b = unit % A.P.B, layer = unit / A.P.B;
  const Seq s = seq_of(A.P, b);
  const int Lb = path_len(A, b, s.n);
  const int T0 = A.T[b];
  if (T0 < 0 || !kv_fits(A, b, T0, Lb)) return;
  constexpr int NE = Chunk<E>::N;
  const int cpr = A.D / NE;  // chunks per (token, head) row
  const ddt_attn_layer lay = A.al[layer];
  const E *Kt = (const E *)lay.Kt, *Vt = (const E *)lay.Vt;
  E *Kc = (E *)lay.Kc, *Vc = (E *)lay.Vc;
  for (int w = threadIdx.x; w < Lb * A.Hkv * cpr; w += blockDim.x) {
    const int r = w / (A.Hkv * cpr), g = (w / cpr) % A.Hkv, d0 = (w % cpr) * NE;
    const int t = T0 + r;
    const int page = A.pt ? A.pt[(size_t)b * A.max_pages + t / DDT_PAGE] : t / DDT_PAGE;
    const size_t src = ((size_t)(s.o + path_node(A, b, r, s.n)) * A.Hkv + g) * A.D + d0;
    const size_t pg = (size_t)page * A.Hkv + g;
    *reinterpret_cast<uint4 *>(Kc + (pg * DDT_PAGE + t % DDT_PAGE) * A.D + d0) =
        *reinterpret_cast<const uint4 *>(Kt + src);
    E v[NE];
    *reinterpret_cast<uint4 *>(v) = *reinterpret_cast<const uint4 *>(Vt + src);
#pragma unroll
    for (int e = 0; e < NE; ++e) Vc[(pg * A.D + d0 + e) * DDT_PAGE + t % DDT_PAGE] = v[e];
  }
}

// T[b] += L[b] once every append of the step has read the old T
__global__ void commit_len_kernel(CommitArgs A) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= A.P.B) return;
  const Seq s = seq_of(A.P, b);
  const int Lb = path_len(A, b, s.n);
  const int T0 = A.T[b];
  if (T0 >= 0 && kv_fits(A, b, T0, Lb))
    A.T[b] = T0 + Lb;
  else
    A.P.status[b] |= DDT_ST_CTX;
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void commit_kernel(CommitArgs A) {
  extern __shared__ float4 commit_lds[];
  int u = blockIdx.x;
  if (u < A.nA) {
    commit_state_tile<T, DK>(A, u, reinterpret_cast<char *>(commit_lds));
    return;
  }
  u -= A.nA;
  if (u < A.nB) {
    if (A.cdt == DDT_BF16)
      commit_prefix<uint16_t>(A, u);
    else
      commit_prefix<float>(A, u);
    return;
  }
  u -= A.nB;
  if (A.kvdt == DDT_F16)
    commit_kv<uint16_t>(A, u);
  else
    commit_kv<float>(A, u);
}

int check_plan(const ddt_plan *P);

}  // namespace ddt

using namespace ddt;

extern "C" int ddt_commit_state(const ddt_plan *P, const int32_t *path, const int32_t *L,
                                int32_t mode, const ddt_gdn_layer *gdn_layers, int32_t n_gdn,
                                int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, int32_t gdn_dtype,
                                int32_t C, int32_t conv_dtype, const ddt_attn_layer *attn_layers,
                                int32_t n_attn, int32_t Hkv, int32_t D, int32_t kv_dtype,
                                const int32_t *page_table, int32_t max_pages, int32_t *T,
                                void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!path || !L) return DDT_E_ARG;
  if (mode != DDT_COMMIT_REPLAY && mode != DDT_COMMIT_SELECT) return DDT_E_ARG;
  if (n_gdn < 0 || n_attn < 0) return DDT_E_SHAPE;
  CommitArgs A{};
  A.P = *P;
  A.path = path;
  A.L = L;
  A.mode = mode;
  A.gl = gdn_layers;
  A.n_gdn = n_gdn;
  A.al = attn_layers;
  A.n_attn = n_attn;
  A.pt = page_table;
  A.max_pages = max_pages;
  A.T = T;
  int dkc = 128;
  if (n_gdn > 0) {
    if (!gdn_layers) return DDT_E_ARG;
    if (Hk < 1 || Hv < 1 || Hv % Hk) return DDT_E_SHAPE;
    if (dk != 16 && dk != 32 && dk != 64 && dk != 128) return DDT_E_SHAPE;
    if (dv < 1 || dv % gdn_rows(dk, dv)) return DDT_E_SHAPE;
    if (gdn_dtype != DDT_BF16 && gdn_dtype != DDT_F32) return DDT_E_DTYPE;
    if (conv_dtype != DDT_BF16 && conv_dtype != DDT_F32) return DDT_E_DTYPE;
    if (C < 0 || C % 8) return DDT_E_SHAPE;
    A.Hk = Hk; A.Hv = Hv; A.dk = dk; A.dv = dv; A.gdt = gdn_dtype; A.C = C; A.cdt = conv_dtype;
    A.R = gdn_rows(dk, dv);
    A.tiles = dv / A.R;
    A.nA = n_gdn * P->B * Hv * A.tiles;
    A.nB = (C > 0) ? n_gdn * P->B : 0;
    dkc = dk;
  }
  int nC = 0;
  if (n_attn > 0) {
    if (!attn_layers || !T) return DDT_E_ARG;
    if (Hkv < 1 || D < 1) return DDT_E_SHAPE;
    if (kv_dtype != DDT_F16 && kv_dtype != DDT_F32) return DDT_E_DTYPE;
    if (!page_table && P->B != 1) return DDT_E_ARG;
    if (page_table && max_pages < 1) return DDT_E_SHAPE;
    const int ne = kv_dtype == DDT_F16 ? 8 : 4;
    if (D % ne) return DDT_E_SHAPE;
    A.Hkv = Hkv; A.D = D; A.kvdt = kv_dtype;
    nC = n_attn * P->B;
  }
  const int blocks = A.nA + A.nB + nC;
  if (blocks == 0) return DDT_OK;
  hipStream_t st = (hipStream_t)stream;
  const size_t lds = (n_gdn > 0 && mode == DDT_COMMIT_REPLAY) ? GdnLds(P->n_max, A.R, dkc).total : 0;
#define DDT_COMMIT(TT, DD)                                                                  \
  do {                                                                                      \
    (void)hipFuncSetAttribute((const void *)commit_kernel<TT, DD>,                          \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);        \
    hipLaunchKernelGGL((commit_kernel<TT, DD>), dim3(blocks), dim3(256), lds, st, A);      \
  } while (0)
  const bool bf = (n_gdn == 0) || gdn_dtype == DDT_BF16;
  switch (dkc) {
    case 16: if (bf) DDT_COMMIT(uint16_t, 16); else DDT_COMMIT(float, 16); break;
    case 32: if (bf) DDT_COMMIT(uint16_t, 32); else DDT_COMMIT(float, 32); break;
    case 64: if (bf) DDT_COMMIT(uint16_t, 64); else DDT_COMMIT(float, 64); break;
    default: if (bf) DDT_COMMIT(uint16_t, 128); else DDT_COMMIT(float, 128); break;
  }
#undef DDT_COMMIT
  r = launch_status();
  if (r || n_attn == 0) return r;
  hipLaunchKernelGGL(commit_len_kernel, dim3((P->B + 63) / 64), dim3(64), 0, st, A);
  return launch_status();
}
