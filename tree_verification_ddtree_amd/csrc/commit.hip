// Commit of the accepted path.
//
// After the walk the accepted node's linear-attention state becomes the
// committed state -- the pages' "tree-aware SSM state rollback"
// (lucebox-hub README, "02 · DFlash DDtree", "Implemented here") -- the
// conv prefix advances over the accepted tokens, and their K/V enter the
// cache.  One launch covers every layer: a flat grid whose first blocks
// append the accepted K/V (one per attention layer and sequence), then
// advance the conv prefixes, then update (or select, or replay) the
// delta-net state tiles; a second, tiny launch advances T.
#include "gdn_wy.h"

namespace ddt {

struct CommitArgs {
  ddt_plan P;
  const int32_t *path, *L;
  int mode;
  const ddt_gdn_layer *gl;
  int n_gdn, Hk, Hv, dk, dv, gdt, C, cdt, tiles;
  const ddt_attn_layer *al;
  int n_attn, Hkv, D, kvdt;
  const int32_t *pt;
  int max_pages;
  int32_t *T;
  int nA, nB, nC;  // block counts of the state, prefix and K/V parts
  int ncg;         // prefix column groups (256 chunks of 16 bytes each)
};

__device__ __forceinline__ int path_len(const CommitArgs &A, int b, int n) {
  int l = A.L[b];
  return l < 0 ? 0 : (l > n ? n : l);
}

// Whether sequence b is committed: with attention layers its cache must take
// the Lb accepted tokens (T0 + Lb <= 16 * max_pages, for a paged and for a
// contiguous cache alike).  Every part of the commit asks the same question
// on the same T[b] (only commit_len_kernel, which runs after them, changes
// it), so a sequence is committed whole or not at all.
__device__ __forceinline__ int seq_T0(const CommitArgs &A, int b) { return A.n_attn ? A.T[b] : 0; }
__device__ __forceinline__ bool seq_fits(const CommitArgs &A, int T0, int Lb) {
  if (A.n_attn == 0) return true;
  return T0 >= 0 && (long long)T0 + Lb <= (long long)A.max_pages * DDT_PAGE;
}
__device__ __forceinline__ int path_node(const CommitArgs &A, int b, int r, int n) {
  int x = A.path[(size_t)b * A.P.n_max + r];
  return (x >= 0 && x < n) ? x : 0;
}

// UPDATE rows per pass (every thread owns 8 columns of one row per pass)
// and passes per workgroup.
template <int DK>
struct UpdShape {
  static constexpr int LPR = DK / 8, RPP = 256 / LPR, PASSES = 2, ROWS = RPP * PASSES;
  static_assert(ROWS == (256 / (DK / 8)) * 2, "host computes the same row count");
};

// UPDATE: the committed rows row0 .. row0 + ROWS - 1 (clipped to dv) of one
// value head become the state of the last path node, rebuilt from the u
// the tree kernel saved.  Per row, the same sequence of fp32 operations as
// gdn_state (ancestors nearest first), so the result is bitwise the state
// the tree kernel would persist.  The path comes in with one load per lane
// (lane r holds path node r) and is broadcast from registers, so that every
// key, gate and u load of the path goes out in one batch instead of waiting
// for a path entry each; nothing goes through LDS.
template <typename T, int DK>
__device__ void commit_update_rows(const CommitArgs &A, const ddt_gdn_layer &lay, const Seq &s, int b,
                                   int h, int row0, int Lb, int pnode, float *Shead) {
  using SH = UpdShape<DK>;
  // global views of the record's pointers (see as_global)
  const auto k = as_global((const T *)lay.k);
  const auto al = as_global((const T *)lay.alpha);
  const auto nu = as_global(lay.node_u);
  const auto Sg = as_global_w(Shead);
  const int g = h / (A.Hv / A.Hk);
  const int tid = threadIdx.x, c0 = (tid % SH::LPR) * 8, rsub = tid / SH::LPR;
  auto uidx = [&](int gn, int row) { return ((size_t)gn * A.Hv + h) * A.dv + row; };
  auto node = [&](int r) { return s.o + __builtin_amdgcn_readlane(pnode, r); };
  int rows[SH::PASSES];
  bool on[SH::PASSES];
  float acc[SH::PASSES][8], sc[SH::PASSES][8], ui[SH::PASSES];
  const int gi = node(Lb - 1);
#pragma unroll
  for (int p = 0; p < SH::PASSES; ++p) {
    const int r = row0 + rsub + SH::RPP * p;
    on[p] = r < A.dv;
    rows[p] = on[p] ? r : row0;
    load8(Sg + (size_t)rows[p] * DK + c0, sc[p]);
    ui[p] = nu[uidx(gi, rows[p])];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[p][e] = 0.f;
  }
  float ki[8];
  load8(k + ((size_t)gi * A.Hk + g) * DK + c0, ki);
  const float ai = load1(al + (size_t)gi * A.Hv + h);
  constexpr int NA = 4;  // ancestors per batch
  float w = 1.f;
  // ancestors r0, r0 - 1, .., r0 - NA + 1 (nearest first); the first batch is
  // straight-line code so that its loads go out with the state's
  auto batch = [&](int r0) {
    float ka[NA][8], aa[NA], ua[SH::PASSES][NA];
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const int ga = node(max(r0 - t, 0));
      load8(k + ((size_t)ga * A.Hk + g) * DK + c0, ka[t]);
      aa[t] = load1(al + (size_t)ga * A.Hv + h);
#pragma unroll
      for (int p = 0; p < SH::PASSES; ++p) ua[p][t] = nu[uidx(ga, rows[p])];
    }
    float cw[NA];  // a_i w(a,i) of each ancestor, nearest first
#pragma unroll
    for (int t = 0; t < NA; ++t)
      if (r0 - t >= 0) {
        cw[t] = ai * w;
        w *= aa[t];
      }
#pragma unroll
    for (int p = 0; p < SH::PASSES; ++p) {
#pragma unroll
      for (int t = 0; t < NA; ++t)
        if (r0 - t >= 0) {
          const float c = cw[t] * ua[p][t];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[p][e] = fmaf(c, ka[t][e], acc[p][e]);
        }
    }
  };
  if (Lb >= 2) batch(Lb - 2);
  for (int r0 = Lb - 2 - NA; r0 >= 0; r0 -= NA) batch(r0);
  const float cs = ai * w;
#pragma unroll
  for (int p = 0; p < SH::PASSES; ++p) {
    if (!on[p]) continue;
    float s8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s8[e] = fmaf(ui[p], ki[e], fmaf(cs, sc[p][e], acc[p][e]));
    st8f(Sg + (size_t)rows[p] * DK + c0, s8);
  }
}

template <typename T, int DK, int MODE>
__device__ void commit_state_tile(const CommitArgs &A, int unit, char *lds) {
  constexpr int LPR = DK / 8;
  const int tile = unit % A.tiles;
  int rest = unit / A.tiles;
  const int h = rest % A.Hv;
  rest /= A.Hv;
  const int b = rest % A.P.B;
  const int layer = rest / A.P.B;
  const int tid = threadIdx.x;
  const bool lane_on = tid < GDN_R * LPR;
  const int lr = tid / LPR, c0 = (tid % LPR) * 8, row0 = tile * GDN_R;
  const Seq s = seq_of(A.P, b);
  const ddt_gdn_layer lay = A.gl[layer];
  int praw = 0;  // UPDATE: lane r's path entry r
  if constexpr (MODE == DDT_COMMIT_UPDATE) praw = A.path[(size_t)b * A.P.n_max + min(tid & 63, A.P.n_max - 1)];
  const int Lb = path_len(A, b, s.n);
  const int T0 = seq_T0(A, b);
  // the layer record, the path, its length and the committed length arrive
  // in one round trip (without this the compiler moves each load behind the
  // branch before it)
  if constexpr (MODE == DDT_COMMIT_UPDATE) asm volatile("" ::"v"(praw), "v"(Lb), "v"(T0), "v"(lay.node_u));
  if (Lb == 0 || !seq_fits(A, T0, Lb)) return;
  float *Sbase = lay.S_c + (((size_t)b * A.Hv + h) * A.dv + row0) * DK;
  if (MODE == DDT_COMMIT_SELECT) {
    if (!lay.node_states) {
      if (tid == 0) atomicOr((unsigned *)&A.P.status[b], DDT_ST_COMMIT);
      return;
    }
    if (!lane_on) return;
    const int gn = s.o + path_node(A, b, Lb - 1, s.n);
    float s8[8];
    ld8f(lay.node_states + (((size_t)gn * A.Hv + h) * A.dv + row0 + lr) * DK + c0, s8);
    st8f(Sbase + lr * DK + c0, s8);
    return;
  }
  if (MODE == DDT_COMMIT_UPDATE) {
    if (!lay.node_u) {
      if (tid == 0) atomicOr((unsigned *)&A.P.status[b], DDT_ST_COMMIT);
      return;
    }
    const int pnode = (praw >= 0 && praw < s.n) ? praw : 0;  // as path_node
    commit_update_rows<T, DK>(A, lay, s, b, h, tile * UpdShape<DK>::ROWS, Lb, pnode,
                              lay.S_c + ((size_t)b * A.Hv + h) * A.dv * DK);
    return;
  }
  // Replay: the tree kernel's evaluation restricted to the accepted path, a
  // chain whose nodes take positions 0..Lb-1 (position r has ancestors
  // 0..r-1, visited nearest first as in the tree).
  const GdnLds L(A.P.n_max);
  GdnView V(lds, L, A.P.n_max);
  const int g = h / (A.Hv / A.Hk);
  const T *k = (const T *)lay.k;
  auto gid = [&](int r) { return s.o + path_node(A, b, r, s.n); };
  auto chain = [&](int r) { return ~0ull >> (63 - r); };
  gdn_front<T, DK>(V, Lb, gid, chain, (const T *)lay.q, k, (const T *)lay.v, (const T *)lay.alpha,
                   (const T *)lay.beta, Sbase, A.Hk, A.Hv, A.dv, g, h, row0);
  __syncthreads();
  gdn_scalar<false>(V, Lb, Lb, 1.f);
  __syncthreads();
  if (lane_on) {
    float s8[8];
    auto krow = [&](int r) { return k + ((size_t)gid(r) * A.Hk + g) * DK; };
    gdn_state(V, Lb - 1, lr, c0, Sbase + lr * DK, krow, s8);
    st8f(Sbase + lr * DK + c0, s8);
  }
}

// 16-byte chunk of E elements
template <typename E>
struct Chunk {
  static constexpr int N = 16 / sizeof(E);
};

// One unit = one (layer, sequence, group of 256 16-byte column chunks).
// Every slot's source is loaded before any slot is written: new slot j reads
// position Lb + j of prefix ++ x[path], and a thread's columns are its own.
template <typename E>
__device__ void commit_prefix(const CommitArgs &A, int unit) {
  constexpr int NE = Chunk<E>::N;
  const int cg = unit % A.ncg;
  unit /= A.ncg;
  const int b = unit % A.P.B, layer = unit / A.P.B;
  const ddt_gdn_layer lay = A.gl[layer];
  if (!lay.x || !lay.prefix) return;
  const Seq s = seq_of(A.P, b);
  const int Lb = path_len(A, b, s.n), W1 = A.P.W - 1;
  if (Lb == 0 || W1 == 0 || !seq_fits(A, seq_T0(A, b), Lb)) return;
  const int c = (cg * 256 + (int)threadIdx.x) * NE;
  if (c >= A.C) return;
  E *pre = (E *)lay.prefix + (size_t)b * W1 * A.C;
  const E *x = (const E *)lay.x;
  uint4 v[DDT_MAX_W - 1];
#pragma unroll
  for (int j = 0; j < DDT_MAX_W - 1; ++j) {
    if (j < W1) {
      const int pos = Lb + j;
      const E *src = pos < W1 ? pre + (size_t)pos * A.C + c
                              : x + (size_t)(s.o + path_node(A, b, pos - W1, s.n)) * A.C + c;
      v[j] = *reinterpret_cast<const uint4 *>(src);
    }
  }
#pragma unroll
  for (int j = 0; j < DDT_MAX_W - 1; ++j)
    if (j < W1) *reinterpret_cast<uint4 *>(pre + (size_t)j * A.C + c) = v[j];
}

template <typename E>
__device__ void commit_kv(const CommitArgs &A, int unit) {
  const int b = unit % A.P.B, layer = unit / A.P.B;
  const Seq s = seq_of(A.P, b);
  const int Lb = path_len(A, b, s.n);
  const int T0 = A.T[b];
  if (!seq_fits(A, T0, Lb)) return;
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
  if (seq_fits(A, T0, Lb))
    A.T[b] = T0 + Lb;
  else
    A.P.status[b] |= DDT_ST_CTX;
}

// One instantiation per mode, so that the replay's register demand does not
// lower the occupancy of the streaming modes.
// The short K/V and prefix units come first in the grid, so that they run
// beside the state tiles instead of after them.
template <typename T, int DK, int MODE>
__global__ __launch_bounds__(256) void commit_kernel(CommitArgs A) {
  extern __shared__ float4 commit_lds[];
  int u = blockIdx.x;
  if (u < A.nC) {
    if (A.kvdt == DDT_F16)
      commit_kv<uint16_t>(A, u);
    else
      commit_kv<float>(A, u);
    return;
  }
  u -= A.nC;
  if (u < A.nB) {
    if (A.cdt == DDT_BF16)
      commit_prefix<uint16_t>(A, u);
    else
      commit_prefix<float>(A, u);
    return;
  }
  u -= A.nB;
  commit_state_tile<T, DK, MODE>(A, u, reinterpret_cast<char *>(commit_lds));
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
  if (mode != DDT_COMMIT_REPLAY && mode != DDT_COMMIT_SELECT && mode != DDT_COMMIT_UPDATE)
    return DDT_E_ARG;
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
    if (dv < GDN_R || dv % GDN_R) return DDT_E_SHAPE;
    if (gdn_dtype != DDT_BF16 && gdn_dtype != DDT_F32) return DDT_E_DTYPE;
    if (conv_dtype != DDT_BF16 && conv_dtype != DDT_F32) return DDT_E_DTYPE;
    if (C < 0 || C % 8) return DDT_E_SHAPE;
    A.Hk = Hk; A.Hv = Hv; A.dk = dk; A.dv = dv; A.gdt = gdn_dtype; A.C = C; A.cdt = conv_dtype;
    if (mode == DDT_COMMIT_UPDATE) {
      const int rows = (256 / (dk / 8)) * 2;  // UpdShape<dk>::ROWS
      A.tiles = (dv + rows - 1) / rows;
    } else {
      A.tiles = dv / GDN_R;
    }
    A.nA = n_gdn * P->B * Hv * A.tiles;
    A.ncg = (C / (conv_dtype == DDT_BF16 ? 8 : 4) + 255) / 256;
    A.nB = (C > 0) ? n_gdn * P->B * A.ncg : 0;
    dkc = dk;
  }
  if (n_attn > 0) {
    if (!attn_layers || !T) return DDT_E_ARG;
    if (Hkv < 1 || D < 1) return DDT_E_SHAPE;
    if (kv_dtype != DDT_F16 && kv_dtype != DDT_F32) return DDT_E_DTYPE;
    if (!page_table && P->B != 1) return DDT_E_ARG;
    if (max_pages < 1) return DDT_E_SHAPE;  // the cache's capacity, paged or contiguous
    const int ne = kv_dtype == DDT_F16 ? 8 : 4;
    if (D % ne) return DDT_E_SHAPE;
    A.Hkv = Hkv; A.D = D; A.kvdt = kv_dtype;
    A.nC = n_attn * P->B;
  }
  const int blocks = A.nA + A.nB + A.nC;
  if (blocks == 0) return DDT_OK;
  hipStream_t st = (hipStream_t)stream;
  const bool bf = (n_gdn == 0) || gdn_dtype == DDT_BF16;
  const size_t lds = (n_gdn > 0 && mode == DDT_COMMIT_REPLAY) ? GdnLds(P->n_max).total : 0;
#define DDT_COMMIT3(TT, DD, MM)                                                           \
  do {                                                                                    \
    (void)hipFuncSetAttribute((const void *)commit_kernel<TT, DD, MM>,                    \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);      \
    hipLaunchKernelGGL((commit_kernel<TT, DD, MM>), dim3(blocks), dim3(256), lds, st, A); \
  } while (0)
#define DDT_COMMIT(TT, DD)                                                         \
  do {                                                                             \
    if (mode == DDT_COMMIT_REPLAY) DDT_COMMIT3(TT, DD, DDT_COMMIT_REPLAY);         \
    else if (mode == DDT_COMMIT_SELECT) DDT_COMMIT3(TT, DD, DDT_COMMIT_SELECT);    \
    else DDT_COMMIT3(TT, DD, DDT_COMMIT_UPDATE);                                   \
  } while (0)
  switch (dkc) {
    case 16: if (bf) DDT_COMMIT(uint16_t, 16); else DDT_COMMIT(float, 16); break;
    case 32: if (bf) DDT_COMMIT(uint16_t, 32); else DDT_COMMIT(float, 32); break;
    case 64: if (bf) DDT_COMMIT(uint16_t, 64); else DDT_COMMIT(float, 64); break;
    default: if (bf) DDT_COMMIT(uint16_t, 128); else DDT_COMMIT(float, 128); break;
  }
#undef DDT_COMMIT
#undef DDT_COMMIT3
  r = launch_status();
  if (r || n_attn == 0) return r;
  hipLaunchKernelGGL(commit_len_kernel, dim3((P->B + 63) / 64), dim3(64), 0, st, A);
  return launch_status();
}
