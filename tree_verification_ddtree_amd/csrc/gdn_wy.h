// Gated delta rule over a tree of tokens in its WY form (shared by the tree
// kernel and the commit).
//
// Row r of a value head's state evolves on its own: for node i with parent
// p, s_i = a_i s_p + u_i k_i with u_i = b_i (v_i - a_i s_p . k_i).  Unrolled
// along the root path, every s_p . x is a combination of the committed
// row's products S_c . x and of the keys of the ancestors:
//   s_p . x = P_i (S_c . x) + sum_{a ancestor of i} w(a,i) u_a (k_a . x)
// with w(a,i) the product of the gates strictly between a and i and P_i the
// product of the gates of all ancestors of i.  So, per row,
//   u_i = b_i (v_i - a_i P_i D_i) - sum_a b_i a_i w(a,i) (k_a.k_i) u_a
//   o_i = scale (a_i (P_i F_i + sum_a w(a,i) (k_a.q_i) u_a) + u_i k_i.q_i)
//   s_i = sum_a a_i w(a,i) u_a k_a + a_i P_i S_c + u_i k_i
// where D_i = S_c . k_i and F_i = S_c . q_i.  Every dot product above is an
// entry of one small matrix product, [S_c tile ; K] x [k_0 q_0 k_1 q_1 ...],
// done on the matrix cores with operands fetched straight from global
// memory.  The scalar part then runs with one lane per (node, 4 rows): the
// lane walks its node's root path in registers, so no lane waits on
// another.  Trees deeper than that register path fall back to a
// level-by-level solve through LDS with per-node coefficient records.
//
// Matrix-core precision: with bf16 inputs, k and q are bf16 already and the
// fp32 committed rows are split exactly into three bf16 parts (8 + 8 + 8
// significand bits), so every product is exact and only the fp32
// accumulation rounds.  With fp32 inputs the fp32 matrix instruction is used.
//
// Every product entry depends only on its own row and column, and both
// solves evaluate, for every node, the same sequence of fp32 operations
// (ancestors nearest first), so a node's u and state come out bitwise the
// same whether the tree, only its root path, or only the saved u of that
// path is used.
#pragma once
#include "common.h"

namespace ddt {

typedef float gf32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int gu32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 gbf16x8 __attribute__((ext_vector_type(8)));

constexpr int GDN_R = 16;     // state rows per workgroup (one matrix-core row block)
// Floats per node in the node-major row arrays (v, D, F, U, O): the 16 rows
// and 4 of padding.  Lanes of the solve read the rows of different nodes;
// with a stride of 16 floats every node's row r falls on the same two LDS
// banks, with 20 the nodes spread over the banks, 16-byte alignment kept.
constexpr int GDN_RS = 20;
constexpr int GDN_MAXA = 8;   // nearest ancestors whose coefficients a node record keeps
constexpr int GDN_PATH = 12;  // deepest tree (levels) the register path solve takes

// Everything the level-by-level solve needs of one node (128 bytes).
struct GdnRec {
  int i, cnt;            // node; ancestors recorded (<= GDN_MAXA)
  float bi, c1;          // b_i; -(a_i P_i)
  float ai, P, kqd, wM;  // a_i; P_i; k_i . q_i; w(.,i) past the recorded ancestors
  int a[GDN_MAXA];       // ancestors, nearest first (padding: i)
  float m[GDN_MAXA];     // -(b_i a_i w(a,i) k_a . k_i)
  float h[GDN_MAXA];     // w(a,i) k_a . q_i
};

// LDS carve-up, every array 16-byte aligned; per-node row data is
// node-major ([node][GDN_RS], rows first) so a lane's 4 rows are one
// 16-byte access.
struct GdnLds {
  int n16, gs;
  size_t v, al, be, anc, lvl, pos, lvs, meta, Gm, D, F, U, O, rec, total;
  __host__ __device__ GdnLds(int nmax) {
    auto up = [](size_t x) { return (x + 15) / 16 * 16; };
    n16 = (nmax + 15) / 16 * 16;
    gs = 2 * n16;
    v = 0;                                       // [nmax][GDN_RS] v of the tile's rows
    al = up(v + (size_t)nmax * GDN_RS * 4);      // [nmax]
    be = up(al + (size_t)nmax * 4);              // [nmax]
    anc = up(be + (size_t)nmax * 4);             // [nmax] u64, self included
    lvl = up(anc + (size_t)nmax * 8);            // [nmax] nodes by level
    pos = up(lvl + (size_t)nmax * 4);            // [nmax] position in lvl
    lvs = up(pos + (size_t)nmax * 4);            // [nmax + 2] level starts
    meta = up(lvs + (size_t)(nmax + 2) * 4);     // [4]: number of levels
    Gm = up(meta + 16);                          // [n16][gs] k_a . (k|q)_j
    D = up(Gm + (size_t)n16 * gs * 4);           // [nmax][GDN_RS] S_c . k_j
    F = up(D + (size_t)nmax * GDN_RS * 4);       // [nmax][GDN_RS] S_c . q_j
    U = up(F + (size_t)nmax * GDN_RS * 4);       // [nmax][GDN_RS] u
    O = up(U + (size_t)nmax * GDN_RS * 4);       // [nmax][GDN_RS] outputs
    rec = up(O + (size_t)nmax * GDN_RS * 4);     // [nmax] GdnRec (deep trees only)
    total = up(rec + (size_t)nmax * sizeof(GdnRec));
  }
};

struct GdnView {
  float *v, *al, *be, *Gm, *D, *F, *U, *O;
  unsigned long long *anc;
  int *lvl, *pos, *lvs, *meta;
  GdnRec *rec;
  int nmax, gs;
  __device__ GdnView(char *base, const GdnLds &L, int nmax_) : nmax(nmax_), gs(L.gs) {
    v = reinterpret_cast<float *>(base + L.v);
    al = reinterpret_cast<float *>(base + L.al);
    be = reinterpret_cast<float *>(base + L.be);
    anc = reinterpret_cast<unsigned long long *>(base + L.anc);
    lvl = reinterpret_cast<int *>(base + L.lvl);
    pos = reinterpret_cast<int *>(base + L.pos);
    lvs = reinterpret_cast<int *>(base + L.lvs);
    meta = reinterpret_cast<int *>(base + L.meta);
    Gm = reinterpret_cast<float *>(base + L.Gm);
    D = reinterpret_cast<float *>(base + L.D);
    F = reinterpret_cast<float *>(base + L.F);
    U = reinterpret_cast<float *>(base + L.U);
    O = reinterpret_cast<float *>(base + L.O);
    rec = reinterpret_cast<GdnRec *>(base + L.rec);
  }
};

// closest ancestor of a node still in `bits` (indices grow along a root path)
__device__ __forceinline__ int top_bit(unsigned long long bits) { return 63 - __clzll((long long)bits); }

__device__ __forceinline__ gu32x4 ld16(const void *p) { return *reinterpret_cast<const gu32x4 *>(p); }

// 16-byte piece of T -> 16 / sizeof(T) floats
template <typename T>
__device__ __forceinline__ void piece_f32(gu32x4 x, float *f) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(x[i] << 16);
      f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
  }
}

// piece idx of the per-node v rows (16 / sizeof(T) elements) -> LDS fp32
template <typename T>
__device__ __forceinline__ void put_v(GdnView &V, int idx, gu32x4 x) {
  constexpr int UE = 16 / (int)sizeof(T), VP = GDN_R / UE;
  float f[UE];
  piece_f32<T>(x, f);
  float *dst = V.v + (idx / VP) * GDN_RS + (idx % VP) * UE;
  *reinterpret_cast<gf32x4 *>(dst) = gf32x4{f[0], f[1], f[2], f[3]};
  if constexpr (UE == 8) *reinterpret_cast<gf32x4 *>(dst + 4) = gf32x4{f[4], f[5], f[6], f[7]};
}

// exact three-way split of 8 fp32 values into bf16 parts hi, mid, lo
__device__ __forceinline__ void split3(gf32x4 x0, gf32x4 x1, gu32x4 (&o)[3]) {
  unsigned short p[3][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = e < 4 ? x0[e] : x1[e - 4];
    const unsigned u0 = __float_as_uint(x);
    const float r1 = x - __uint_as_float(u0 & 0xffff0000u);
    const unsigned u1 = __float_as_uint(r1);
    const float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
    p[0][e] = (unsigned short)(u0 >> 16);
    p[1][e] = (unsigned short)(u1 >> 16);
    p[2][e] = (unsigned short)(__float_as_uint(r2) >> 16);
  }
#pragma unroll
  for (int part = 0; part < 3; ++part)
#pragma unroll
    for (int w = 0; w < 4; ++w) o[part][w] = (unsigned)p[part][2 * w] | ((unsigned)p[part][2 * w + 1] << 16);
}

// Everything a workgroup reads for node set j = 0..n-1 (global node gid(j))
// and the committed rows row0..row0+15 of value head h (Srows), with the
// matrix-core products done on the way:
//   v of the 16 rows, gates, ancestor masks (anc_of(j), self included) -> LDS
//   D, F (committed rows x k, q) and Gm (keys x k, q) -> LDS
// Every global load of a thread is issued before its first use.  Operand
// layouts of the products (16 x 16 output): lane l feeds A row l%16 and B
// column l%16 with its share of the reduction dimension (k = 8(l/16) ..
// 8(l/16)+7 of each 32-wide step for the bf16 form; the contiguous quarter
// (l/16) of the channels for the 16x16x4 fp32 form) and receives rows
// 4(l/16) .. 4(l/16)+3 of column l%16.  Column c of kq is k (even c) or q
// (odd c) of node c/2; row block 0 is the committed tile, row block 1+m the
// keys of nodes 16m .. 16m+15.  Wave w takes column blocks w, w+4, ...
// NRB key row blocks are loaded whatever n is; rows and columns past the
// tree are read clamped to its last node (unconditional loads, so that none
// waits on another) and their products are never stored.
template <typename T, int DK, int NRB, class Gid, class Anc>
__device__ void gdn_front_rb(GdnView &V, int n, Gid gid, Anc anc_of, const T *__restrict__ q,
                             const T *__restrict__ k, const T *__restrict__ v,
                             const T *__restrict__ alpha, const T *__restrict__ beta,
                             const float *__restrict__ Srows, int Hk, int Hv, int dv, int g, int h,
                             int row0) {
  constexpr int UE = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int VP = GDN_R / UE;           // pieces of one node's 16 v entries
  constexpr int MAXRB = NRB;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nw = nth >> 6;
  const int lane = tid & 63, i16 = lane & 15, kk = lane >> 4;
  const int nrb = (n + 15) / 16, ncb = (2 * n + 15) / 16;
  const gu32x4 z = {0u, 0u, 0u, 0u};
  auto vsrc = [&](int idx) {
    return *(reinterpret_cast<const gu32x4 *>(v + ((size_t)gid(idx / VP) * Hv + h) * dv + row0) + idx % VP);
  };
  auto put_vs = [&](gu32x4 first) {
    const int nv = n * VP;
    if (tid < nv) put_v<T>(V, tid, first);
    for (int idx = tid + nth; idx < nv; idx += nth) put_v<T>(V, idx, vsrc(idx));
  };
  // ---- per-node inputs (loads first, stores once the product loads are out)
  const gu32x4 vb = vsrc(min(tid, n * VP - 1));
  const int jt = min(tid, n - 1);
  const float a0 = load1(alpha + (size_t)gid(jt) * Hv + h);
  const float b0 = load1(beta + (size_t)gid(jt) * Hv + h);
  const unsigned long long m0 = anc_of(jt);
  auto kq_row = [&](int c) -> const T * {  // column c of kq, c < 2n
    return ((c & 1) ? q : k) + ((size_t)gid(c >> 1) * Hk + g) * DK;
  };
  auto store_D = [&](int c, const gf32x4 &acc) {
    if (c < 2 * n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ((c & 1) ? V.F : V.D)[(c >> 1) * GDN_RS + 4 * kk + e] = acc[e];
    }
  };
  auto store_G = [&](int c, int m, const gf32x4 &g4) {
    if (c < 2 * n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 16 * m + 4 * kk + e;
        if (a < n) V.Gm[a * V.gs + c] = g4[e];
      }
    }
  };
  if (wave >= ncb) put_vs(vb);
  if constexpr (sizeof(T) == 2) {
    constexpr int NS = (DK + 31) / 32;
    gu32x4 sa[3][NS], ka[MAXRB][NS], bv[NS];
    if (wave < ncb) {
      // the committed rows are split only after the key loads are out: a
      // split right after its load would wait for it before they issue
      gf32x4 sx[NS][2];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int k0 = 32 * s + 8 * kk;
        sx[s][0] = sx[s][1] = gf32x4{0.f, 0.f, 0.f, 0.f};
        if (DK >= 32 || k0 < DK) {
          sx[s][0] = *reinterpret_cast<const gf32x4 *>(Srows + i16 * DK + k0);
          sx[s][1] = *reinterpret_cast<const gf32x4 *>(Srows + i16 * DK + k0 + 4);
        }
      }
#pragma unroll
      for (int m = 0; m < MAXRB; ++m)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int k0 = 32 * s + 8 * kk, a = min(16 * m + i16, n - 1);
          if constexpr (DK >= 32)
            ka[m][s] = ld16(k + ((size_t)gid(a) * Hk + g) * DK + k0);
          else
            ka[m][s] = k0 < DK ? ld16(k + ((size_t)gid(a) * Hk + g) * DK + k0) : z;
        }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        gu32x4 t3[3];
        split3(sx[s][0], sx[s][1], t3);
#pragma unroll
        for (int part = 0; part < 3; ++part) sa[part][s] = t3[part];
      }
    }
    for (int cb = wave; cb < ncb; cb += nw) {
      const int c = 16 * cb + i16;
      const T *bsrc = kq_row(min(c, 2 * n - 1));
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int k0 = 32 * s + 8 * kk;
        if constexpr (DK >= 32)
          bv[s] = ld16(bsrc + k0);
        else
          bv[s] = k0 < DK ? ld16(bsrc + k0) : z;
      }
      if (cb == wave) put_vs(vb);
      gf32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int part = 2; part >= 0; --part)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, sa[part][s]),
                                                        __builtin_bit_cast(gbf16x8, bv[s]), acc, 0, 0, 0);
      store_D(c, acc);
#pragma unroll
      for (int m = 0; m < MAXRB; ++m) {
        if (m < nrb) {
          gf32x4 g4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NS; ++s)
            g4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, ka[m][s]),
                                                         __builtin_bit_cast(gbf16x8, bv[s]), g4, 0, 0, 0);
          store_G(c, m, g4);
        }
      }
    }
  } else {
    constexpr int KS = DK / 4;  // channels per lane group
    constexpr int NP = KS / 4;  // float4 pieces per operand
    gf32x4 sa[NP], ka[MAXRB][NP], bv[NP];
    if (wave < ncb) {
#pragma unroll
      for (int s = 0; s < NP; ++s) sa[s] = *reinterpret_cast<const gf32x4 *>(Srows + i16 * DK + kk * KS + 4 * s);
#pragma unroll
      for (int m = 0; m < MAXRB; ++m)
#pragma unroll
        for (int s = 0; s < NP; ++s) {
          const int a = min(16 * m + i16, n - 1);
          ka[m][s] = *reinterpret_cast<const gf32x4 *>(k + ((size_t)gid(a) * Hk + g) * DK + kk * KS + 4 * s);
        }
    }
    auto prod = [&](const gf32x4 *A) {
      gf32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(A[s][0], bv[s][0], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(A[s][1], bv[s][1], c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(A[s][2], bv[s][2], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(A[s][3], bv[s][3], c1, 0, 0, 0);
      }
      return c0 + c1;
    };
    for (int cb = wave; cb < ncb; cb += nw) {
      const int c = 16 * cb + i16;
      const T *bsrc = kq_row(min(c, 2 * n - 1));
#pragma unroll
      for (int s = 0; s < NP; ++s)
        bv[s] = *reinterpret_cast<const gf32x4 *>(bsrc + kk * KS + 4 * s);
      if (cb == wave) put_vs(vb);
      store_D(c, prod(sa));
#pragma unroll
      for (int m = 0; m < MAXRB; ++m)
        if (m < nrb) store_G(c, m, prod(ka[m]));
    }
  }
  if (tid < n) {
    V.al[tid] = a0;
    V.be[tid] = b0;
    V.anc[tid] = m0;
  }
  for (int j = tid + nth; j < n; j += nth) {
    V.al[j] = load1(alpha + (size_t)gid(j) * Hv + h);
    V.be[j] = load1(beta + (size_t)gid(j) * Hv + h);
    V.anc[j] = anc_of(j);
  }
}

template <typename T, int DK, class Gid, class Anc>
__device__ void gdn_front(GdnView &V, int n, Gid gid, Anc anc_of, const T *__restrict__ q,
                          const T *__restrict__ k, const T *__restrict__ v,
                          const T *__restrict__ alpha, const T *__restrict__ beta,
                          const float *__restrict__ Srows, int Hk, int Hv, int dv, int g, int h,
                          int row0) {
  static_assert(DDT_MAX_NODES == 64, "key row blocks: 1, 2 or 4 of 16 nodes");
  if (n <= 16)
    gdn_front_rb<T, DK, 1>(V, n, gid, anc_of, q, k, v, alpha, beta, Srows, Hk, Hv, dv, g, h, row0);
  else if (n <= 32)
    gdn_front_rb<T, DK, 2>(V, n, gid, anc_of, q, k, v, alpha, beta, Srows, Hk, Hv, dv, g, h, row0);
  else
    gdn_front_rb<T, DK, 4>(V, n, gid, anc_of, q, k, v, alpha, beta, Srows, Hk, Hv, dv, g, h, row0);
}

// The two bf16 parts of 8 fp32 values x: hi is x rounded to bf16 (nearest
// even), lo the rounding of x - hi (exact in fp32).  hi + lo keeps 16
// significand bits, |x - (hi + lo)| <= 2^-16 |x|, and hi + lo is exact in
// fp32.  Each part comes as 8 bf16 in order (16 bytes), the layout of a
// matrix-core operand slice; the packed fp32 -> bf16 conversion does two
// values at once.
typedef __bf16 gbf16x2 __attribute__((ext_vector_type(2)));
typedef float gf32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_hilo8(const float (&v)[8], gu32x4 &hi, gu32x4 &lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector((gf32x2){v[2 * p], v[2 * p + 1]}, gbf16x2));
    const gf32x2 r = {v[2 * p] - __uint_as_float(h << 16), v[2 * p + 1] - __uint_as_float(h & 0xffff0000u)};
    hi[p] = h;
    lo[p] = __builtin_bit_cast(unsigned, __builtin_convertvector(r, gbf16x2));
  }
}
// hi + lo of element e of such a pair
__device__ __forceinline__ float hilo_value(const gu32x4 &hi, const gu32x4 &lo, int e) {
  const unsigned hw = hi[e >> 1], lw = lo[e >> 1];
  return (e & 1) ? __uint_as_float(hw & 0xffff0000u) + __uint_as_float(lw & 0xffff0000u)
                 : __uint_as_float(hw << 16) + __uint_as_float(lw << 16);
}
// A row held as hi and lo planes, read as fp32 values hi + lo (gdn_state).
struct PlaneRow {
  const uint16_t *h, *l;
  __device__ PlaneRow operator+(int c) const { return {h + c, l + c}; }
};
__device__ __forceinline__ void load8(PlaneRow r, float *f) {
  const gu32x4 a = *reinterpret_cast<const gu32x4 *>(r.h), b = *reinterpret_cast<const gu32x4 *>(r.l);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = hilo_value(a, b, e);
}

// Committed-row operand of the products for this lane (row i16, the
// lane's k-share of every 32-wide step), split exactly into three bf16
// parts; a caller loads it early and splits it while its other loads are
// on their way.
template <int DK>
struct SrowOperand {
  static constexpr int NS = (DK + 31) / 32;
  gf32x4 x[NS][2];
  gu32x4 sa[3][NS];  // the parts: hi, mid, lo
  __device__ __forceinline__ void load(const float *__restrict__ Srows) {
    const int lane = threadIdx.x & 63, i16 = lane & 15, kk = lane >> 4;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int k0 = 32 * s + 8 * kk;
      x[s][0] = x[s][1] = gf32x4{0.f, 0.f, 0.f, 0.f};
      if (k0 < DK) {
        x[s][0] = *reinterpret_cast<const gf32x4 *>(Srows + i16 * DK + k0);
        x[s][1] = *reinterpret_cast<const gf32x4 *>(Srows + i16 * DK + k0 + 4);
      }
    }
  }
  // the split, made to happen where it is called (the compiler would
  // otherwise move it to its first use, behind a workgroup barrier)
  __device__ __forceinline__ void split() {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      gu32x4 t3[3];
      split3(x[s][0], x[s][1], t3);
#pragma unroll
      for (int part = 0; part < 3; ++part) {
        sa[part][s] = t3[part];
        asm volatile("" ::"v"(sa[part][s]));
      }
    }
  }
};

// q and k rows of the fused layer in LDS: hi and lo planes of bf16 (node
// j's row of each at j * ld), whose values hi + lo are the layer's q and k.
struct QkPlanes {
  const uint16_t *qh, *ql, *kh, *kl;
  int ld;
};

// gdn_front for q and k that the workgroup computed itself (the fused
// layer): matrix operands are read straight from the planes (16 bytes per
// slice and part); the tile's v rows are already in V.v, and this thread's
// gates and mask (node tid, n <= blockDim) and its committed-row operand
// were loaded (and split) by the caller.  Same products and LDS outputs as
// gdn_front.  D and F sum the part products (row, column) lo*hi, mid*hi,
// hi*lo, hi*hi and the key products lo*hi, hi*lo, hi*hi: every dropped term
// stays below about 2^-15 of |row| |column|.  Rows and columns past the
// tree read the last node, so their products are finite, and they are
// never stored.
template <int DK, int NRB>
__device__ void gdn_front_lds_rb(GdnView &V, int n, const QkPlanes &Q, const SrowOperand<DK> &S) {
  constexpr int NS = SrowOperand<DK>::NS;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nw = nth >> 6;
  const int lane = tid & 63, i16 = lane & 15, kk = lane >> 4;
  const int ncb = (2 * n + 15) / 16;
  const gu32x4 z = {0u, 0u, 0u, 0u};
  // hi and lo operand slices of row `row` of planes (h, l), channels k0 .. k0 + 7
  auto slice = [&](const uint16_t *h, const uint16_t *l, int row, int k0, gu32x4 (&o)[2]) {
    if (DK >= 32 || k0 < DK) {
      o[0] = *reinterpret_cast<const gu32x4 *>(h + row * Q.ld + k0);
      o[1] = *reinterpret_cast<const gu32x4 *>(l + row * Q.ld + k0);
    } else {
      o[0] = o[1] = z;
    }
  };
  // Key row block m is needed by column block cb only if the block holds a
  // node at or before cb's last node (the solve reads k_a . x_b for a <= b
  // only): m < nm(cb).  When there are fewer column blocks than waves, an
  // idle wave takes the key row blocks m >= 1 of a column block (the last
  // ones need the most), so that no wave forms all of them.
  auto nm_of = [&](int cb) { return min(n - 1, 8 * cb + 7) / 16 + 1; };
  const int spare = ncb < nw ? nw - ncb : 0;
  auto helped = [&](int cb) { return ncb - 1 - cb < spare && nm_of(cb) >= 2; };
  // column block cb: operands of column c = 16 cb + i16 (k of node c/2 for
  // even c, q for odd c; past the tree the last node's)
  auto column = [&](int cb, gu32x4 (&bv)[NS][2]) {
    const int c = 16 * cb + i16;
    const bool isq = c & 1;
    const int cn = min(c, 2 * n - 1) >> 1;
#pragma unroll
    for (int s = 0; s < NS; ++s) slice(isq ? Q.qh : Q.kh, isq ? Q.ql : Q.kl, cn, 32 * s + 8 * kk, bv[s]);
  };
  // key row blocks m_lo .. m_hi - 1 against column block cb (operands read
  // by the caller for those blocks): k_a . k_b, k_a . q_b into Gm
  auto key_cells = [&](int cb, int m_lo, int m_hi, const gu32x4 (&bv)[NS][2], const gu32x4 (&ka)[NRB][NS][2]) {
    gf32x4 g4[NRB];
#pragma unroll
    for (int m = 0; m < NRB; ++m) {
      g4[m] = gf32x4{0.f, 0.f, 0.f, 0.f};
      if (m < m_lo || m >= m_hi) continue;  // the same in every lane
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        g4[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, ka[m][s][1]),
                                                        __builtin_bit_cast(gbf16x8, bv[s][0]), g4[m], 0, 0, 0);
        g4[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, ka[m][s][0]),
                                                        __builtin_bit_cast(gbf16x8, bv[s][1]), g4[m], 0, 0, 0);
        g4[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, ka[m][s][0]),
                                                        __builtin_bit_cast(gbf16x8, bv[s][0]), g4[m], 0, 0, 0);
      }
    }
    const int c = 16 * cb + i16;
    if (c < 2 * n) {
#pragma unroll
      for (int m = 0; m < NRB; ++m) {
        if (m < m_lo || m >= m_hi) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * m + 4 * kk + e;
          if (r < n) V.Gm[r * V.gs + c] = g4[m][e];
        }
      }
    }
  };
  auto key_rows = [&](int m_lo, int m_hi, gu32x4 (&ka)[NRB][NS][2]) {
#pragma unroll
    for (int m = 0; m < NRB; ++m) {
      if (m < m_lo || m >= m_hi) continue;
#pragma unroll
      for (int s = 0; s < NS; ++s) slice(Q.kh, Q.kl, min(16 * m + i16, n - 1), 32 * s + 8 * kk, ka[m][s]);
    }
  };
  if (wave >= ncb) {  // a spare wave: the upper key row blocks of one column block
    const int cb = ncb - 1 - (wave - ncb);
    if (cb < 0 || !helped(cb)) return;
    const int nm = nm_of(cb);
    gu32x4 bv[NS][2], ka[NRB][NS][2];
    column(cb, bv);
    key_rows(1, nm, ka);
    key_cells(cb, 1, nm, bv, ka);
    return;
  }
  const auto &sa = S.sa;
  for (int cb = wave; cb < ncb; cb += nw) {
    const int c = 16 * cb + i16;
    const bool isq = c & 1;
    const int mhi = helped(cb) ? 1 : nm_of(cb);
    // every operand read of the column block before any product is stored
    gu32x4 bv[NS][2], ka[NRB][NS][2];
    column(cb, bv);
    key_rows(0, mhi, ka);
    gf32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, sa[2][s]),
                                                    __builtin_bit_cast(gbf16x8, bv[s][0]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, sa[1][s]),
                                                    __builtin_bit_cast(gbf16x8, bv[s][0]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, sa[0][s]),
                                                    __builtin_bit_cast(gbf16x8, bv[s][1]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8, sa[0][s]),
                                                    __builtin_bit_cast(gbf16x8, bv[s][0]), acc, 0, 0, 0);
    }
    if (c < 2 * n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) (isq ? V.F : V.D)[(c >> 1) * GDN_RS + 4 * kk + e] = acc[e];
    }
    key_cells(cb, 0, mhi, bv, ka);
  }
}

// The row-block count (16 nodes each) picks the instantiation, so that all
// of a column block's operand reads are unconditional and issue together.
template <int DK>
__device__ void gdn_front_lds(GdnView &V, int n, const QkPlanes &Q, const SrowOperand<DK> &S, float a0, float b0,
                              unsigned long long m0) {
  const int nrb = (n + 15) / 16;
  if (nrb <= 1)
    gdn_front_lds_rb<DK, 1>(V, n, Q, S);
  else if (nrb <= 2)
    gdn_front_lds_rb<DK, 2>(V, n, Q, S);
  else
    gdn_front_lds_rb<DK, DDT_MAX_NODES / 16>(V, n, Q, S);
  const int tid = threadIdx.x;
  if (tid < n) {
    V.al[tid] = a0;
    V.be[tid] = b0;
    V.anc[tid] = m0;
  }
}

// The depth class of a tree from the masks (lane j < n holds node j's),
// the same in every lane: 4, 8 or GDN_PATH when every node's level count
// (its mask's popcount) fits, else 64.  The solve only compares the level
// count with those bounds, and three ballots decide that without the
// cross-lane round trips of a maximum.
__device__ __forceinline__ int gdn_nlev(int n, unsigned long long a) {
  const int lane = threadIdx.x & 63;
  const int d = lane < n ? __popcll(a) : 0;
  if (__ballot(d > GDN_PATH)) return 64;
  if (__ballot(d > 8)) return GDN_PATH;
  if (__ballot(d > 4)) return 8;
  return 4;
}

// ------------------------------------------------------------ register path solve
// One lane per (node i, rows r0..r0+RW-1): u of every node on i's root path,
// root first, then i's outputs.  Requires every node's depth < PMAX; the
// loops are unrolled to PMAX levels (and predicated per lane), so the
// caller picks the smallest PMAX that holds the tree.  The operations for
// an element do not depend on PMAX or RW: RW = 2 (trees of up to 32 nodes)
// puts two lanes on a node, so a wavefront issues half the row arithmetic.
template <bool WANT_O, int PMAX, int RW>
__device__ void gdn_path_solve(GdnView &V, int n, float scale) {
  static_assert(PMAX <= GDN_PATH, "register path bound");
  static_assert(RW == 2 || RW == 4, "rows per lane");
  typedef float vec __attribute__((ext_vector_type(RW)));
  constexpr int NL = 256 * RW / GDN_R;  // node lanes: 64 (RW 4) or 32 (RW 2)
  const int i = threadIdx.x % NL, r0 = (threadIdx.x / NL) * RW;
  if (i >= n || r0 >= GDN_R) return;
  const unsigned long long anc = V.anc[i] & ((2ull << i) - 1);
  const int d = min(__popcll(anc) - 1, PMAX - 1);
  // path root first; slots past the node hold the node itself, so every
  // slot is a valid index and the loops below need no per-lane branches
  // (their results past depth d are computed and never used)
  int p[PMAX];
  {
    unsigned long long bits = anc;
#pragma unroll
    for (int k = 0; k < PMAX; ++k) {
      p[k] = bits ? __ffsll((long long)bits) - 1 : i;
      bits &= bits - 1;
    }
  }
  float al[PMAX], be[PMAX], g[PMAX][PMAX];
  vec Dk[PMAX], vk[PMAX];
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    al[k] = V.al[p[k]];
    be[k] = V.be[p[k]];
    Dk[k] = *reinterpret_cast<const vec *>(V.D + p[k] * GDN_RS + r0);
    vk[k] = *reinterpret_cast<const vec *>(V.v + p[k] * GDN_RS + r0);
#pragma unroll
    for (int j = 0; j < k; ++j) g[j][k] = V.Gm[p[j] * V.gs + 2 * p[k]];  // k_j . k_k
  }
  vec u[PMAX], ul = (vec)(0.f);
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    const float ba = be[k] * al[k];
    float w = 1.f;
    vec acc = (vec)(0.f);
#pragma unroll
    for (int j = k - 1; j >= 0; --j) {  // ancestors nearest first
      const float m = -(ba * (w * g[j][k]));
#pragma unroll
      for (int e = 0; e < RW; ++e) acc[e] = fmaf(m, u[j][e], acc[e]);
      w *= al[j];
    }
    const float c1 = -(al[k] * w);
#pragma unroll
    for (int e = 0; e < RW; ++e) u[k][e] = fmaf(be[k], fmaf(c1, Dk[k][e], vk[k][e]), acc[e]);
    if (k == d) ul = u[k];
  }
  *reinterpret_cast<vec *>(V.U + i * GDN_RS + r0) = ul;
  if (WANT_O) {
    float hq[PMAX];
#pragma unroll
    for (int j = 0; j < PMAX; ++j) hq[j] = V.Gm[p[j] * V.gs + 2 * i + 1];  // k_j . q_i
    const vec Fi = *reinterpret_cast<const vec *>(V.F + i * GDN_RS + r0);
    const float kqd = V.Gm[i * V.gs + 2 * i + 1];
    float w = 1.f, ai = 0.f;
    vec y = (vec)(0.f);
#pragma unroll
    for (int j = PMAX - 1; j >= 0; --j) {
      if (j == d) ai = al[j];
      const bool on = j < d;  // ancestors of i, nearest first
      const float hh = w * hq[j];
#pragma unroll
      for (int e = 0; e < RW; ++e) y[e] = on ? fmaf(hh, u[j][e], y[e]) : y[e];
      w = on ? w * al[j] : w;
    }
    vec o;
#pragma unroll
    for (int e = 0; e < RW; ++e) o[e] = scale * fmaf(ai, fmaf(w, Fi[e], y[e]), ul[e] * kqd);
    *reinterpret_cast<vec *>(V.O + i * GDN_RS + r0) = o;
  }
}

template <bool WANT_O, int PMAX>
__device__ void gdn_path_solve(GdnView &V, int n, float scale) {
  if (n <= 32)
    gdn_path_solve<WANT_O, PMAX, 2>(V, n, scale);
  else
    gdn_path_solve<WANT_O, PMAX, 4>(V, n, scale);
}

// ------------------------------------------------------------ deep-tree solve
// Level lists, run by one wavefront: lane j < n holds node j's ancestor mask.
// lvl = nodes ordered by (depth, index), pos = inverse, lvs[d] = first
// position of depth d, meta[0] = number of levels.
__device__ void gdn_levels(GdnView &V, int n, unsigned long long a) {
  const int lane = threadIdx.x & 63;
  const bool on = lane < n;
  const int d = on ? __popcll(a) - 1 : 64;
  // depths of a plan's tree are contiguous (0..levels-1); the bound on dd
  // keeps a corrupt mask from looping, and pos stays in range regardless
  int base = 0, pos = min(lane, n - 1), dd = 0;
  for (; dd < 64 && base < n; ++dd) {
    const unsigned long long m = __ballot(d == dd);
    if (d == dd) pos = base + __popcll(m & ((1ull << lane) - 1));
    if (lane == 0) V.lvs[dd] = base;
    base += __popcll(m);
  }
  if (lane == 0) {
    V.lvs[dd] = n;
    V.meta[0] = dd;
  }
  if (on) {
    V.lvl[pos] = lane;
    V.pos[lane] = pos;
  }
}

// Next (up to) eight ancestors of a node from `bits`, nearest first; -1 pads.
__device__ __forceinline__ void next8(unsigned long long &bits, int (&a)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    a[t] = bits ? top_bit(bits) : -1;
    if (a[t] >= 0) bits &= ~(1ull << a[t]);
  }
}

// One record per node, stored at its level-order position.
__device__ void gdn_records(GdnView &V, int n) {
  static_assert(GDN_MAXA == 8, "records hold eight ancestors");
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    GdnRec R;
    const float ai = V.al[i], bi = V.be[i], ba = bi * ai;
    unsigned long long bits = V.anc[i] & ((1ull << i) - 1);
    int a[8];
    next8(bits, a);
    float G[8], H[8], A[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int x = a[t] < 0 ? i : a[t];
      G[t] = V.Gm[x * V.gs + 2 * i];
      H[t] = V.Gm[x * V.gs + 2 * i + 1];
      A[t] = V.al[x];
    }
    __builtin_amdgcn_sched_barrier(0);
    float w = 1.f;
    int cnt = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (a[t] >= 0) {
        R.a[t] = a[t];
        R.m[t] = -(ba * (w * G[t]));
        R.h[t] = w * H[t];
        w *= A[t];
        ++cnt;
      } else {
        R.a[t] = i;
        R.m[t] = 0.f;
        R.h[t] = 0.f;
      }
    }
    R.wM = w;
    while (bits) {
      const int x = top_bit(bits);
      bits &= ~(1ull << x);
      w *= V.al[x];
    }
    R.i = i;
    R.cnt = cnt;
    R.bi = bi;
    R.ai = ai;
    R.P = w;
    R.c1 = -(ai * w);
    R.kqd = V.Gm[i * V.gs + 2 * i + 1];
    V.rec[min(V.pos[i], n - 1)] = R;
  }
}

// u (and, when WANT_O, the output) of one node for row r.  The node's loads
// go out first, then `between` runs (the caller's prefetch), then the
// arithmetic: the same operations, in the same order, as the path solve.
template <bool WANT_O, class Between>
__device__ __forceinline__ void gdn_node(GdnView &V, const GdnRec &R, int n, int r, float scale,
                                         Between between) {
  // indices are clamped so that even a corrupt plan cannot send a read
  // outside the arrays
  const int i = min((unsigned)R.i, (unsigned)(n - 1));
  float Ua[GDN_MAXA];
#pragma unroll
  for (int t = 0; t < GDN_MAXA; ++t) Ua[t] = V.U[min((unsigned)R.a[t], (unsigned)(n - 1)) * GDN_RS + r];
  const float Di = V.D[i * GDN_RS + r], vi = V.v[i * GDN_RS + r];
  const float Fi = WANT_O ? V.F[i * GDN_RS + r] : 0.f;
  between();
  __builtin_amdgcn_sched_barrier(0);
  float acc = 0.f, y = 0.f;
#pragma unroll
  for (int t = 0; t < GDN_MAXA; ++t)
    if (t < R.cnt) {
      acc = fmaf(R.m[t], Ua[t], acc);
      if (WANT_O) y = fmaf(R.h[t], Ua[t], y);
    }
  if (R.cnt == GDN_MAXA) {  // ancestors past the recorded ones
    unsigned long long bits = V.anc[i] & ((1ull << (R.a[GDN_MAXA - 1] & 63)) - 1) & ((1ull << i) - 1);
    const float ba = R.bi * R.ai;
    float w = R.wM;
    while (bits) {
      const int a = top_bit(bits);
      bits &= ~(1ull << a);
      const float ua = V.U[a * GDN_RS + r];
      acc = fmaf(-(ba * (w * V.Gm[a * V.gs + 2 * i])), ua, acc);
      if (WANT_O) y = fmaf(w * V.Gm[a * V.gs + 2 * i + 1], ua, y);
      w *= V.al[a];
    }
  }
  const float u = fmaf(R.bi, fmaf(R.c1, Di, vi), acc);
  V.U[i * GDN_RS + r] = u;
  if (WANT_O) V.O[i * GDN_RS + r] = scale * fmaf(R.ai, fmaf(R.P, Fi, y), u * R.kqd);
}

__device__ __forceinline__ GdnRec load_rec(const GdnView &V, int p) {
  GdnRec R;
  const gu32x4 *src = reinterpret_cast<const gu32x4 *>(V.rec + p);
  gu32x4 *dst = reinterpret_cast<gu32x4 *>(&R);
#pragma unroll
  for (int t = 0; t < (int)(sizeof(GdnRec) / 16); ++t) dst[t] = src[t];
  return R;
}

// Level-by-level solve for deep trees.  Needs 256 threads: thread t handles
// row t / 16 and slot t % 16; a row's threads share one wavefront, so the
// results of one level are visible to the next without a workgroup
// barrier.  Level starts live in one register (lane d holds lvs[d]); the
// record of the next level is loaded while the current one is computed.
template <bool WANT_O>
__device__ void gdn_level_solve(GdnView &V, int n, float scale) {
  const int r = threadIdx.x >> 4, slot = threadIdx.x & 15, lane = threadIdx.x & 63;
  const int nlev = __builtin_amdgcn_readfirstlane(V.meta[0]);
  const int lvv = V.lvs[min(lane, nlev)];
  auto lvs = [&](int d) { return d >= nlev ? n : __builtin_amdgcn_readlane(lvv, d); };
  int p = slot, pe = lvs(1);
  GdnRec cur = load_rec(V, min(p, n - 1)), nxt;
  for (int d = 0; d < nlev; ++d) {
    const int pn = lvs(d + 1) + slot, pen = lvs(d + 2);
    auto prefetch = [&]() { nxt = load_rec(V, min(pn, n - 1)); };
    if (p < pe)
      gdn_node<WANT_O>(V, cur, n, r, scale, prefetch);
    else
      prefetch();
    for (int q = p + 16; q < pe; q += 16) gdn_node<WANT_O>(V, load_rec(V, min(q, n - 1)), n, r, scale, [] {});
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
    p = pn;
    pe = pen;
  }
}

// The whole scalar part after the products, called by every thread of a
// 256-thread workgroup after a barrier that follows gdn_front.  `nlev` (a
// bound on the tree's levels, such as gdn_nlev's class) must be the same in
// every thread.
template <bool WANT_O>
__device__ void gdn_scalar(GdnView &V, int n, int nlev, float scale) {
  if (nlev <= 4) {
    gdn_path_solve<WANT_O, 4>(V, n, scale);
  } else if (nlev <= 8) {
    gdn_path_solve<WANT_O, 8>(V, n, scale);
  } else if (nlev <= GDN_PATH) {
    gdn_path_solve<WANT_O, GDN_PATH>(V, n, scale);
  } else {
    if (threadIdx.x < 64) gdn_levels(V, n, threadIdx.x < n ? V.anc[threadIdx.x] : 0ull);
    __syncthreads();
    gdn_records(V, n);
    __syncthreads();
    gdn_level_solve<WANT_O>(V, n, scale);
  }
}

// State of node i for columns c0..c0+7 of committed row Srow (global), from
// the keys (global rows krow(a)), the gates and u (LDS) of the node and its
// ancestors.  The same operations, in the same order, as the commit's
// rebuild from saved u.
template <class KRow>
__device__ __forceinline__ void gdn_state(const GdnView &V, int i, int r, int c0, const float *Srow,
                                          KRow krow, float (&s)[8]) {
  const float ai = V.al[i];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
  unsigned long long bits = V.anc[i] & ((1ull << i) - 1);
  float w = 1.f;
  while (bits) {
    const int a = top_bit(bits);
    bits &= ~(1ull << a);
    const float c = (ai * w) * V.U[a * GDN_RS + r];
    float ka[8];
    load8(krow(a) + c0, ka);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = fmaf(c, ka[e], s[e]);
    w *= V.al[a];
  }
  float sc[8], ki[8];
  ld8f(Srow + c0, sc);
  load8(krow(i) + c0, ki);
  const float cs = ai * w, ui = V.U[i * GDN_RS + r];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = fmaf(ui, ki[e], fmaf(cs, sc[e], s[e]));
}

}  // namespace ddt
