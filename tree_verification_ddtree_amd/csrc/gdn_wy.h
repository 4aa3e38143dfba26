// Gated delta rule over a tree of tokens in its WY form (shared by the tree
// kernel and the commit's replay).
//
// Row r of a value head's state evolves on its own: for node i with parent
// p, s_i = a_i s_p + u_i k_i with u_i = b_i (v_i - a_i s_p . k_i).  Unrolled
// along the root path, every s_p . x is a combination of the committed
// row's products S_c . x and of the keys of the ancestors:
//   s_p . x = P_i (S_c . x) + sum_{a ancestor of i} w(a,i) u_a (k_a . x)
// with w(a,i) the product of the gates strictly between a and i and P_i the
// product of the gates of all ancestors of i.  So, per row,
//   u_i = b_i (v_i - a_i P_i D_i) - sum_a M(i,a) u_a,  M(i,a) = b_i a_i w(a,i) k_a.k_i
//   o_i = scale (a_i (P_i F_i + sum_a w(a,i) (k_a.q_i) u_a) + u_i k_i.q_i)
//   s_i = a_i P_i S_c + sum_a a_i w(a,i) u_a k_a + u_i k_i
// where D_i = S_c . k_i and F_i = S_c . q_i.  The products D, F and the
// pair coefficients are independent work; only the scalar solve for u is
// ordered, by tree level, and needs no cross-lane reduction.
//
// Every dot product is a lane-group sum whose value does not depend on the
// position of the node in the batch, and every recurrence walks ancestors
// in the same order (nearest first), so a node's state comes out bitwise the
// same whether the tree or only its root path is processed.
#pragma once
#include "common.h"

namespace ddt {

// LDS carve-up, every array 16-byte aligned
struct GdnLds {
  size_t kq, v, al, be, P, kqd, anc, gid, dep, lvl, lvs, D, F, M, N, Wt, U, O, total;
  __host__ __device__ GdnLds(int nmax, int R, int dk) {
    auto up = [](size_t x) { return (x + 15) / 16 * 16; };
    const size_t nn = (size_t)nmax * nmax * 4;
    kq = 0;
    v = up(kq + (size_t)nmax * 2 * dk * 4);  // k, q as fp32
    al = up(v + (size_t)nmax * R * 4);
    be = up(al + (size_t)nmax * 4);
    P = up(be + (size_t)nmax * 4);
    kqd = up(P + (size_t)nmax * 4);
    anc = up(kqd + (size_t)nmax * 4);
    gid = up(anc + (size_t)nmax * 8);
    dep = up(gid + (size_t)nmax * 4);
    lvl = up(dep + (size_t)nmax * 4);
    lvs = up(lvl + (size_t)nmax * 4);
    D = up(lvs + (size_t)(nmax + 1) * 4);
    F = up(D + (size_t)R * nmax * 4);
    M = up(F + (size_t)R * nmax * 4);
    N = up(M + nn);
    Wt = up(N + nn);
    U = up(Wt + nn);
    O = up(U + (size_t)R * nmax * 4);
    total = up(O + (size_t)nmax * R * 4);
  }
};

struct GdnView {
  float *kq, *v, *al, *be, *P, *kqd, *D, *F, *M, *N, *Wt, *U, *O;
  unsigned long long *anc;
  int *gid, *dep, *lvl, *lvs;
  int nmax, R;
  __device__ GdnView(char *base, const GdnLds &L, int nmax_, int R_) : nmax(nmax_), R(R_) {
    kq = reinterpret_cast<float *>(base + L.kq);
    v = reinterpret_cast<float *>(base + L.v);
    al = reinterpret_cast<float *>(base + L.al);
    be = reinterpret_cast<float *>(base + L.be);
    P = reinterpret_cast<float *>(base + L.P);
    kqd = reinterpret_cast<float *>(base + L.kqd);
    anc = reinterpret_cast<unsigned long long *>(base + L.anc);
    gid = reinterpret_cast<int *>(base + L.gid);
    dep = reinterpret_cast<int *>(base + L.dep);
    lvl = reinterpret_cast<int *>(base + L.lvl);
    lvs = reinterpret_cast<int *>(base + L.lvs);
    D = reinterpret_cast<float *>(base + L.D);
    F = reinterpret_cast<float *>(base + L.F);
    M = reinterpret_cast<float *>(base + L.M);
    N = reinterpret_cast<float *>(base + L.N);
    Wt = reinterpret_cast<float *>(base + L.Wt);
    U = reinterpret_cast<float *>(base + L.U);
    O = reinterpret_cast<float *>(base + L.O);
  }
};

// closest ancestor of node i still in `bits` (indices grow along a root path)
__device__ __forceinline__ int top_bit(unsigned long long bits) { return 63 - __clzll((long long)bits); }

// dot of 8 local columns with an LDS row, finished over the lane group
template <int LPR>
__device__ __forceinline__ float ldot(const float (&a)[8], const float *b) {
  float bb[8];
  ld8f(b, bb);
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    d0 = fmaf(a[e], bb[e], d0);
    d1 = fmaf(a[e + 4], bb[e + 4], d1);
  }
  return group_sum<LPR>(d0 + d1);
}
template <int LPR>
__device__ __forceinline__ float ldot2(const float *a, const float *b) {
  float aa[8];
  ld8f(a, aa);
  return ldot<LPR>(aa, b);
}

// Stage the inputs of nodes gid[0..n) (global ids, already in LDS):
// k and q rows of key head g as fp32, v of the tile's rows, gates.
template <typename T, int DK>
__device__ void gdn_stage(GdnView &V, int n, const T *__restrict__ q, const T *__restrict__ k,
                          const T *__restrict__ v, const T *__restrict__ alpha,
                          const T *__restrict__ beta, int Hk, int Hv, int dv, int g, int h,
                          int row0) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int U = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int PPR = DK / U;             // pieces per k or q row
  constexpr int MAXP = 8;                 // pieces staged in registers per thread
  const int tid = threadIdx.x, nth = blockDim.x;
  const int np = n * 2 * PPR;
  auto src = [&](int idx) -> const u32x4 * {
    const int j = idx / (2 * PPR), which = (idx / PPR) & 1, pc = idx % PPR;
    return reinterpret_cast<const u32x4 *>((which ? q : k) + ((size_t)V.gid[j] * Hk + g) * DK) + pc;
  };
  auto put = [&](int idx, u32x4 x) {
    const int j = idx / (2 * PPR), which = (idx / PPR) & 1, pc = idx % PPR;
    float *dst = V.kq + ((size_t)j * 2 + which) * DK + pc * U;
    if constexpr (sizeof(T) == 2) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(x[i] << 16);
        f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
      }
      st8f(dst, f);
    } else {
      *reinterpret_cast<u32x4 *>(dst) = x;
    }
  };
  // every global load of this thread first (clamped indices), then the stores
  u32x4 buf[MAXP];
#pragma unroll
  for (int u = 0; u < MAXP; ++u) buf[u] = *src(min(tid + u * nth, np - 1));
  float vb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = min(tid + u * nth, n * V.R - 1);
    vb[u] = load1(v + ((size_t)V.gid[idx / V.R] * Hv + h) * dv + row0 + idx % V.R);
  }
  const int jt = min(tid, n - 1);
  const float a0 = load1(alpha + (size_t)V.gid[jt] * Hv + h);
  const float b0 = load1(beta + (size_t)V.gid[jt] * Hv + h);
#pragma unroll
  for (int u = 0; u < MAXP; ++u)
    if (tid + u * nth < np) put(tid + u * nth, buf[u]);
  for (int idx = tid + MAXP * nth; idx < np; idx += nth) put(idx, *src(idx));
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (tid + u * nth < n * V.R) V.v[tid + u * nth] = vb[u];
  for (int idx = tid + 4 * nth; idx < n * V.R; idx += nth)
    V.v[idx] = load1(v + ((size_t)V.gid[idx / V.R] * Hv + h) * dv + row0 + idx % V.R);
  if (tid < n) {
    V.al[tid] = a0;
    V.be[tid] = b0;
  }
  for (int j = tid + nth; j < n; j += nth) {
    V.al[j] = load1(alpha + (size_t)V.gid[j] * Hv + h);
    V.be[j] = load1(beta + (size_t)V.gid[j] * Hv + h);
  }
}

// Products with the committed rows and the per-node coefficients.
// Thread (lr, cg) owns columns c0..c0+7 of tile row lr; sc = those values.
// want_F: also S_c . q (outputs); coefs for nodes [0, n).
template <int LPR, int DK>
__device__ void gdn_products(GdnView &V, int n, const float (&sc)[8], int lr, int cg,
                             bool want_F) {
  const int c0 = cg * 8;
  // four nodes at a time so the lane-group sums of independent dots overlap
  for (int j0 = 0; j0 < n; j0 += 4) {
    float d[4], f[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(j0 + u, n - 1);
      d[u] = ldot<LPR>(sc, V.kq + (size_t)j * 2 * DK + c0);
      f[u] = want_F ? ldot<LPR>(sc, V.kq + ((size_t)j * 2 + 1) * DK + c0) : 0.f;
    }
    if (cg == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u < n) {
          V.D[lr * V.nmax + j0 + u] = d[u];
          V.F[lr * V.nmax + j0 + u] = f[u];
        }
    }
  }
  // pair coefficients: row group lr takes nodes i = lr, lr + R, ...
  for (int i = lr; i < n; i += V.R) {
    const float *ki = V.kq + (size_t)i * 2 * DK + c0;
    const float *qi = V.kq + ((size_t)i * 2 + 1) * DK + c0;
    const float ai = V.al[i], ba = V.be[i] * ai;
    unsigned long long bits = V.anc[i] & ~(1ull << i);
    float w = 1.f;
    while (bits) {
      const int a = top_bit(bits);
      bits &= ~(1ull << a);
      const float *ka = V.kq + (size_t)a * 2 * DK + c0;
      const float G = ldot2<LPR>(ka, ki);
      const float H = want_F ? ldot2<LPR>(ka, qi) : 0.f;
      if (cg == 0) {
        V.Wt[i * V.nmax + a] = w;
        V.M[i * V.nmax + a] = ba * (w * G);
        V.N[i * V.nmax + a] = w * H;
      }
      w *= V.al[a];
    }
    const float kqv = want_F ? ldot2<LPR>(ki, qi) : 0.f;
    if (cg == 0) {
      V.P[i] = w;
      V.kqd[i] = kqv;
    }
  }
}

// Level lists from dep[0..n): lvl = nodes ordered by (depth, index),
// lvs[d] = first position of depth d.  Returns the number of levels.
__device__ int gdn_levels(GdnView &V, int n) {
  int maxd = 0;
  for (int j = 0; j < n; ++j) maxd = max(maxd, V.dep[j]);
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    const int d = V.dep[t];
    int pos = 0;
    for (int j = 0; j < n; ++j) pos += (V.dep[j] < d) || (V.dep[j] == d && j < t);
    V.lvl[pos] = t;
  }
  for (int d = threadIdx.x; d <= maxd + 1; d += blockDim.x) {
    int c = 0;
    for (int j = 0; j < n; ++j) c += V.dep[j] < d;
    V.lvs[d] = c;
  }
  return maxd + 1;
}

// u for every (row, node), level by level.  Of the nth = R * lanes-per-row
// active threads, thread t handles row t / TS and slot t % TS; a row's threads share one wavefront, so results of one level
// are visible to the next without a workgroup barrier.
__device__ void gdn_solve(GdnView &V, int nlev, int nth) {
  const int TS = nth / V.R;
  const int r = threadIdx.x / TS, slot = threadIdx.x % TS;
  float *Ur = V.U + r * V.nmax;
  for (int d = 0; d < nlev; ++d) {
    for (int s = V.lvs[d] + slot; s < V.lvs[d + 1]; s += TS) {
      const int i = V.lvl[s];
      const float ai = V.al[i];
      float u = V.be[i] * fmaf(-(ai * V.P[i]), V.D[r * V.nmax + i], V.v[i * V.R + r]);
      unsigned long long bits = V.anc[i] & ~(1ull << i);
      while (bits) {
        const int a = top_bit(bits);
        bits &= ~(1ull << a);
        u = fmaf(-V.M[i * V.nmax + a], Ur[a], u);
      }
      Ur[i] = u;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// outputs o_i of every (row, node) into O[node][row]
__device__ void gdn_outputs(GdnView &V, int n, float scale, int nth) {
  const int TS = nth / V.R;
  const int r = threadIdx.x / TS, slot = threadIdx.x % TS;
  const float *Ur = V.U + r * V.nmax;
  for (int i = slot; i < n; i += TS) {
    float y = V.P[i] * V.F[r * V.nmax + i];
    unsigned long long bits = V.anc[i] & ~(1ull << i);
    while (bits) {
      const int a = top_bit(bits);
      bits &= ~(1ull << a);
      y = fmaf(V.N[i * V.nmax + a], Ur[a], y);
    }
    V.O[i * V.R + r] = scale * fmaf(V.al[i], y, Ur[i] * V.kqd[i]);
  }
}

// state of node i for this lane's 8 columns of row lr
template <int DK>
__device__ __forceinline__ void gdn_state(GdnView &V, int i, const float (&sc)[8], int lr, int cg,
                                          float (&s)[8]) {
  const int c0 = cg * 8;
  const float *Ur = V.U + lr * V.nmax;
  const float ai = V.al[i];
  const float cs = ai * V.P[i];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = cs * sc[e];
  unsigned long long bits = V.anc[i] & ~(1ull << i);
  while (bits) {
    const int a = top_bit(bits);
    bits &= ~(1ull << a);
    const float c = (ai * V.Wt[i * V.nmax + a]) * Ur[a];
    float ka[8];
    ld8f(V.kq + (size_t)a * 2 * DK + c0, ka);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = fmaf(c, ka[e], s[e]);
  }
  float ki[8];
  ld8f(V.kq + (size_t)i * 2 * DK + c0, ki);
  const float ui = Ur[i];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = fmaf(ui, ki[e], s[e]);
}

}  // namespace ddt
