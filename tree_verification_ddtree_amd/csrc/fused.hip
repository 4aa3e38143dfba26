// Fused linear-attention layer: tree conv -> SiLU -> split q | k | v -> L2
// norm of q and k -> tree gated delta-net, in one launch.
//
// The pages run a whole forward in one persistent dispatch with no host
// round trips between layers (lucebox-hub README, "01 · Megakernel") and
// list the tree conv and tree delta-net kernels of the DDTree verify side by
// side ("02 · DFlash DDtree", "Implemented here").  The layer stage between
// them is the Gated DeltaNet one (Yang, Kautz, Hatamizadeh, "Gated Delta
// Networks", 2024): a short causal conv with SiLU over the projected
// q | k | v channels, q and k L2-normalised per head, then the gated delta
// rule.  Conv channels are [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)], head-major;
// the norm is x / sqrt(sum x^2 + 1e-6).
//
// A workgroup owns 16 state rows of one value head, as the delta-net kernel
// does.  Its prologue computes what those rows need: the q and k of its key
// head (2*dk channels, with their norms) and its own 16 v channels, for
// every node of the tree, from one round of global loads (x rows, taps,
// prefix rows, conv windows).  The x slice is staged in LDS, where it
// aliases the delta-net area that is only filled afterwards.  The
// normalised q and k stay in LDS as fp32 rows and feed the matrix-core
// products directly (gdn_front_lds); the rest is the delta-net kernel's
// solve.  Sixteen workgroups share a key head and each computes its q and k
// itself: 2*dk*(n + W-1) extra reads from L2 per workgroup instead of a
// second launch.
#include "gdn_wy.h"

namespace ddt {

constexpr float FUSED_EPS = 1e-6f;

// LDS carve-up (bytes): the delta-net area first, with the x staging
// [nmax][2 dk + 16] fp32 aliasing it during the prologue; then q and k rows
// [nmax][dk + 4] fp32 (4 floats of padding keep the operand reads of 16
// rows on distinct banks), per-node partial sums of squares [nmax][4], and
// the conv windows [nmax][W_max - 1].
struct FusedLds {
  GdnLds g;
  int ldk, xw;
  size_t qn, kn, ssq, win, total;
  __host__ __device__ FusedLds(int nmax, int dk) : g(nmax) {
    auto up = [](size_t x) { return (x + 15) / 16 * 16; };
    ldk = dk + 4;
    xw = 2 * dk + GDN_R;
    const size_t xs_bytes = (size_t)nmax * xw * 4;
    qn = up(g.total > xs_bytes ? g.total : xs_bytes);
    kn = up(qn + (size_t)nmax * ldk * 4);
    ssq = up(kn + (size_t)nmax * ldk * 4);
    win = up(ssq + (size_t)nmax * 4 * 4);
    total = up(win + (size_t)nmax * (DDT_MAX_W - 1) * 4);
  }
};

// sum over aligned groups of G lanes (G up to 64); every lane of a group
// gets bitwise the same sum (each step adds one pair in both partners)
template <int G>
__device__ __forceinline__ float group_sum64(float v) {
  v = group_sum<(G < 16 ? G : 16)>(v);
  if (G >= 32) v += __shfl_xor(v, 16);
  if (G >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <typename T, int DK>
__global__ __launch_bounds__(256, 1) void fused_kernel(ddt_plan P, const T *__restrict__ x,
                                                       const T *__restrict__ prefix, const T *__restrict__ w,
                                                       const float *__restrict__ alpha,
                                                       const float *__restrict__ beta,
                                                       const float *__restrict__ S_c, int Hk, int Hv, int dv,
                                                       float scale, float *__restrict__ out,
                                                       float *__restrict__ q_out, float *__restrict__ k_out,
                                                       float *__restrict__ v_out, float *__restrict__ node_states,
                                                       float *__restrict__ node_u) {
  constexpr int MW = DDT_MAX_W;               // widest conv
  constexpr int UE = 16 / (int)sizeof(T);     // elements per 16-byte piece
  constexpr int XW = 2 * DK + GDN_R;          // staged channels per node: q, k of the key head, v of the tile
  constexpr int PPN = XW / UE;                // pieces per node row
  constexpr int G = DK < 64 ? DK : 64;        // lanes per norm group
  constexpr int LPR = DK / 8;                 // lanes per state row when storing states
  extern __shared__ float4 lds4[];
  char *base = reinterpret_cast<char *>(lds4);
  const FusedLds FL(P.n_max, DK);
  GdnView V(base, FL.g, P.n_max);
  float *xs = reinterpret_cast<float *>(base);  // prologue only
  float *qn = reinterpret_cast<float *>(base + FL.qn);
  float *kn = reinterpret_cast<float *>(base + FL.kn);
  float *ssq = reinterpret_cast<float *>(base + FL.ssq);
  int *wins = reinterpret_cast<int *>(base + FL.win);
  const int ldk = FL.ldk;
  const int b = blockIdx.z, h = blockIdx.y, row0 = blockIdx.x * GDN_R;
  const int tid = threadIdx.x;
  const Seq s = seq_of(P, b);
  const int n = s.n;
  if (n == 0) return;
  const int g = h / (Hv / Hk);
  const int W = P.W, W1 = W - 1;
  const size_t C = (size_t)2 * Hk * DK + (size_t)Hv * dv;
  // global channel of staged channel lc
  auto gch = [&](int lc) -> size_t {
    return lc < DK ? (size_t)g * DK + lc
                   : lc < 2 * DK ? (size_t)Hk * DK + (size_t)g * DK + (lc - DK)
                                 : (size_t)2 * Hk * DK + (size_t)h * dv + row0 + (lc - 2 * DK);
  };
  // ---- one round of loads
  const bool qk = tid < 2 * DK;           // thread owns q/k channel tid
  const int vc = tid & (GDN_R - 1);       // and v channel vc of nodes tid/16 + 16 r
  float tq[MW], tv[MW], pq[MW - 1], pv[MW - 1];  // taps (index j = j tokens back), prefix slots
  {
    const size_t cq = gch(qk ? tid : 0), cv = gch(2 * DK + vc);
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      tq[j] = j < W ? load1(w + cq * W + (W - 1 - j)) : 0.f;
      tv[j] = j < W ? load1(w + cv * W + (W - 1 - j)) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < MW - 1; ++j) {
      pq[j] = j < W1 ? load1(prefix + ((size_t)b * W1 + j) * C + cq) : 0.f;
      pv[j] = j < W1 ? load1(prefix + ((size_t)b * W1 + j) * C + cv) : 0.f;
    }
  }
  for (int e = tid; e < n * W1; e += blockDim.x) wins[e] = P.win[(size_t)s.o * W1 + e];
  {
    const int np = n * PPN;
    for (int p0 = tid; p0 < np; p0 += 4 * 256) {
      gu32x4 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = min(p0 + 256 * u, np - 1);
        const int j = p / PPN, lc = (p % PPN) * UE;
        r[u] = ld16(x + (size_t)(s.o + j) * C + gch(lc));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + 256 * u;
        if (p < np) {
          const int j = p / PPN, lc = (p % PPN) * UE;
          float f[UE];
          piece_f32<T>(r[u], f);
          float *d = xs + j * XW + lc;
          *reinterpret_cast<gf32x4 *>(d) = gf32x4{f[0], f[1], f[2], f[3]};
          if constexpr (UE == 8) *reinterpret_cast<gf32x4 *>(d + 4) = gf32x4{f[4], f[5], f[6], f[7]};
        }
      }
    }
  }
  __syncthreads();
  // conv + SiLU of staged channel lc at node i: y = act(sum_j tap_j tok_j(i)),
  // tok_0 = the node itself, tok_j = its j-th previous token (window entry)
  auto conv = [&](int i, int lc, const float (&tp)[MW], const float (&pr)[MW - 1]) {
    float acc = tp[0] * xs[i * XW + lc];
#pragma unroll
    for (int j = 1; j < MW; ++j) {
      if (j < W) {
        const int src = wins[i * W1 + j - 1];
        float v;
        if (src >= 0) {
          v = xs[min(src, n - 1) * XW + lc];
        } else {
          const int sl = min(-src - 1, W1 - 1);
          v = 0.f;
#pragma unroll
          for (int jj = 0; jj < MW - 1; ++jj) v = jj == sl ? pr[jj] : v;
        }
        acc = fmaf(tp[j], v, acc);
      }
    }
    return acc / (1.0f + __expf(-acc));
  };
  // ---- pass 1: sums of squares of q and k per node (one partial per group
  // of G lanes; a head is DK / G groups), and the v channels
  if (tid < 2 * DK) {
    for (int i = 0; i < n; ++i) {
      const float y = conv(i, tid, tq, pq);
      const float ss = group_sum64<G>(y * y);
      if ((tid & (G - 1)) == 0) ssq[i * 4 + tid / G] = ss;
    }
  }
  constexpr int VR = DDT_MAX_NODES * GDN_R / 256;  // v (node, channel) pairs per thread
  float yv[VR];
#pragma unroll
  for (int r = 0; r < VR; ++r) {
    const int j = tid / GDN_R + (256 / GDN_R) * r;
    yv[r] = j < n ? conv(j, 2 * DK + vc, tv, pv) : 0.f;
  }
  __syncthreads();
  // ---- pass 2: the same conv values, normalised, into the q and k rows
  if (tid < 2 * DK) {
    const int hg = (tid / DK) * (DK / G);  // first group of this thread's head
    for (int i = 0; i < n; ++i) {
      const float y = conv(i, tid, tq, pq);
      float nrm = ssq[i * 4 + hg];
      if (DK / G == 2) nrm += ssq[i * 4 + hg + 1];
      const float yn = y / sqrtf(nrm + FUSED_EPS);
      if (tid < DK)
        qn[i * ldk + tid] = yn;
      else
        kn[i * ldk + tid - DK] = yn;
    }
  }
  __syncthreads();  // the x staging is dead from here on
#pragma unroll
  for (int r = 0; r < VR; ++r) {
    const int j = tid / GDN_R + (256 / GDN_R) * r;
    if (j < n) {
      V.v[j * GDN_R + vc] = yv[r];
      if (v_out) v_out[((size_t)(s.o + j) * Hv + h) * dv + row0 + vc] = yv[r];
    }
  }
  // one workgroup per key head hands q and k out (for the commit)
  if ((q_out || k_out) && blockIdx.x == 0 && h % (Hv / Hk) == 0) {
    for (int e = tid; e < n * DK; e += blockDim.x) {
      const int i = e / DK, c = e % DK;
      const size_t o = ((size_t)(s.o + i) * Hk + g) * DK + c;
      if (q_out) q_out[o] = qn[i * ldk + c];
      if (k_out) k_out[o] = kn[i * ldk + c];
    }
  }
  const float *Srows = S_c + (((size_t)b * Hv + h) * dv + row0) * DK;
  auto gid = [&](int j) { return s.o + j; };
  auto anc_of = [&](int j) { return (P.anc[s.o + j] & ((2ull << j) - 1)) | (1ull << j); };
  gdn_front_lds<DK>(V, n, gid, anc_of, qn, kn, ldk, alpha, beta, Srows, Hv, h);
  __syncthreads();
  const int nlev = gdn_nlev(n, (tid & 63) < n ? V.anc[tid & 63] : 0ull);
  gdn_scalar<true>(V, n, nlev, scale);
  __syncthreads();
  for (int idx = tid; idx < n * 4; idx += blockDim.x) {
    const int i = idx >> 2, c = (idx & 3) * 4;
    *reinterpret_cast<float4 *>(out + ((size_t)(s.o + i) * Hv + h) * dv + row0 + c) =
        *reinterpret_cast<const float4 *>(V.O + i * GDN_R + c);
    if (node_u)
      *reinterpret_cast<float4 *>(node_u + ((size_t)(s.o + i) * Hv + h) * dv + row0 + c) =
          *reinterpret_cast<const float4 *>(V.U + i * GDN_R + c);
  }
  if (node_states && tid < GDN_R * LPR) {
    const int lr = tid / LPR, c0 = (tid % LPR) * 8;
    auto krow = [&](int a) { return kn + a * ldk; };
    for (int i = 0; i < n; ++i) {
      float st[8];
      gdn_state(V, i, lr, c0, Srows + lr * DK, krow, st);
      st8f(node_states + (((size_t)(s.o + i) * Hv + h) * dv + row0 + lr) * DK + c0, st);
    }
  }
}

int check_plan(const ddt_plan *P);

template <typename T>
static void launch_fused(int dk, dim3 grid, size_t lds, hipStream_t st, const ddt_plan &P, const void *x,
                         const void *pre, const void *w, const float *al, const float *be, const float *S,
                         int Hk, int Hv, int dv, float scale, float *out, float *qo, float *ko, float *vo,
                         float *ns, float *nu) {
#define DDT_FUSED(D)                                                                                   \
  do {                                                                                                 \
    (void)hipFuncSetAttribute((const void *)fused_kernel<T, D>,                                        \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                   \
    hipLaunchKernelGGL((fused_kernel<T, D>), grid, dim3(256), lds, st, P, (const T *)x, (const T *)pre, \
                       (const T *)w, al, be, S, Hk, Hv, dv, scale, out, qo, ko, vo, ns, nu);          \
  } while (0)
  switch (dk) {
    case 16: DDT_FUSED(16); break;
    case 32: DDT_FUSED(32); break;
    case 64: DDT_FUSED(64); break;
    default: DDT_FUSED(128); break;
  }
#undef DDT_FUSED
}

}  // namespace ddt

using namespace ddt;

extern "C" size_t ddt_tree_conv_gdn_lds(int32_t n_max, int32_t dk) {
  if (n_max < 1 || n_max > DDT_MAX_NODES || (dk != 16 && dk != 32 && dk != 64 && dk != 128)) return 0;
  return FusedLds(n_max, dk).total;
}

extern "C" int ddt_tree_conv_gdn(const ddt_plan *P, const void *x, const void *prefix, const void *w,
                                 int32_t dtype, const float *alpha, const float *beta, const float *S_c,
                                 int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale, float *out,
                                 float *q_out, float *k_out, float *v_out, float *node_states, float *node_u,
                                 void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!x || !w || !alpha || !beta || !S_c || !out || (P->W > 1 && !prefix)) return DDT_E_ARG;
  if (Hk < 1 || Hv < 1 || Hv % Hk) return DDT_E_SHAPE;
  if (dk != 16 && dk != 32 && dk != 64 && dk != 128) return DDT_E_SHAPE;
  if (dv < GDN_R || dv % GDN_R) return DDT_E_SHAPE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  const size_t lds = FusedLds(P->n_max, dk).total;
  if (lds > 160 * 1024) return DDT_E_SHAPE;
  dim3 grid(dv / GDN_R, Hv, P->B);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == DDT_BF16)
    launch_fused<uint16_t>(dk, grid, lds, st, *P, x, prefix, w, alpha, beta, S_c, Hk, Hv, dv, scale, out, q_out,
                           k_out, v_out, node_states, node_u);
  else
    launch_fused<float>(dk, grid, lds, st, *P, x, prefix, w, alpha, beta, S_c, Hk, Hv, dv, scale, out, q_out,
                        k_out, v_out, node_states, node_u);
  return launch_status();
}
