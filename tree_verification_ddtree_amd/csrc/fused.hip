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
// head (2*dk channels) and its own 16 v channels, for every node of the
// tree, from one round of global loads (x rows, taps, prefix rows, conv
// windows, and already the committed rows and gates the products need
// later, so that their latency hides under the conv).  The x slice is
// staged in LDS, where it aliases the delta-net area that is only filled
// afterwards.  A thread convolves 8 channels of a node at a time; the lanes
// holding one q or k row add their squares, normalise, and store the row as
// two bf16 planes hi and lo (hi + lo is the layer's q or k, within 2^-16 of
// the normalised value and exact in fp32), which are the matrix-core
// operands of the products as they stand (gdn_front_lds); the rest is the
// delta-net kernel's solve.  Sixteen workgroups share a key head and each computes its q and k
// itself: 2*dk*(n + W-1) extra reads from L2 per workgroup instead of a
// second launch.
#include "gdn_wy.h"

namespace ddt {

constexpr float FUSED_EPS = 1e-6f;

// LDS carve-up (bytes): the delta-net area first, with the prologue's
// staging aliasing it (prefix and node rows [W_max - 1 + nmax][2 dk + 16]
// and the taps [W_max][2 dk + 16], fp32); then the q and k rows as four
// bf16 planes q hi, q lo, k hi, k lo [nmax][dk + 8] (8 elements of padding
// keep the operand reads of 16 rows on distinct banks) and the conv
// windows as staged rows [nmax][W_max].
struct FusedLds {
  GdnLds g;
  int ldh, xw;
  size_t qk, win, total;
  __host__ __device__ FusedLds(int nmax, int dk) : g(nmax) {
    auto up = [](size_t x) { return (x + 15) / 16 * 16; };
    ldh = dk + 8;
    xw = 2 * dk + GDN_R;
    const size_t xs_bytes = (size_t)(nmax + 2 * DDT_MAX_W - 1) * xw * 4;  // staged rows + tap rows
    qk = up(g.total > xs_bytes ? g.total : xs_bytes);
    win = up(qk + (size_t)4 * nmax * ldh * 2);
    total = up(win + (size_t)nmax * DDT_MAX_W * 4);
  }
};

// Everything the first round of loads needs comes first among the
// arguments, in 14 dwords: the library is built to preload the first
// argument dwords into scalar registers at dispatch (14 of its 16 user
// registers are free for them), so those loads wait for no argument fetch.
// sizes = n_max | W << 8 | dv << 16, heads = Hk | Hv << 16.
template <typename T, int DK, int MW>
__global__ __launch_bounds__(256, 1) void fused_kernel(int plan_B, int plan_n_total, int sizes, int heads,
                                                       const float *__restrict__ S_c, const T *__restrict__ x,
                                                       const T *__restrict__ prefix, const T *__restrict__ w,
                                                       int32_t *plan_win, const float *__restrict__ alpha,
                                                       const float *__restrict__ beta, ddt_plan P, float scale,
                                                       float *__restrict__ out, float *__restrict__ q_out,
                                                       float *__restrict__ k_out, float *__restrict__ v_out,
                                                       float *__restrict__ node_states, float *__restrict__ node_u) {
  // MW: conv width class (4 or 8); taps at or past W are zero
  P.B = plan_B;
  P.n_total = plan_n_total;
  P.n_max = sizes & 0xff;
  P.W = (sizes >> 8) & 0xff;
  P.win = plan_win;
  const int dv = (int)((unsigned)sizes >> 16), Hk = heads & 0xffff, Hv = (int)((unsigned)heads >> 16);
  constexpr int UE = 16 / (int)sizeof(T);     // elements per 16-byte piece
  constexpr int XW = 2 * DK + GDN_R;          // staged channels per node: q, k of the key head, v of the tile
  constexpr int PPN = XW / UE;                // pieces per node row
  constexpr int LPR = DK / 8;                 // lanes per state row when storing states
  extern __shared__ float4 lds4[];
  char *base = reinterpret_cast<char *>(lds4);
  const FusedLds FL(P.n_max, DK);
  GdnView V(base, FL.g, P.n_max);
  float *xs = reinterpret_cast<float *>(base);  // prologue only
  uint16_t *qk = reinterpret_cast<uint16_t *>(base + FL.qk);  // planes q hi, q lo, k hi, k lo
  const int ldh = FL.ldh;
  const size_t plane = (size_t)P.n_max * ldh;
  const QkPlanes Q{qk, qk + plane, qk + 2 * plane, qk + 3 * plane, ldh};
  int *wins = reinterpret_cast<int *>(base + FL.win);
  const int b = blockIdx.z, h = blockIdx.y, row0 = blockIdx.x * GDN_R;
  const int tid = threadIdx.x;
  const Seq s = seq_of(P, b);
  const int n = __builtin_amdgcn_readfirstlane(s.n);
  if (n == 0) return;
  const int g = h / (Hv / Hk);
  const int W = P.W, W1 = W - 1;
  const size_t C = (size_t)2 * Hk * DK + (size_t)Hv * dv;
  // global channel of staged channel lc (selects, no branches)
  const int gq0 = g * DK, gk0 = Hk * DK + g * DK - DK, gv0 = 2 * Hk * DK + h * dv + row0 - 2 * DK;
  auto gch = [&](int lc) -> int { return lc + (lc < DK ? gq0 : (lc < 2 * DK ? gk0 : gv0)); };
  // ---- one round of loads.  Staged rows: the W-1 prefix rows (oldest
  // first), then the n node rows, so that every conv window entry names a
  // staged row.  Taps are staged too, tap-major (row j = j tokens back).
  const int R = W1 + n;
  float *tw = xs + (size_t)(W1 + P.n_max) * XW;
  constexpr int NWE = (DDT_MAX_NODES * MW + 255) / 256;  // window entries per thread
  constexpr int RPR = 256 / PPN;  // staged rows per pass of the workgroup (one piece column per thread)
  constexpr int NRR = 4;          // passes of the first round
  const int ne = n * MW, W1w = W1 > 0 ? W1 : 1;  // plan rows hold max(W-1, 1) entries
  const int pc = tid % PPN, pr = tid / PPN;      // this thread's piece column and first row
  const bool pon = pr < RPR;
  const int gc = gch(pc * UE);
  auto row_src = [&](int row) {
    const bool pre = row < W1;
    const size_t o = pre ? ((size_t)b * W1 + row) * C : (size_t)(s.o + row - W1) * C;
    return (pre ? prefix : x) + o + gc;
  };
  // A staged row is two planes of XW / 2 floats: channels 8 c .. 8 c + 3
  // at 4 c of the first, 8 c + 4 .. 8 c + 7 at 4 c of the second.  The conv
  // reads 8 channels as one 16-byte slot of each plane, so the 16 lanes of a
  // read that take adjacent 8-channel groups cover 256 contiguous bytes, all
  // the banks once (8 floats side by side would put lanes c and c + 8 on
  // the same banks).
  auto put_piece = [&](int row, gu32x4 v) {
    float f[UE];
    piece_f32<T>(v, f);
    const int c4 = pc * UE / 4;  // first group of 4 channels of the piece
    float *d = xs + row * XW + (c4 & 1) * (XW / 2) + (c4 >> 1) * 4;
    *reinterpret_cast<gf32x4 *>(d) = gf32x4{f[0], f[1], f[2], f[3]};
    if constexpr (UE == 8) *reinterpret_cast<gf32x4 *>(d + XW / 2) = gf32x4{f[4], f[5], f[6], f[7]};
  };
  // every first-round global load is issued before any store (a store
  // waits for its value, and for everything issued before it): the
  // committed rows first (their split into bf16 parts runs while the rest
  // is on its way), then x / prefix pieces, taps, window entries, and this
  // thread's gates and mask, which are needed only after the conv
  const float *Srows = S_c + (((size_t)b * Hv + h) * dv + row0) * DK;
  const bool s_wave = (tid >> 6) < (2 * n + 15) / 16;  // wavefronts that form committed-row products
  SrowOperand<DK> So;
  if (s_wave) So.load(Srows);
  gu32x4 r[NRR];
#pragma unroll
  for (int u = 0; u < NRR; ++u) r[u] = ld16(row_src(min(pr + RPR * u, R - 1)));
  constexpr int NTC = (XW + 255) / 256;  // staged channels per thread for the taps
  float tl[NTC][MW];
#pragma unroll
  for (int q = 0; q < NTC; ++q) {
    const T *wc = w + (size_t)gch(min(tid + 256 * q, XW - 1)) * W;
#pragma unroll
    for (int k = 0; k < MW; ++k) tl[q][k] = load1(wc + min(k, W - 1));
  }
  int wr[NWE];
#pragma unroll
  for (int k = 0; k < NWE; ++k) {
    const int e = min(tid + 256 * k, ne - 1), i = e / MW, j = e % MW;
    wr[k] = P.win[(size_t)(s.o + i) * W1w + min(max(j - 1, 0), W1w - 1)];
  }
  // every other argument, fetched in one round while those loads are in
  // flight (the compiler would otherwise fetch each group where it is first
  // used, one wait each)
  asm volatile("" ::"s"(P.anc), "s"(alpha), "s"(beta), "s"(scale), "s"(out), "s"(q_out), "s"(k_out), "s"(v_out),
               "s"(node_states), "s"(node_u));
  auto anc_of = [&](int j) { return (P.anc[s.o + j] & ((2ull << j) - 1)) | (1ull << j); };
  const int jt = min(tid, n - 1);
  const float a0 = alpha[(size_t)(s.o + jt) * Hv + h], b0 = beta[(size_t)(s.o + jt) * Hv + h];
  const unsigned long long m0 = anc_of(jt);
  if (s_wave) So.split();
  // ---- stores into the staging area
#pragma unroll
  for (int u = 0; u < NRR; ++u)
    if (pon && pr + RPR * u < R) put_piece(pr + RPR * u, r[u]);
  for (int r0 = pr + RPR * NRR; r0 < R; r0 += RPR * NRR) {  // more rows than one round holds
    if (!pon) break;
    gu32x4 rr[NRR];
#pragma unroll
    for (int u = 0; u < NRR; ++u) rr[u] = ld16(row_src(min(r0 + RPR * u, R - 1)));
#pragma unroll
    for (int u = 0; u < NRR; ++u)
      if (r0 + RPR * u < R) put_piece(r0 + RPR * u, rr[u]);
  }
  // taps, tap-major: row j = j tokens back (memory index W-1-j), zero past W
#pragma unroll
  for (int q = 0; q < NTC; ++q) {
    const int c = tid + 256 * q;
    if (c < XW) {
#pragma unroll
      for (int k = 0; k < MW; ++k) {
        if (k < W) tw[(W - 1 - k) * XW + c] = tl[q][k];
        if (k >= W) tw[k * XW + c] = 0.f;
      }
    }
  }
  // staged rows of every node's window, MW per node: the node itself, then
  // its previous tokens (node j: row W-1+j; prefix slot s: row s); entries
  // at or past W, whose taps are zero, repeat the node's own row
#pragma unroll
  for (int k = 0; k < NWE; ++k) {
    const int e = tid + 256 * k;
    if (e < ne) {
      const int i = e / MW, j = e % MW, src = wr[k];
      int rw = W1 + i;
      if (j >= 1 && j < W) rw = src >= 0 ? W1 + min(src, n - 1) : min(-src - 1, W1 - 1);
      wins[e] = rw;
    }
  }
  __syncthreads();
  // ---- the conv.  Task = 8 channels of one node.  Thread t owns q|k chunk
  // t % QKC for nodes t / QKC + NG k, and (vt = 255 - t < 2n) v chunk vt % 2
  // of node vt / 2: the v tasks go to the last wavefronts, whose q|k tasks
  // run out first when n is not a multiple of NG.
  constexpr int QKC = 2 * DK / 8;
  constexpr int NG = 256 / QKC;
  const int vt = 255 - tid;
  const int qc = tid % QKC, ng = tid / QKC, vch = vt & 1, iv = min(vt >> 1, n - 1);
  float tq[MW][8], tvv[MW][8];
#pragma unroll
  for (int j = 0; j < MW; ++j) {
    ld8f(tw + j * XW + 8 * qc, tq[j]);
    ld8f(tw + j * XW + 2 * DK + 8 * vch, tvv[j]);
  }
  // y = SiLU(sum_j tap_j tok_j(i)) for 8 channels from lc0 (tok_0 = node i);
  // no branches, so that all of a task's reads issue together
  auto conv8 = [&](int i, int lc0, const float (&tp)[MW][8], float (&y)[8]) {
    int rows[MW];
#pragma unroll
    for (int j = 0; j < MW; j += 4) {
      const int4 r4 = *reinterpret_cast<const int4 *>(wins + i * MW + j);
      rows[j] = r4.x;
      rows[j + 1] = r4.y;
      rows[j + 2] = r4.z;
      rows[j + 3] = r4.w;
    }
    float xv[MW][8];
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      const float4 a = *reinterpret_cast<const float4 *>(xs + rows[j] * XW + lc0 / 2);
      const float4 c = *reinterpret_cast<const float4 *>(xs + rows[j] * XW + XW / 2 + lc0 / 2);
      xv[j][0] = a.x, xv[j][1] = a.y, xv[j][2] = a.z, xv[j][3] = a.w;
      xv[j][4] = c.x, xv[j][5] = c.y, xv[j][6] = c.z, xv[j][7] = c.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = tp[0][e] * xv[0][e];
#pragma unroll
      for (int j = 1; j < MW; ++j) a = fmaf(tp[j][e], xv[j][e], a);
      y[e] = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
    }
  };
  // q and k rows: the DK / 8 lanes that hold one row (aligned groups of
  // adjacent lanes) add their squares, so every thread normalises its own
  // 8 values and stores their bf16 parts hi and lo in the planes (hi + lo is
  // the layer's q or k, within 2^-16 of the normalised value, plus the
  // hardware reciprocal square root's one ulp); the workgroup that hands q
  // and k out writes hi + lo as fp32
  {
    const int nk = (n + NG - 1) / NG;  // tasks of the busiest thread, the same in every thread
    const bool isk = qc >= DK / 8;
    const int c0 = 8 * (isk ? qc - DK / 8 : qc);
    uint16_t *dh = const_cast<uint16_t *>(isk ? Q.kh : Q.qh) + c0, *dl = const_cast<uint16_t *>(isk ? Q.kl : Q.ql) + c0;
    float *ho = isk ? k_out : q_out;
    const bool hand = ho && blockIdx.x == 0 && h % (Hv / Hk) == 0;
    auto finish = [&](int i, const float (&y)[8]) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
      ss = group_sum<DK / 8>(ss);
      const float inv = __builtin_amdgcn_rsqf(ss + FUSED_EPS);
      float yn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) yn[e] = y[e] * inv;
      gu32x4 hi, lo;
      split_hilo8(yn, hi, lo);
      if (i < n) {
        *reinterpret_cast<gu32x4 *>(dh + i * ldh) = hi;
        *reinterpret_cast<gu32x4 *>(dl + i * ldh) = lo;
        if (hand) {
          float *o = ho + ((size_t)(s.o + i) * Hk + g) * DK + c0;
          *reinterpret_cast<gf32x4 *>(o) =
              gf32x4{hilo_value(hi, lo, 0), hilo_value(hi, lo, 1), hilo_value(hi, lo, 2), hilo_value(hi, lo, 3)};
          *reinterpret_cast<gf32x4 *>(o + 4) =
              gf32x4{hilo_value(hi, lo, 4), hilo_value(hi, lo, 5), hilo_value(hi, lo, 6), hilo_value(hi, lo, 7)};
        }
      }
    };
    constexpr int NKU = 3;  // tasks unrolled together (n <= 24 at DK = 128)
    if (nk <= NKU) {
      // independent tasks side by side: the window and row reads of all of
      // them issue together, and the SiLU of one hides the latency of another
      float y[NKU][8];
#pragma unroll
      for (int k = 0; k < NKU; ++k) conv8(min(ng + NG * k, n - 1), 8 * qc, tq, y[k]);
#pragma unroll
      for (int k = 0; k < NKU; ++k)
        if (k < nk) finish(ng + NG * k, y[k]);
    } else {
      for (int k = 0; k < nk; ++k) {
        const int i = ng + NG * k;
        float y[8];
        conv8(min(i, n - 1), 8 * qc, tq, y);
        finish(i, y);
      }
    }
  }
  float yv[8];
  if (192 - 64 * (tid >> 6) < 2 * n) {  // this wavefront holds v tasks
    conv8(iv, 2 * DK + 8 * vch, tvv, yv);
    // computed before the barrier (the compiler would move it to the stores)
    asm volatile("" ::"v"(yv[0]), "v"(yv[1]), "v"(yv[2]), "v"(yv[3]), "v"(yv[4]), "v"(yv[5]), "v"(yv[6]), "v"(yv[7]));
  }
  __syncthreads();  // the x staging is dead from here on
  if (vt < 2 * n) {
    st8f(V.v + iv * GDN_RS + 8 * vch, yv);
    if (v_out) st8f(v_out + ((size_t)(s.o + iv) * Hv + h) * dv + row0 + 8 * vch, yv);
  }
  // (the front reads only the q and k rows; the barrier after it orders V.v)
  gdn_front_lds<DK>(V, n, Q, So, a0, b0, m0);
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
    auto krow = [&](int a) { return PlaneRow{Q.kh + a * ldh, Q.kl + a * ldh}; };
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
#define DDT_FUSED(D, M)                                                                                   \
  do {                                                                                                    \
    (void)hipFuncSetAttribute((const void *)fused_kernel<T, D, M>,                                        \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                      \
    hipLaunchKernelGGL((fused_kernel<T, D, M>), grid, dim3(256), lds, st, P.B, P.n_total,                 \
                       P.n_max | (P.W << 8) | (dv << 16), Hk | (Hv << 16), S, (const T *)x, (const T *)pre,     \
                       (const T *)w, P.win, al, be, P, scale, out, qo, ko, vo, ns, nu);                        \
  } while (0)
#define DDT_FUSED_W(D)        \
  do {                        \
    if (P.W <= 4)             \
      DDT_FUSED(D, 4);        \
    else                      \
      DDT_FUSED(D, DDT_MAX_W); \
  } while (0)
  switch (dk) {
    case 16: DDT_FUSED_W(16); break;
    case 32: DDT_FUSED_W(32); break;
    case 64: DDT_FUSED_W(64); break;
    default: DDT_FUSED_W(128); break;
  }
#undef DDT_FUSED_W
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
  if (Hk < 1 || Hv < 1 || Hv % Hk || Hv > 65535) return DDT_E_SHAPE;  // (Hk, Hv and dv go in 16 bits each)
  if (dk != 16 && dk != 32 && dk != 64 && dk != 128) return DDT_E_SHAPE;
  if (dv < GDN_R || dv % GDN_R || dv > 65535) return DDT_E_SHAPE;
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
