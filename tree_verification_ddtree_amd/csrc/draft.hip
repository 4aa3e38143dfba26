// Ahead of the verify step: draft top-K, log-sum-exp and DDTree construction.
//
// The draft model's K most likely tokens (K from 1 to 8) and each draft
// position's log-sum-exp are read from the device logits in place
// (codehub lucebox-hub@main, "GPU draft top-K & verify-argmax (DFlash)"),
// and DDTree builds the budget-N tree of draft tokens that the verify step
// checks (lucebox-hub README, "02 · DFlash DDtree", "Algorithms used").
// The pages give no selection rule; the reading taken here: positions are
// drafted in one block, so a node at depth d has as candidate children the
// top-K tokens of draft position d (0-based); a node's score is the sum of
// the log-probabilities on its root path; the tree is the root plus the
// N-1 best nodes under (score descending, then the candidate ranks along
// the path lexicographically, a prefix first), which is closed under taking
// parents and is what best-first expansion selects.
//
//  draft_chunk_kernel  one workgroup per (sequence, position, chunk of the
//                      vocabulary): every thread keeps a sorted top-K and an
//                      online (max, sum of exponentials) over its elements
//                      (16-byte loads), then the workgroup merges them.
//  draft_merge_kernel  one wavefront per (sequence, position): merges the
//                      chunks into the top-K and the log-sum-exp.
//  draft_tree_kernel   one wavefront per sequence, one lane per tree node:
//                      each selected node offers its best unselected child;
//                      a wave-wide arg-best picks the next node, N-1 times.
// Every merge is a fixed pattern of exchanges over a strict total order, so
// results do not depend on timing.
#include "common.h"

namespace ddt {

constexpr int DRAFT_KMAX = 8;
constexpr int DRAFT_LMAX = 16;  // rank codes hold 16 levels of 4 bits
constexpr int DRAFT_CMAX = 64;  // vocabulary chunks per position (one lane each in the merge)
constexpr int DRAFT_EMPTY = 0x7fffffff;

// (logit a, index ia) ranks before (b, ib): larger logit, then lower index
__device__ __forceinline__ bool cand_before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// Insert (x, t) into a sorted list if it ranks before the last entry; an
// unrolled bubble, so the list stays in registers.
template <int K>
__device__ __forceinline__ void list_insert(float (&v)[K], int (&ix)[K], float x, int t) {
  if (!cand_before(x, t, v[K - 1], ix[K - 1])) return;
  v[K - 1] = x;
  ix[K - 1] = t;
#pragma unroll
  for (int k = K - 1; k > 0; --k) {
    const bool sw = cand_before(v[k], ix[k], v[k - 1], ix[k - 1]);
    const float tv = v[k];
    const int ti = ix[k];
    v[k] = sw ? v[k - 1] : v[k];
    ix[k] = sw ? ix[k - 1] : ix[k];
    v[k - 1] = sw ? tv : v[k - 1];
    ix[k - 1] = sw ? ti : ix[k - 1];
  }
}

// Partner lane's list merged into this lane's: both lanes end with the top-K
// of the union (the order is strict and the lists are disjoint).
template <int K>
__device__ __forceinline__ void list_xor_merge(float (&v)[K], int (&ix)[K], int mask) {
  float pv[K];
  int pi[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    pv[k] = __shfl_xor(v[k], mask);
    pi[k] = __shfl_xor(ix[k], mask);
  }
#pragma unroll
  for (int k = 0; k < K; ++k) list_insert<K>(v, ix, pv[k], pi[k]);
}

// (max, sum of 2^((x - max) log2 e)) pairs
__device__ __forceinline__ void ms_combine(float &m, float &s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;  // both empty
  const float a = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - mm) * 1.4426950408889634f);
  const float b = m2 == -INFINITY ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - mm) * 1.4426950408889634f);
  m = mm;
  s = a + b;  // commutative: both partner lanes get the same bits
}

__device__ __forceinline__ void ms_add(float &m, float &s, float x) {
  if (!(x > -INFINITY)) return;  // -inf and NaN add nothing
  if (x > m) {
    s = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - x) * 1.4426950408889634f);
    m = x;
  }
  s += __builtin_amdgcn_exp2f((x - m) * 1.4426950408889634f);
}

struct DraftWs {
  int2 *cand;  // [B][L][C][K] (logit bits, index)
  float2 *ms;  // [B][L][C] (max, sum)
};

template <typename T, int K>
__global__ __launch_bounds__(256) void draft_chunk_kernel(const T *__restrict__ logits, int L, int V, int C,
                                                          int chunk, int vec, DraftWs W) {
  const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const T *row = logits + ((size_t)b * L + i) * V;
  const int e0 = c * chunk, e1 = min(V, e0 + chunk);
  float v[K];
  int ix[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    v[k] = -INFINITY;
    ix[k] = DRAFT_EMPTY;
  }
  float m = -INFINITY, s = 0.f;
  if (vec) {
    // 8 elements per 16-byte (bf16) or 32-byte (fp32) read; e0 and the row
    // start are multiples of 8 elements, the ragged tail goes one by one
    const int nv = (e1 - e0) / 8;
    for (int j = tid; j < nv; j += 256) {
      float f[8];
      load8(row + e0 + 8 * j, f);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        if (f[x] > v[K - 1]) list_insert<K>(v, ix, f[x], e0 + 8 * j + x);
        ms_add(m, s, f[x]);
      }
    }
    for (int e = e0 + 8 * nv + tid; e < e1; e += 256) {
      const float f = load1(row + e);
      if (f > v[K - 1]) list_insert<K>(v, ix, f, e);
      ms_add(m, s, f);
    }
  } else {
    for (int e = e0 + tid; e < e1; e += 256) {
      const float f = load1(row + e);
      if (f > v[K - 1]) list_insert<K>(v, ix, f, e);
      ms_add(m, s, f);
    }
  }
  // wavefront: exchange with lanes 1, 2, ..., 32 apart
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    list_xor_merge<K>(v, ix, o);
    ms_combine(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
  }
  __shared__ float sv[4][K], sm[4], ss[4];
  __shared__ int si[4][K];
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      sv[w][k] = v[k];
      si[w][k] = ix[k];
    }
    sm[w] = m;
    ss[w] = s;
  }
  __syncthreads();
  if (tid == 0) {
    for (int q = 1; q < 4; ++q) {
#pragma unroll
      for (int k = 0; k < K; ++k) list_insert<K>(v, ix, sv[q][k], si[q][k]);
      ms_combine(m, s, sm[q], ss[q]);
    }
    const size_t r = ((size_t)b * L + i) * C + c;
#pragma unroll
    for (int k = 0; k < K; ++k) W.cand[r * K + k] = make_int2(__float_as_int(v[k]), ix[k]);
    W.ms[r] = make_float2(m, s);
  }
}

template <int K>
__global__ __launch_bounds__(64) void draft_merge_kernel(int L, int C, DraftWs W, int32_t *__restrict__ topk_idx,
                                                         float *__restrict__ topk_logit, float *__restrict__ lse) {
  const int i = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  float v[K];
  int ix[K];
  float m = -INFINITY, s = 0.f;
  const size_t r0 = ((size_t)b * L + i) * C;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    v[k] = -INFINITY;
    ix[k] = DRAFT_EMPTY;
  }
  if (lane < C) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int2 e = W.cand[(r0 + lane) * K + k];
      v[k] = __int_as_float(e.x);
      ix[k] = e.y;
    }
    const float2 p = W.ms[r0 + lane];
    m = p.x;
    s = p.y;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    list_xor_merge<K>(v, ix, o);
    ms_combine(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
  }
  if (lane < K) {
    // lane k writes entry k (read from the lane-uniform list by unrolled select)
    float vk = v[0];
    int ik = ix[0];
#pragma unroll
    for (int k = 1; k < K; ++k) {
      vk = lane == k ? v[k] : vk;
      ik = lane == k ? ix[k] : ik;
    }
    const bool ok = ik != DRAFT_EMPTY;
    topk_idx[((size_t)b * L + i) * K + lane] = ok ? ik : -1;
    topk_logit[((size_t)b * L + i) * K + lane] = ok ? vk : -INFINITY;
  }
  if (lane == 0) lse[(size_t)b * L + i] = m == -INFINITY ? -INFINITY : m + __logf(s);
}

// One wavefront per sequence; lane j is tree node j once selected.  A
// candidate is (score, code): code packs the candidate ranks along the root
// path, 4 bits per level from the top (rank + 1, 0 past the node's depth),
// so comparing codes as integers is the lexicographic order with a prefix
// first.
__global__ __launch_bounds__(64) void draft_tree_kernel(const int32_t *__restrict__ topk_idx,
                                                        const float *__restrict__ topk_logit,
                                                        const float *__restrict__ lse, int L, int K, int N,
                                                        const int32_t *__restrict__ root_token,
                                                        int32_t *__restrict__ parent, int32_t *__restrict__ tok,
                                                        float *__restrict__ score, int32_t *__restrict__ n_nodes) {
  const int b = blockIdx.x, lane = threadIdx.x;
  __shared__ float lp[DRAFT_LMAX * DRAFT_KMAX];
  __shared__ int lt[DRAFT_LMAX * DRAFT_KMAX];
  for (int e = lane; e < L * K; e += 64) {
    const int i = e / K;
    const float z = lse[(size_t)b * L + i], x = topk_logit[(size_t)b * L * K + e];
    const int t = topk_idx[(size_t)b * L * K + e];
    // log p = logit - LSE; no candidate where the entry or the row is empty
    lp[e] = (t >= 0 && x > -INFINITY && z > -INFINITY) ? x - z : -INFINITY;
    lt[e] = t;
  }
  __syncthreads();
  // node state (lane j = node j)
  int par = -1, dep = 0, nxt = 0, tk = root_token[b];
  float sc = 0.f;
  unsigned long long code = 0ull;
  int cnt = 1;
  for (int it = 1; it < N; ++it) {
    float cs = -INFINITY;
    unsigned long long cc = ~0ull;
    if (lane < cnt && dep < L && nxt < K) {
      const float l = lp[dep * K + nxt];
      if (l > -INFINITY) {
        cs = sc + l;
        cc = code | ((unsigned long long)(nxt + 1) << (60 - 4 * dep));
      }
    }
    // arg-best over the wave: higher score, then lower code (codes differ)
    float bs = cs;
    unsigned long long bc = cc;
    int bl = lane;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float os = __shfl_xor(bs, o);
      const unsigned long long oc = __shfl_xor(bc, o);
      const int ol = __shfl_xor(bl, o);
      const bool take = os > bs || (os == bs && oc < bc);
      bs = take ? os : bs;
      bc = take ? oc : bc;
      bl = take ? ol : bl;
    }
    if (!(bs > -INFINITY)) break;  // no candidate left (the same in every lane)
    const int wl = __builtin_amdgcn_readfirstlane(bl);
    const int wdep = __shfl(dep, wl), wnxt = __shfl(nxt, wl);
    if (lane == wl) ++nxt;
    if (lane == cnt) {
      par = wl;
      dep = wdep + 1;
      nxt = 0;
      tk = lt[wdep * K + wnxt];
      sc = bs;
      code = bc;
    }
    ++cnt;
  }
  if (lane < cnt) {
    parent[(size_t)b * N + lane] = par;
    tok[(size_t)b * N + lane] = tk;
    score[(size_t)b * N + lane] = sc;
  }
  if (lane == 0) n_nodes[b] = cnt;
}

static int draft_chunks(int B, int L, int V) {
  // about 1024 workgroups over the batch, chunks of at least 2048 entries
  int C = (1024 + B * L - 1) / (B * L);
  const int by_len = (V + 2047) / 2048;
  if (C > by_len) C = by_len;
  if (C > DRAFT_CMAX) C = DRAFT_CMAX;
  return C < 1 ? 1 : C;
}

}  // namespace ddt

using namespace ddt;

extern "C" size_t ddt_draft_topk_workspace(int32_t B, int32_t L, int32_t V, int32_t K) {
  if (B < 1 || L < 1 || V < 1 || K < 1 || K > DRAFT_KMAX) return 0;
  const size_t rows = (size_t)B * L * draft_chunks(B, L, V);
  return rows * K * sizeof(int2) + rows * sizeof(float2) + 256;
}

extern "C" int ddt_draft_topk(const void *logits, int32_t B, int32_t L, int32_t V, int32_t dtype, int32_t K,
                              int32_t *topk_idx, float *topk_logit, float *lse, void *workspace,
                              size_t ws_bytes, void *stream) {
  if (!logits || !topk_idx || !topk_logit || !lse || !workspace) return DDT_E_ARG;
  if (B < 1 || B > 65535 || L < 1 || L > 65535 || V < 1 || K < 1 || K > DRAFT_KMAX) return DDT_E_SHAPE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  if (ws_bytes < ddt_draft_topk_workspace(B, L, V, K)) return DDT_E_WS;
  const int C = draft_chunks(B, L, V);
  int chunk = (V + C - 1) / C;
  chunk = (chunk + 7) / 8 * 8;  // chunk starts stay 8-element aligned
  const size_t esz = dtype == DDT_BF16 ? 2 : 4;
  const int vec = ((uintptr_t)logits % 16 == 0) && ((size_t)V * esz % 16 == 0);
  DraftWs W;
  const size_t rows = (size_t)B * L * C;
  char *p = (char *)(((uintptr_t)workspace + 255) / 256 * 256);
  W.cand = (int2 *)p;
  W.ms = (float2 *)(p + rows * K * sizeof(int2));
  hipStream_t st = (hipStream_t)stream;
  dim3 grid(C, L, B);
#define DDT_DRAFT(KK)                                                                                 \
  do {                                                                                                \
    if (dtype == DDT_BF16)                                                                            \
      hipLaunchKernelGGL((draft_chunk_kernel<uint16_t, KK>), grid, dim3(256), 0, st,                  \
                         (const uint16_t *)logits, L, V, C, chunk, vec, W);                           \
    else                                                                                              \
      hipLaunchKernelGGL((draft_chunk_kernel<float, KK>), grid, dim3(256), 0, st, (const float *)logits, \
                         L, V, C, chunk, vec, W);                                                     \
    hipLaunchKernelGGL((draft_merge_kernel<KK>), dim3(L, B), dim3(64), 0, st, L, C, W, topk_idx,      \
                       topk_logit, lse);                                                              \
  } while (0)
  switch (K) {
    case 1: DDT_DRAFT(1); break;
    case 2: DDT_DRAFT(2); break;
    case 3: DDT_DRAFT(3); break;
    case 4: DDT_DRAFT(4); break;
    case 5: DDT_DRAFT(5); break;
    case 6: DDT_DRAFT(6); break;
    case 7: DDT_DRAFT(7); break;
    default: DDT_DRAFT(8); break;
  }
#undef DDT_DRAFT
  return launch_status();
}

extern "C" int ddt_tree_build(const int32_t *topk_idx, const float *topk_logit, const float *lse, int32_t B,
                              int32_t L, int32_t K, int32_t N, const int32_t *root_token, int32_t *parent,
                              int32_t *tok, float *score, int32_t *n_nodes, void *stream) {
  if (!topk_idx || !topk_logit || !lse || !root_token || !parent || !tok || !score || !n_nodes) return DDT_E_ARG;
  if (B < 1 || B > 65535 || L < 1 || L > DRAFT_LMAX || K < 1 || K > DRAFT_KMAX) return DDT_E_SHAPE;
  if (N < 1 || N > DDT_MAX_NODES) return DDT_E_SHAPE;
  hipLaunchKernelGGL(draft_tree_kernel, dim3(B), dim3(64), 0, (hipStream_t)stream, topk_idx, topk_logit, lse, L,
                     K, N, root_token, parent, tok, score, n_nodes);
  return launch_status();
}
