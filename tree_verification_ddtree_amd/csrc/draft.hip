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
//                      vocabulary): every thread keeps a sorted best-8 list
//                      and an online (max, sum of exponentials); each group
//                      of 8 read values that can improve the list is sorted
//                      and merged in (bitonic networks: no branches, no
//                      register indexing); lists and sums then meet in a
//                      butterfly over the wavefront and in LDS.
//  draft_merge_kernel  one wavefront per (sequence, position): the same
//                      butterfly over the chunks' lists and sums gives the
//                      top-K (a prefix of the best 8) and the log-sum-exp.
//  draft_tree_kernel   one wavefront per sequence, one lane per tree node:
//                      each selected node offers its best unselected child;
//                      a wave-wide arg-best picks the next node, N-1 times.
// Every merge is a fixed pattern of exchanges over a strict total order, so
// results do not depend on timing.
#include "common.h"

namespace ddt {

constexpr int DRAFT_KMAX = 8;   // lists are kept 8 long; K <= 8 reads a prefix
constexpr int DRAFT_LMAX = 16;  // rank codes hold 16 levels of 4 bits
constexpr int DRAFT_CMAX = 64;  // vocabulary chunks per position (one lane each in the merge)
constexpr int DRAFT_EMPTY = 0x7fffffff;

// (logit a, index ia) ranks before (b, ib): larger logit, then lower index.
// Empty entries are (-inf, DRAFT_EMPTY) and rank after every real one.
__device__ __forceinline__ bool cand_before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// compare-exchange: entry p ends up before entry q
__device__ __forceinline__ void cex(float &vp, int &ip, float &vq, int &iq) {
  const bool sw = cand_before(vq, iq, vp, ip);
  const float tv = vp;
  const int ti = ip;
  vp = sw ? vq : vp;
  ip = sw ? iq : ip;
  vq = sw ? tv : vq;
  iq = sw ? ti : iq;
}

// Sort 8 entries, best first (bitonic network, 24 compare-exchanges).
__device__ __forceinline__ void sort8(float (&v)[8], int (&ix)[8]) {
#pragma unroll
  for (int k = 2; k <= 8; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int l = i ^ j;
        if (l > i) {
          if ((i & k) == 0)
            cex(v[i], ix[i], v[l], ix[l]);
          else
            cex(v[l], ix[l], v[i], ix[i]);
        }
      }
}

// a := the best 8 of a and b, best first (both sorted best first): the
// better of a[k] and b[7-k] form a bitonic sequence holding the best 8,
// which three rounds of compare-exchanges sort.
__device__ __forceinline__ void merge8(float (&a)[8], int (&ia)[8], const float (&b)[8], const int (&ib)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool tb = cand_before(b[7 - k], ib[7 - k], a[k], ia[k]);
    a[k] = tb ? b[7 - k] : a[k];
    ia[k] = tb ? ib[7 - k] : ia[k];
  }
#pragma unroll
  for (int j = 4; j > 0; j >>= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & j) == 0) cex(a[i], ia[i], a[i + j], ia[i + j]);
}

// Partner value at butterfly stage S (pairs are symmetric): DPP inside a
// row of 16 lanes (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror), then lanes 16 and 32 apart.
template <int S>
__device__ __forceinline__ int xpart(int v) {
  if constexpr (S == 0) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  else if constexpr (S == 1) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  else if constexpr (S == 2) return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
  else if constexpr (S == 3) return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
  else if constexpr (S == 4) return __shfl_xor(v, 16);
  else return __shfl_xor(v, 32);
}
template <int S>
__device__ __forceinline__ float xpartf(float v) {
  return __int_as_float(xpart<S>(__float_as_int(v)));
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

// One butterfly stage over a lane's list and (max, sum): every lane ends
// with the pair's best 8 and combined sum.
template <int S>
__device__ __forceinline__ void stage(float (&v)[8], int (&ix)[8], float &m, float &s) {
  float pv[8];
  int pi[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    pv[k] = xpartf<S>(v[k]);
    pi[k] = xpart<S>(ix[k]);
  }
  merge8(v, ix, pv, pi);
  ms_combine(m, s, xpartf<S>(m), xpartf<S>(s));
}
template <int S>
__device__ __forceinline__ void stage_ms(float &m, float &s) {
  ms_combine(m, s, xpartf<S>(m), xpartf<S>(s));
}
__device__ __forceinline__ void wave_merge(float (&v)[8], int (&ix)[8], float &m, float &s) {
  stage<0>(v, ix, m, s);
  stage<1>(v, ix, m, s);
  stage<2>(v, ix, m, s);
  stage<3>(v, ix, m, s);
  stage<4>(v, ix, m, s);
  stage<5>(v, ix, m, s);
}

// 8 read values at vocabulary indices e..e+7 -> a sorted list; NaN and -inf
// become empty entries
__device__ __forceinline__ void take8(const float (&f)[8], int e, float (&v)[8], int (&ix)[8]) {
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const bool ok = f[x] > -INFINITY;
    v[x] = ok ? f[x] : -INFINITY;
    ix[x] = ok ? e + x : DRAFT_EMPTY;
  }
  sort8(v, ix);
}

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// (value, index) as one unsigned key: larger key = larger value, then
// lower index (NaN never reaches a key; -0 counts as +0, as in compares)
__device__ __forceinline__ unsigned long long okey(float v, int i) {
  const unsigned u = __float_as_uint(v + 0.0f);
  const unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned)(0x7fffffff - i);
}
__device__ __forceinline__ float okey_value(unsigned long long k) {
  const unsigned o = (unsigned)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

struct DraftWs {
  int2 *cand;  // [B][L][C][8] (logit bits, index)
  float2 *ms;  // [B][L][C] (max, sum)
};

constexpr int DRAFT_GMAX = 12;   // groups of 8 elements a thread holds (chunk <= 256*8*12)
constexpr int DRAFT_BUF = 512;   // LDS slots for the elements that pass the bar

// 8 raw elements of a group, held as plain vectors so they stay in
// registers: bf16 as 4 words (one 16-byte read), fp32 as 8 floats
typedef unsigned int draft_u4 __attribute__((ext_vector_type(4)));
typedef float draft_f8 __attribute__((ext_vector_type(8)));
template <typename T>
struct RawOf;
template <>
struct RawOf<uint16_t> {
  typedef draft_u4 type;
};
template <>
struct RawOf<float> {
  typedef draft_f8 type;
};

__device__ __forceinline__ draft_u4 raw_empty(const uint16_t *) {
  return draft_u4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};  // -inf pairs
}
__device__ __forceinline__ draft_f8 raw_empty(const float *) {
  return draft_f8{-INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY};
}
__device__ __forceinline__ draft_u4 raw_load(const uint16_t *p) { return *reinterpret_cast<const draft_u4 *>(p); }
__device__ __forceinline__ draft_f8 raw_load(const float *p) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
  return draft_f8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}
// element by element, -inf past e1
__device__ __forceinline__ draft_u4 raw_load_each(const uint16_t *row, int e, int e1) {
  uint32_t h[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) h[x] = e + x < e1 ? (uint32_t)row[e + x] : 0xff80u;
  return draft_u4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}
__device__ __forceinline__ draft_f8 raw_load_each(const float *row, int e, int e1) {
  draft_f8 f;
#pragma unroll
  for (int x = 0; x < 8; ++x) f[x] = e + x < e1 ? row[e + x] : -INFINITY;
  return f;
}
__device__ __forceinline__ float raw_at(draft_u4 u, int x) {
  const uint32_t w = u[x >> 1];
  return __uint_as_float((x & 1) ? (w & 0xffff0000u) : (w << 16));
}
__device__ __forceinline__ float raw_at(draft_f8 f, int x) { return f[x]; }

// One workgroup per (sequence, position, chunk).  Pass 1 reads the chunk
// once into registers (G groups of 8 per thread), folds every element into
// the thread's online (max, sum of exponentials) and keeps each group's
// largest value.  A bar no larger than the chunk's 8th best value comes
// from ranking the thread bests (below); pass 2 puts the elements at or above
// it (groups whose largest value is below it are skipped) into an LDS
// buffer, and one wavefront places them by rank.  A buffer that overflows
// (vast runs of values equal to the bar) sends every element through
// per-thread sorted lists instead.
template <typename T, int G>
__global__ __launch_bounds__(256) void draft_chunk_kernel(const T *__restrict__ logits, int L, int V, int C,
                                                          int chunk, int vec, DraftWs Ws) {
  const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const T *row = logits + ((size_t)b * L + i) * V;
  const int e0 = c * chunk, e1 = min(V, e0 + chunk);
  const int ng = (e1 - e0 + 7) / 8;
  __shared__ __align__(16) unsigned long long tkey[256], top8[32];
  __shared__ float bv[DRAFT_BUF], lv[4][8], sm[4], ss[4], barl;
  __shared__ int bi[DRAFT_BUF], li[4][8], nbuf;
  if (tid == 0) nbuf = 0;
  // ---- pass 1: read, log-sum-exp terms, thread best
  typename RawOf<T>::type r[G];
  const int nfull = (e1 - e0) / 8;  // groups wholly inside the chunk
  if (vec && nfull > 0) {
    // every read issued before any is used: the address is clamped into the
    // chunk and groups past the last whole one are replaced afterwards
#pragma unroll
    for (int g = 0; g < G; ++g) r[g] = raw_load(row + e0 + 8 * min(tid + 256 * g, nfull - 1));
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = tid + 256 * g;
      if (j >= nfull) r[g] = j < ng ? raw_load_each(row, e0 + 8 * j, e1) : raw_empty(row);
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = tid + 256 * g;
      r[g] = j < ng ? raw_load_each(row, e0 + 8 * j, e1) : raw_empty(row);
    }
  }
  float m = -INFINITY, s = 0.f, tv = -INFINITY, gmx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    gmx[g] = -INFINITY;
    if (tid + 256 * g < ng) {
      float f[8], gm = -INFINITY;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        f[x] = raw_at(r[g], x);
        gm = fmaxf(gm, f[x]);  // fmaxf drops NaN
      }
      if (gm > m) {
        s = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - gm) * 1.4426950408889634f);
        m = gm;
      }
      if (gm > -INFINITY) {
        const float mc = m * 1.4426950408889634f;
#pragma unroll
        for (int x = 0; x < 8; ++x)
          s += f[x] > -INFINITY ? __builtin_amdgcn_exp2f(fmaf(f[x], 1.4426950408889634f, -mc)) : 0.f;
      }
      gmx[g] = gm;
      tv = fmaxf(tv, gm);
    }
  }
  // ---- the bar: the 8th largest of the workgroup's 256 thread bests: 8
  // distinct elements are at least that large, so the chunk's 8 best are
  // all at or above it.  Keys order (value, then lower thread) as unsigned
  // 64-bit integers.  Every wavefront ranks its 64 keys (one compare each,
  // broadcast LDS reads) and keeps its best 8; the workgroup's 8th best is
  // the 8th of those 32.
#pragma unroll
  for (int o = 0; o < 6; ++o) {
    if (o == 0) stage_ms<0>(m, s);
    if (o == 1) stage_ms<1>(m, s);
    if (o == 2) stage_ms<2>(m, s);
    if (o == 3) stage_ms<3>(m, s);
    if (o == 4) stage_ms<4>(m, s);
    if (o == 5) stage_ms<5>(m, s);
  }
  if (lane == 0) {
    sm[w] = m;
    ss[w] = s;
  }
  const unsigned long long mykey = okey(tv, tid);
  tkey[tid] = mykey;  // a wave reads back only its own lanes' keys (LDS keeps one wave's order)
  {
    int rk = 0;
#pragma unroll 8
    for (int j = 0; j < 64; j += 2) {
      const ulonglong2 q = *reinterpret_cast<const ulonglong2 *>(&tkey[w * 64 + j]);
      rk += (q.x > mykey) + (q.y > mykey);
    }
    if (rk < 8) top8[w * 8 + rk] = mykey;
  }
  __syncthreads();
  if (w == 0 && lane < 32) {
    const unsigned long long k = top8[lane];
    int rk = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) rk += top8[j] > k;
    if (rk == 7) barl = okey_value(k);
  }
  __syncthreads();
  const float barv = barl;
  // ---- pass 2: elements at or above the bar
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (gmx[g] >= barv && gmx[g] > -INFINITY) {
      const int e = e0 + 8 * (tid + 256 * g);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float f = raw_at(r[g], x);
        if (f > -INFINITY && f >= barv) {
          const int at = atomicAdd(&nbuf, 1);
          if (at < DRAFT_BUF) {
            bv[at] = f;
            bi[at] = e + x;
          }
        }
      }
    }
  }
  __syncthreads();
  const int n = nbuf;
  float v[8];
  int ix[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v[k] = -INFINITY;
    ix[k] = DRAFT_EMPTY;
  }
  if (n <= DRAFT_BUF) {
    // every candidate placed by its rank among the candidates (read from
    // LDS; the entries are distinct, so the ranks are too): slot k of the
    // chunk's list is the candidate of rank k
    if (w == 0) {
      for (int c0 = 0; c0 < n; c0 += 64) {
        const int me = c0 + lane;
        const float cv = me < n ? bv[me] : -INFINITY;
        const int ci = me < n ? bi[me] : DRAFT_EMPTY;
        const unsigned long long ck = okey(cv, ci);
        int rk = 0;
#pragma unroll 4
        for (int j = 0; j < n; ++j) rk += okey(bv[j], bi[j]) > ck;
        if (me < n && rk < 8) {
          lv[0][rk] = cv;
          li[0][rk] = ci;
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[k] = k < n ? lv[0][k] : -INFINITY;
        ix[k] = k < n ? li[0][k] : DRAFT_EMPTY;
      }
    }
  } else {
    // rare: every element through per-thread sorted lists
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (tid + 256 * g < ng) {
        const int e = e0 + 8 * (tid + 256 * g);
        float f[8], gv[8];
        int gi[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) f[x] = raw_at(r[g], x);
        take8(f, e, gv, gi);
        merge8(v, ix, gv, gi);
      }
    }
    float dm = -INFINITY, ds = 0.f;
    wave_merge(v, ix, dm, ds);
    __syncthreads();  // the bars are no longer read
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        lv[w][k] = v[k];
        li[w][k] = ix[k];
      }
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        float qv[8];
        int qi[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          qv[k] = lv[q][k];
          qi[k] = li[q][k];
        }
        merge8(v, ix, qv, qi);
      }
    }
  }
  if (tid == 0) {
    for (int q = 1; q < 4; ++q) ms_combine(m, s, sm[q], ss[q]);
    const size_t rr = ((size_t)b * L + i) * C + c;
#pragma unroll
    for (int k = 0; k < 8; ++k) Ws.cand[rr * 8 + k] = make_int2(__float_as_int(v[k]), ix[k]);
    Ws.ms[rr] = make_float2(m, s);
  }
}

__global__ __launch_bounds__(64) void draft_merge_kernel(int L, int C, int K, DraftWs Ws,
                                                         int32_t *__restrict__ topk_idx,
                                                         float *__restrict__ topk_logit, float *__restrict__ lse) {
  const int i = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  float v[8];
  int ix[8];
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v[k] = -INFINITY;
    ix[k] = DRAFT_EMPTY;
  }
  const size_t r0 = ((size_t)b * L + i) * C;
  if (lane < C) {  // one chunk a lane
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int2 e = Ws.cand[(r0 + lane) * 8 + k];
      v[k] = __int_as_float(e.x);
      ix[k] = e.y;
    }
    const float2 p = Ws.ms[r0 + lane];
    m = p.x;
    s = p.y;
  }
  wave_merge(v, ix, m, s);
  if (lane < K) {
    // lane k writes entry k (unrolled select from the list every lane holds)
    float vk = v[0];
    int ik = ix[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      vk = lane == k ? v[k] : vk;
      ik = lane == k ? ix[k] : ik;
    }
    const bool ok = ik != DRAFT_EMPTY;
    topk_idx[((size_t)b * L + i) * K + lane] = ok ? ik : -1;
    topk_logit[((size_t)b * L + i) * K + lane] = ok ? vk : -INFINITY;
  }
  if (lane == 0) lse[(size_t)b * L + i] = m == -INFINITY ? -INFINITY : m + __logf(s);
}

// One wavefront per sequence; lane j is tree node j once selected and then
// holds its unselected candidate children (the top-K of its depth's
// position: log p and token) as a register queue, best first, so its
// candidate is always queue entry 0.  A candidate is ranked by score, then
// by its code: the candidate ranks along the root path, 4 bits per level
// from the top (rank + 1, 0 past the node's depth), so that comparing codes
// as integers is the lexicographic order with a prefix first.  Codes of
// different candidates differ.  The best score comes from a DPP max into
// lane 63 (row shifts, then row broadcasts) over the scores as ordered
// integers; only an exact score tie runs the code comparison.  No score is
// -0 (the root's is +0 and each score adds a log p to its parent's), so
// the integer order is the float order with equal floats equal.
typedef float draft_q8f __attribute__((ext_vector_type(8)));
typedef int draft_q8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int score_key(float f) {
  const int u = __float_as_int(f);
  return u ^ ((u >> 31) & 0x7fffffff);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_imax(int a) {
  // lanes without a source (or in rows outside ROWS) see INT_MIN
  const int o = __builtin_amdgcn_update_dpp((int)0x80000000, a, CTRL, ROWS, 0xF, false);
  return o > a ? o : a;
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_umin64(unsigned long long a) {
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(-1, (int)(unsigned)a, CTRL, ROWS, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(-1, (int)(unsigned)(a >> 32), CTRL, ROWS, 0xF, false);
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  return o < a ? o : a;
}
__device__ __forceinline__ int wave_imax_to63(int a) {
  a = dpp_imax<0x111, 0xF>(a);  // row_shr:1
  a = dpp_imax<0x112, 0xF>(a);  // row_shr:2
  a = dpp_imax<0x114, 0xF>(a);  // row_shr:4
  a = dpp_imax<0x118, 0xF>(a);  // row_shr:8: lane 15 of each row holds the row's maximum
  a = dpp_imax<0x142, 0xA>(a);  // row_bcast:15 into rows 1 and 3
  return dpp_imax<0x143, 0xC>(a);  // row_bcast:31 into rows 2 and 3: lane 63 holds the maximum
}
__device__ __forceinline__ unsigned long long wave_umin64_to63(unsigned long long a) {
  a = dpp_umin64<0x111, 0xF>(a);
  a = dpp_umin64<0x112, 0xF>(a);
  a = dpp_umin64<0x114, 0xF>(a);
  a = dpp_umin64<0x118, 0xF>(a);
  a = dpp_umin64<0x142, 0xA>(a);
  return dpp_umin64<0x143, 0xC>(a);
}
__device__ __forceinline__ unsigned long long readlane64(unsigned long long v, int l) {
  return ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
         (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, l);
}

__global__ __launch_bounds__(64) void draft_tree_kernel(const int32_t *__restrict__ topk_idx,
                                                        const float *__restrict__ topk_logit,
                                                        const float *__restrict__ lse, int L, int K, int N,
                                                        const int32_t *__restrict__ root_token,
                                                        int32_t *__restrict__ parent, int32_t *__restrict__ tok,
                                                        float *__restrict__ score, int32_t *__restrict__ n_nodes) {
  const int b = blockIdx.x, lane = threadIdx.x;
  // row i = position i's candidates as log p and token; row L is empty (a
  // node at depth L has no children)
  __shared__ draft_q8f lp[DRAFT_LMAX + 1];
  __shared__ draft_q8i lt[DRAFT_LMAX + 1];
  for (int e = lane; e < (L + 1) * DRAFT_KMAX; e += 64) {
    const int i = e / DRAFT_KMAX, k = e % DRAFT_KMAX;
    float x = -INFINITY;
    int t = -1;
    if (i < L && k < K) {
      const float z = lse[(size_t)b * L + i];
      x = topk_logit[((size_t)b * L + i) * K + k];
      t = topk_idx[((size_t)b * L + i) * K + k];
      // log p = logit - LSE; no candidate where the entry or the row is empty
      x = (t >= 0 && x > -INFINITY && z > -INFINITY) ? x - z : -INFINITY;
    }
    ((float *)lp)[e] = x;
    ((int *)lt)[e] = t;
  }
  __syncthreads();
  int par = -1, dep = 0, nxt = 0, tk = root_token[b];
  float sc = 0.f;
  unsigned long long code = 0ull;
  // the root's queue (row 0); lanes not yet nodes hold none
  draft_q8f rl = lp[0];
  draft_q8i rt = lt[0];
  if (lane != 0) rl = (draft_q8f)(-INFINITY);
  int cnt = 1;
  for (int it = 1; it < N; ++it) {
    const float cs = sc + rl.s0;  // -inf when the lane has no candidate
    const int ck = score_key(cs);
    const int bk = __builtin_amdgcn_readlane(wave_imax_to63(ck), 63);
    if (bk == score_key(-INFINITY)) break;  // no candidate left (the same in every lane)
    const unsigned long long tied = __ballot(ck == bk);
    int wl = __ffsll((long long)tied) - 1;
    if (__popcll(tied) > 1) {  // exact score tie: the smallest code wins
      const unsigned sh = (unsigned)(60 - 4 * dep) & 63u;
      const unsigned long long cc = code | ((unsigned long long)(nxt + 1) << sh);
      const unsigned long long bc = readlane64(wave_umin64_to63(ck == bk ? cc : ~0ull), 63);
      wl = __ffsll((long long)__ballot(ck == bk && cc == bc)) - 1;
    }
    const int wdep = __builtin_amdgcn_readlane(dep, wl), wnxt = __builtin_amdgcn_readlane(nxt, wl);
    const int wtk = __builtin_amdgcn_readlane(rt.s0, wl);
    const float bs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), wl));
    const unsigned long long wcode = readlane64(code, wl) | ((unsigned long long)(wnxt + 1) << (60 - 4 * wdep));
    // the winner moves on to its next child
    const bool w = lane == wl;
    const draft_q8f nl = __builtin_shufflevector(rl, (draft_q8f)(-INFINITY), 1, 2, 3, 4, 5, 6, 7, 8);
    const draft_q8i nt = __builtin_shufflevector(rt, rt, 1, 2, 3, 4, 5, 6, 7, 7);
    rl = w ? nl : rl;
    rt = w ? nt : rt;
    nxt += w ? 1 : 0;
    if (lane == cnt) {  // the new node
      par = wl;
      dep = wdep + 1;
      nxt = 0;
      tk = wtk;
      sc = bs;
      code = wcode;
      rl = lp[dep];
      rt = lt[dep];
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
  // about one workgroup per compute unit over the batch, chunks of at least
  // 2048 entries, and no more than DRAFT_GMAX groups of 8 per thread
  int C = (256 + B * L - 1) / (B * L);
  const int by_len = (V + 2047) / 2048;
  if (C > by_len) C = by_len;
  const int need = (V + 256 * 8 * DRAFT_GMAX - 1) / (256 * 8 * DRAFT_GMAX);
  if (C < need) C = need;
  if (C > DRAFT_CMAX) C = DRAFT_CMAX;
  return C < 1 ? 1 : C;
}

}  // namespace ddt

using namespace ddt;

extern "C" size_t ddt_draft_topk_workspace(int32_t B, int32_t L, int32_t V, int32_t K) {
  if (B < 1 || L < 1 || V < 1 || K < 1 || K > DRAFT_KMAX) return 0;
  const size_t rows = (size_t)B * L * draft_chunks(B, L, V);
  return rows * 8 * sizeof(int2) + rows * sizeof(float2) + 256;
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
  if (chunk > 256 * 8 * DRAFT_GMAX) return DDT_E_SHAPE;  // V above 64 chunks of the register budget
  const size_t esz = dtype == DDT_BF16 ? 2 : 4;
  const int vec = ((uintptr_t)logits % 16 == 0) && ((size_t)V * esz % 16 == 0);
  DraftWs W;
  const size_t rows = (size_t)B * L * C;
  char *p = (char *)(((uintptr_t)workspace + 255) / 256 * 256);
  W.cand = (int2 *)p;
  W.ms = (float2 *)(p + rows * 8 * sizeof(int2));
  hipStream_t st = (hipStream_t)stream;
  dim3 grid(C, L, B);
  const int gpt = ((chunk + 7) / 8 + 255) / 256;  // groups of 8 per thread
#define DDT_CHUNK(GG)                                                                                  \
  do {                                                                                                 \
    if (dtype == DDT_BF16)                                                                             \
      hipLaunchKernelGGL((draft_chunk_kernel<uint16_t, GG>), grid, dim3(256), 0, st,                   \
                         (const uint16_t *)logits, L, V, C, chunk, vec, W);                            \
    else                                                                                               \
      hipLaunchKernelGGL((draft_chunk_kernel<float, GG>), grid, dim3(256), 0, st, (const float *)logits, \
                         L, V, C, chunk, vec, W);                                                      \
  } while (0)
  if (gpt <= 1) DDT_CHUNK(1);
  else if (gpt <= 2) DDT_CHUNK(2);
  else if (gpt <= 4) DDT_CHUNK(4);
  else if (gpt <= 8) DDT_CHUNK(8);
  else DDT_CHUNK(DRAFT_GMAX);
#undef DDT_CHUNK
  hipLaunchKernelGGL(draft_merge_kernel, dim3(L, B), dim3(64), 0, st, L, C, K, W, topk_idx, topk_logit, lse);
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
