// Stochastic tree acceptance: each node's verify sample (temperature, top-k,
// top-p) replaces its argmax in the greedy walk.
//
// Requests without a temperature are sampled with the model card's
// settings, temperature 1.0, top_p 0.95, top_k 20 (codehub lucebox-hub@main,
// "Making requests").  The pages give no acceptance rule for a tree; the
// one taken here: every node reached draws one sample from its own filtered
// target distribution, and the walk moves to the child that carries it (for
// deterministic candidates such as DDTree's this is what recursive
// rejection sampling reduces to).  Every node's sample is independent of
// the walk, so all of them are drawn in parallel and the greedy walk then
// follows them.
//
// Per node the distribution needs only the top_k logits (k <= 32), in
// descending order with ties to the lower index:
//  - samp_chunk_kernel: a 256-thread workgroup holds one chunk of a row in
//    registers as order-preserving 32-bit keys.  A lower bound on the
//    chunk's top k (the bar) comes from the thread maxima: each wavefront
//    takes the ceil(k/4)-th largest of its 64 maxima by DPP maximum rounds,
//    and the smallest of the four wavefronts' values is the bar, so at least
//    k elements reach it.  On ordinary rows only a few elements do; they are
//    compacted into LDS and ranked by counting (value, then lower index
//    first).  Near-flat rows, where more than SAMP_FAST elements reach the
//    bar, take the exact path instead: three histogram passes over the key
//    bits (11, 11, 10 bits) find the k-th largest key, ties at it go to the
//    lowest indices (two passes over the index bits).  Either way the k
//    entries are written sorted;
//  - samp_merge_kernel: one workgroup per row ranks the chunks' entries,
//    then one wavefront forms p_i = 2^((v_i - v_0) log2(e) / T), the top-p
//    cut (smallest prefix with c_i >= top_p * total) and the inverse-CDF
//    draw (first c_i > u * R) with ballots, and hands the sample to the walk
//    as a chunk key.
#include "common.h"

namespace ddt {

constexpr int SAMP_KMAX = 32;    // largest top_k
constexpr int SAMP_CMAX = 16;    // chunks per row
constexpr int SAMP_GMAX = 12;    // 8-element groups per thread
constexpr int SAMP_NCHUNK = 16;  // the walk's chunk-key stride per row (walk.hip)
constexpr int SAMP_FAST = 256;   // candidates above the bar ranked directly

// order-preserving key of a logit; 0 for NaN, -inf (never kept) and padding
__device__ __forceinline__ unsigned samp_key(float f) {
  if (!(f > -INFINITY)) return 0u;
  const unsigned u = __float_as_uint(f + 0.0f);  // -0 counts as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float samp_val(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wavefront maximum of unsigned keys, in every lane: DPP row shifts leave
// each row's maximum in its lane 15, row broadcasts carry it into lane 63
// (0 is the identity: lanes without a source keep theirs).
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned samp_dpp_umax(unsigned a) {
  const unsigned o = (unsigned)__builtin_amdgcn_update_dpp(0, (int)a, CTRL, ROWS, 0xF, false);
  return o > a ? o : a;
}
__device__ __forceinline__ unsigned samp_wave_umax(unsigned a) {
  a = samp_dpp_umax<0x111, 0xF>(a);  // row_shr:1
  a = samp_dpp_umax<0x112, 0xF>(a);  // row_shr:2
  a = samp_dpp_umax<0x114, 0xF>(a);  // row_shr:4
  a = samp_dpp_umax<0x118, 0xF>(a);  // row_shr:8
  a = samp_dpp_umax<0x142, 0xA>(a);  // row_bcast:15 into rows 1 and 3
  a = samp_dpp_umax<0x143, 0xC>(a);  // row_bcast:31 into rows 2 and 3
  return (unsigned)__builtin_amdgcn_readlane((int)a, 63);
}

// Block-wide search in hist[0..nb) (LDS): the bin where, counting from the
// top bin down (or from bin 0 up when !top), the running count reaches
// `need`.  Publishes the bin and the count strictly before it through
// sh[0], sh[1]; sh[2] = total count.  Every thread of the block calls it;
// thread t owns bins t*per .. t*per+per-1 in visiting order, and the
// prefix over threads is a wavefront scan plus the totals of the earlier
// wavefronts.
__device__ void find_bin(const unsigned *hist, int nb, unsigned need, bool top, unsigned *wsum,
                         unsigned *sh) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, per = nb / 256;
  auto bin_of = [&](int i) { return top ? nb - 1 - i : i; };  // i-th bin in visiting order
  unsigned s = 0;
  for (int i = 0; i < per; ++i) s += hist[bin_of(t * per + i)];
  unsigned incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned up = __shfl_up(incl, o);
    if (lane >= o) incl += up;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  for (int q = 0; q < w; ++q) incl += wsum[q];
  const unsigned before = incl - s;
  if (t == 255) sh[2] = incl;
  if (before < need && need <= before + s) {
    unsigned acc = before;
    for (int i = 0; i < per; ++i) {
      const unsigned h = hist[bin_of(t * per + i)];
      if (acc + h >= need) {
        sh[0] = (unsigned)bin_of(t * per + i);
        sh[1] = acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

// The `need`-th largest (with multiplicity) of the keys >= floor (> 0) held
// by the block, E per thread: three histogram passes over 11, 11 and 10 key
// bits.  Returns the key; `need` becomes the number of elements equal to it
// that belong to the selection (the rest of the selection is > the key).
// all = true (and nothing else set) if fewer than `need` keys qualify.
template <int E>
__device__ unsigned radix_kth(const unsigned (&key)[E], unsigned floor, unsigned &need, bool &all,
                              unsigned *hist, unsigned *wsum, unsigned *sh) {
  const int tid = threadIdx.x;
  unsigned prefix = 0u, pmask = 0u;
  all = false;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int nb = pass < 2 ? 2048 : 1024, sft = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    for (int i = tid; i < nb; i += 256) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < E; ++x)
      if (key[x] >= floor && (key[x] & pmask) == prefix) atomicAdd(&hist[(key[x] >> sft) & (nb - 1)], 1u);
    __syncthreads();
    find_bin(hist, nb, need, true, wsum, sh);
    if (pass == 0 && sh[2] < need) {  // sh[2]: the qualifying keys
      all = true;
      __syncthreads();
      return 0u;
    }
    need -= sh[1];
    prefix |= sh[0] << sft;
    pmask |= (unsigned)(nb - 1) << sft;
    __syncthreads();  // sh is rewritten by the next search
  }
  return prefix;
}

template <typename T, int G>
__global__ __launch_bounds__(256) void samp_chunk_kernel(const T *__restrict__ logits, int V, int chunk, int K,
                                                         float2 *__restrict__ cand) {
  constexpr int E = 8 * G;
  __shared__ __align__(16) unsigned hist[2048];
  __shared__ unsigned wsum[4];
  __shared__ unsigned sh[4];
  __shared__ unsigned ckey[SAMP_KMAX];
  __shared__ int cidx[SAMP_KMAX];
  // compacted candidates as (key << 32 | ~index) (+ one dummy slot per thread)
  __shared__ unsigned long long fk[SAMP_FAST + 256];
  const int ck = blockIdx.x, row = blockIdx.y, C = gridDim.x, tid = threadIdx.x;
  const int lo = ck * chunk, hi = min(V, lo + chunk);
  const T *p = logits + (size_t)row * V;
  // element (j, e) of this thread: chunk-local index 8 (tid + 256 j) + e
  unsigned key[E];
  if (V % 8 == 0) {
    constexpr int PW = sizeof(T) == 2 ? 1 : 2;  // 16-byte pieces per 8 elements
    uint4 raw[G][PW];
#pragma unroll
    for (int j = 0; j < G; ++j) {  // unconditional loads at clamped addresses, all issued first
      const int i0 = min(lo + 8 * (tid + 256 * j), max(hi - 8, lo));
#pragma unroll
      for (int q = 0; q < PW; ++q) raw[j][q] = *reinterpret_cast<const uint4 *>(p + i0 + 8 / PW * q);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int i0 = lo + 8 * (tid + 256 * j);
      float f[8];
      if constexpr (sizeof(T) == 2) {
        const unsigned w[4] = {raw[j][0].x, raw[j][0].y, raw[j][0].z, raw[j][0].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[2 * q] = __uint_as_float(w[q] << 16);
          f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          f[4 * q] = __uint_as_float(raw[j][q].x);
          f[4 * q + 1] = __uint_as_float(raw[j][q].y);
          f[4 * q + 2] = __uint_as_float(raw[j][q].z);
          f[4 * q + 3] = __uint_as_float(raw[j][q].w);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) key[8 * j + e] = (i0 + e < hi) ? samp_key(f[e]) : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = lo + 8 * (tid + 256 * j) + e;
        key[8 * j + e] = i < hi ? samp_key(load1(p + min(i, V - 1))) : 0u;
      }
  }
  // ---- a lower bound first.  Each wavefront takes the m-th largest of its
  // 64 thread maxima, m = ceil(K / 4), by m rounds of a wavefront maximum
  // that retires one holder each; the smallest of the four is the bar.  At
  // least m elements of every wavefront are >= it, so at least K elements of
  // the chunk are, and with them its whole top K.  It costs one workgroup
  // barrier, and on ordinary rows leaves only a few elements above it.
  const int lane = tid & 63, w = tid >> 6;
  unsigned tm = 0u;
#pragma unroll
  for (int x = 0; x < E; ++x) tm = max(tm, key[x]);
  unsigned wk = 0u;
  for (int r = 0; r < (K + 3) / 4; ++r) {
    const unsigned mx = samp_wave_umax(tm);
    wk = mx;
    const unsigned long long holders = __ballot(tm == mx);
    if (lane == __ffsll((long long)holders) - 1) tm = 0u;  // retire one holder
  }
  if (lane == 0) wsum[w] = wk;
  __syncthreads();
  unsigned bar = min(min(wsum[0], wsum[1]), min(wsum[2], wsum[3]));
  // 0: some wavefront has fewer than m thread maxima above padding, NaN and
  // -inf, so the bound is void and every finite logit qualifies
  if (bar == 0u) bar = 1u;
  unsigned need;
  bool all;

  // ---- ordinary rows leave only a few elements >= bar: they are compacted
  // into LDS (branch-free stores; elements below the bar go to a
  // per-thread dummy slot) and their ranks counted directly
  float2 *dst = cand + ((size_t)row * C + ck) * K;
  {
    int c = 0;
#pragma unroll
    for (int x = 0; x < E; ++x) c += key[x] >= bar ? 1 : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o);
      if (lane >= o) incl += up;
    }
    __syncthreads();  // wsum was last read for the bar
    if (lane == 63) wsum[w] = (unsigned)incl;
    __syncthreads();
    int slot = incl - c, total = 0;
    for (int q = 0; q < 4; ++q) {
      if (q < w) slot += (int)wsum[q];
      total += (int)wsum[q];
    }
    if (total <= SAMP_FAST) {  // the same in every thread
      // a group of 8 is visited only if one of its elements qualifies
#pragma unroll
      for (int j = 0; j < G; ++j) {
        bool any = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) any |= key[8 * j + e] >= bar;
        if (any) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool q = key[8 * j + e] >= bar;
            const int d = q ? slot : SAMP_FAST + tid;
            fk[d] = ((unsigned long long)key[8 * j + e] << 32) | (0xffffffffu - (unsigned)(lo + 8 * (tid + 256 * j) + e));
            slot += q ? 1 : 0;
          }
        }
      }
      __syncthreads();
      if (tid < total) {
        const unsigned long long mine = fk[tid];
        int rank = 0;
#pragma unroll 4
        for (int j = 0; j < total; ++j) rank += fk[j] > mine;
        if (rank < K)
          dst[rank] = make_float2(samp_val((unsigned)(mine >> 32)), __int_as_float((int)(0xffffffffu - (unsigned)mine)));
      }
      if (tid >= total && tid < K) dst[tid] = make_float2(-INFINITY, __int_as_float(-1));
      return;
    }
  }
  // ---- otherwise (near-flat rows): the chunk's K-th largest key among the
  // elements >= bar, exactly, by histogram passes over the register keys
  need = (unsigned)K;
  const unsigned prefix = radix_kth<E>(key, bar, need, all, hist, wsum, sh);
  // keys > prefix are all kept; `need` of the ties at prefix are kept, the
  // lowest chunk-local indices first (two passes over 8 + 7 index bits)
  unsigned ilim = 0xffffffffu;
  if (!all) {
    // ties at the threshold (the last pass counted them in its bin)
    const unsigned ties = hist[prefix & 1023u];
    if (ties > need) {
      unsigned ipre = 0u, imask = 0u, ineed = need;
      const int isft[2] = {7, 0}, inb[2] = {256, 128};
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        __syncthreads();
        for (int i = tid; i < 256; i += 256) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < E; ++x) {
          const unsigned li = 8u * (unsigned)(tid + 256 * (x >> 3)) + (unsigned)(x & 7);
          if (key[x] == prefix && (li & imask) == ipre) atomicAdd(&hist[(li >> isft[pass]) & (inb[pass] - 1)], 1u);
        }
        __syncthreads();
        find_bin(hist, 256, ineed, false, wsum, sh);
        ineed -= sh[1];
        ipre |= sh[0] << isft[pass];
        imask |= (unsigned)(inb[pass] - 1) << isft[pass];
      }
      ilim = ipre;  // ties with local index <= ilim are kept
    }
  }
  // ---- the kept elements: counted per thread, placed by a block-wide
  // prefix (a wavefront scan and the earlier wavefronts' totals), stored
  // without atomics
  auto keep = [&](int x) {
    const unsigned li = 8u * (unsigned)(tid + 256 * (x >> 3)) + (unsigned)(x & 7);
    return all ? key[x] != 0u : (key[x] > prefix || (key[x] == prefix && li <= ilim));
  };
  int c = 0;
#pragma unroll
  for (int x = 0; x < E; ++x) c += keep(x) ? 1 : 0;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o);
    if (lane >= o) incl += up;
  }
  __syncthreads();  // wsum was last read by the searches
  if (lane == 63) wsum[w] = (unsigned)incl;
  __syncthreads();
  int slot = incl - c, total = 0;
  for (int q = 0; q < 4; ++q) {
    if (q < w) slot += (int)wsum[q];
    total += (int)wsum[q];
  }
  if (c > 0) {
#pragma unroll
    for (int x = 0; x < E; ++x) {
      if (keep(x)) {
        if (slot < SAMP_KMAX) {
          ckey[slot] = key[x];
          cidx[slot] = lo + (int)(8u * (unsigned)(tid + 256 * (x >> 3)) + (unsigned)(x & 7));
        }
        ++slot;
      }
    }
  }
  __syncthreads();
  // sort the kept entries by (value desc, index asc) and write K of them
  const int n = min(total, K);
  if (tid < K) {
    if (tid < n) {
      const unsigned long long mine = ((unsigned long long)ckey[tid] << 32) | (0xffffffffu - (unsigned)cidx[tid]);
      int rank = 0;
      for (int j = 0; j < n; ++j) {
        const unsigned long long o = ((unsigned long long)ckey[j] << 32) | (0xffffffffu - (unsigned)cidx[j]);
        rank += o > mine;
      }
      dst[rank] = make_float2(samp_val(ckey[tid]), __int_as_float(cidx[tid]));
    } else {
      dst[tid] = make_float2(-INFINITY, __int_as_float(-1));
    }
  }
}

__global__ __launch_bounds__(256) void samp_merge_kernel(const float2 *__restrict__ cand, int C, int K,
                                                         const float *__restrict__ uniforms, float tscale,
                                                         float top_p, unsigned long long *__restrict__ part) {
  __shared__ __align__(16) unsigned long long okey[SAMP_CMAX * SAMP_KMAX];
  __shared__ float tv[SAMP_KMAX];
  __shared__ int ti[SAMP_KMAX];
  const int row = blockIdx.x, tid = threadIdx.x, M = C * K;
  const float2 *src = cand + (size_t)row * M;
  for (int i = tid; i < M; i += 256) {
    const float2 c = src[i];
    const int idx = __float_as_int(c.y);
    okey[i] = idx >= 0 ? ((unsigned long long)samp_key(c.x) << 32) | (0xffffffffu - (unsigned)idx) : 0ull;
  }
  __syncthreads();
  for (int i = tid; i < M; i += 256) {
    const unsigned long long mine = okey[i];
    if (mine == 0ull) continue;
    int rank = 0;
    const ulonglong2 *o2 = reinterpret_cast<const ulonglong2 *>(okey);
    for (int j = 0; j < M / 2; ++j) {  // pairs, then the odd one out
      const ulonglong2 v = o2[j];
      rank += (v.x > mine ? 1 : 0) + (v.y > mine ? 1 : 0);
    }
    if (M & 1) rank += okey[M - 1] > mine ? 1 : 0;
    if (rank < K) {
      tv[rank] = samp_val((unsigned)(mine >> 32));
      ti[rank] = (int)(0xffffffffu - (unsigned)(mine & 0xffffffffu));
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  // valid candidates of the row, at most K of them (each rank < K was written)
  int nv = 0;
  for (int i = tid; i < M; i += 64) nv += okey[i] != 0ull ? 1 : 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) nv += __shfl_xor(nv, o);
  nv = min(nv, K);
  const int lane = tid;
  if (nv == 0) {  // no finite logit: the walk flags the row
    if (lane == 0) part[(size_t)row * SAMP_NCHUNK] = 0ull;
    return;
  }
  // unnormalised masses, inclusive prefix sums in lane order (a fixed order)
  const float v0 = tv[0];
  float pm = lane < nv ? __builtin_amdgcn_exp2f((tv[min(lane, nv - 1)] - v0) * tscale) : 0.f;
  float c = pm;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float up = __shfl_up(c, o);
    if (lane >= o) c += up;
  }
  const float total = __shfl(c, nv - 1);
  const unsigned long long cut = __ballot(lane < nv && c >= top_p * total);
  const int m = cut ? __ffsll((long long)cut) : nv;  // kept prefix length
  const float R = __shfl(c, m - 1);
  const float t = uniforms[row] * R;
  const unsigned long long hit = __ballot(lane < m && c > t);
  const int pick = hit ? __ffsll((long long)hit) - 1 : m - 1;
  if (lane == 0) {
    const int tok = ti[pick];
    part[(size_t)row * SAMP_NCHUNK] = (1ull << 32) | (unsigned long long)(0xffffffffu - (unsigned)tok);
  }
}

int check_plan(const ddt_plan *P);
// the greedy walk over per-node tokens given as chunk keys (walk.hip)
int launch_walk(const ddt_plan *P, int V, int nchunk_used, const unsigned long long *part,
                const int32_t *draft_tok, int32_t *tokens, int32_t *path, int32_t *L, int32_t *bonus,
                hipStream_t st);

struct SampCfg {
  int C, chunk, G;
};
static SampCfg samp_cfg(int rows, int V) {
  SampCfg c{};
  int C = (256 + rows - 1) / rows;
  const int cap = SAMP_GMAX * 256 * 8;
  const int need = (V + cap - 1) / cap;
  if (C < need) C = need;
  if (C > SAMP_CMAX) C = SAMP_CMAX;
  const int maxc = (V + 255) / 256;  // chunks of at least 256 elements
  if (C > maxc) C = maxc < 1 ? 1 : maxc;
  c.chunk = ((V + C - 1) / C + 7) / 8 * 8;
  c.C = (V + c.chunk - 1) / c.chunk;
  const int g = (c.chunk + 256 * 8 - 1) / (256 * 8);
  c.G = g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : g <= 8 ? 8 : 12;
  return c;
}

}  // namespace ddt

using namespace ddt;

extern "C" size_t ddt_accept_sample_workspace(const ddt_plan *P, int32_t V, int32_t top_k) {
  if (!P || P->n_total < 1 || V < 1 || top_k < 1 || top_k > SAMP_KMAX) return 0;
  const SampCfg c = samp_cfg(P->n_total, V);
  const size_t part = (size_t)P->n_total * SAMP_NCHUNK * sizeof(unsigned long long);
  return part + (size_t)P->n_total * c.C * top_k * sizeof(float2);
}

extern "C" int ddt_accept_sample(const ddt_plan *P, const void *logits, int32_t dtype, int32_t V,
                                 const int32_t *draft_tok, const float *uniforms, float temperature,
                                 int32_t top_k, float top_p, int32_t *sample, int32_t *path, int32_t *L,
                                 int32_t *bonus, void *ws, size_t ws_bytes, void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!logits || !draft_tok || !uniforms || !sample || !path || !L || !bonus || !ws) return DDT_E_ARG;
  if (V < 1 || top_k < 1 || top_k > SAMP_KMAX) return DDT_E_SHAPE;
  if (!(temperature > 0.f) || !(temperature < INFINITY) || !(top_p > 0.f) || !(top_p <= 1.f)) return DDT_E_RANGE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  const SampCfg c = samp_cfg(P->n_total, V);
  if ((long long)c.chunk > (long long)SAMP_GMAX * 256 * 8 || c.chunk > (1 << 15)) return DDT_E_SHAPE;
  if (ws_bytes < ddt_accept_sample_workspace(P, V, top_k)) return DDT_E_WS;
  hipStream_t st = (hipStream_t)stream;
  auto *part = (unsigned long long *)ws;
  auto *cand = reinterpret_cast<float2 *>((char *)ws + (size_t)P->n_total * SAMP_NCHUNK * sizeof(unsigned long long));
  dim3 grid(c.C, P->n_total);
#define DDT_SAMP(TT, GG) \
  hipLaunchKernelGGL((samp_chunk_kernel<TT, GG>), grid, dim3(256), 0, st, (const TT *)logits, V, c.chunk, top_k, cand)
#define DDT_SAMP_G(TT)            \
  switch (c.G) {                  \
    case 1: DDT_SAMP(TT, 1); break; \
    case 2: DDT_SAMP(TT, 2); break; \
    case 4: DDT_SAMP(TT, 4); break; \
    case 8: DDT_SAMP(TT, 8); break; \
    default: DDT_SAMP(TT, 12); break; \
  }
  if (dtype == DDT_BF16) {
    DDT_SAMP_G(uint16_t);
  } else {
    DDT_SAMP_G(float);
  }
#undef DDT_SAMP_G
#undef DDT_SAMP
  r = launch_status();
  if (r) return r;
  hipLaunchKernelGGL(samp_merge_kernel, dim3(P->n_total), dim3(256), 0, st, cand, c.C, top_k, uniforms,
                     1.4426950408889634f / temperature, top_p, part);
  r = launch_status();
  if (r) return r;
  return launch_walk(P, V, 1, part, draft_tok, sample, path, L, bonus, st);
}
