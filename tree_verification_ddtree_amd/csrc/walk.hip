// Verify argmax and greedy acceptance walk.
//
// The verify argmax is read in place from the device logits and its result
// is validated (codehub lucebox-hub@main, "GPU draft top-K & verify-argmax
// (DFlash)"); acceptance is greedy (same page, "Run the Server", "Making
// requests").  The argmax streams n x V logits (22 x 151,936 bf16 = 6.7 MB
// at budget 22), so it is spread over NCHUNK workgroups per row, each
// reducing a 64-bit key (order-preserving value bits << 32 | ~index): the
// maximum key is the largest value at the smallest index, and max is
// associative, so the result does not depend on reduction order.  NaN is
// keyed as -inf and -0 as +0.  A second kernel (one wavefront per tree)
// combines the chunk keys, validates, and walks the tree with ballots.
#include <mutex>

#include "common.h"

namespace ddt {

constexpr int NCHUNK = 16;

__device__ __forceinline__ unsigned long long key_of(float f, unsigned idx) {
  uint32_t u = __float_as_uint(f);
  if (f != f) u = 0xff800000u;  // NaN -> -inf
  if (f == 0.0f) u = 0u;        // -0 -> +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - idx);
}

__device__ __forceinline__ unsigned long long kmax(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

template <typename T>
__global__ __launch_bounds__(256) void argmax_chunks(const T *__restrict__ logits, int V,
                                                     int n_total, int chunk,
                                                     unsigned long long *__restrict__ part) {
  const int row = blockIdx.y, ck = blockIdx.x;
  const int lo = ck * chunk, hi = min(V, lo + chunk);
  const T *p = logits + (size_t)row * V;
  unsigned long long best = 0;
  // chunk is a multiple of 8 and V % 8 == 0 on the vector path
  const bool vec = (V % 8 == 0);
  if (vec) {
    for (int i = lo + threadIdx.x * 8; i < hi; i += 256 * 8) {
      float f[8];
      load8(p + i, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) best = kmax(best, key_of(f[e], (unsigned)(i + e)));
    }
  } else {
    for (int i = lo + threadIdx.x; i < hi; i += 256) best = kmax(best, key_of(load1(p + i), i));
  }
  for (int off = 32; off > 0; off >>= 1) best = kmax(best, __shfl_xor(best, off));
  __shared__ unsigned long long red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0)
    part[(size_t)row * NCHUNK + ck] = kmax(kmax(red[0], red[1]), kmax(red[2], red[3]));
}

__global__ __launch_bounds__(64) void walk_kernel(ddt_plan P, int V, int nchunk_used,
                                                  const unsigned long long *__restrict__ part,
                                                  const int32_t *__restrict__ tok,
                                                  int32_t *__restrict__ amax,
                                                  int32_t *__restrict__ path,
                                                  int32_t *__restrict__ L,
                                                  int32_t *__restrict__ bonus) {
  __shared__ int am[64];
  const int b = blockIdx.x, c = threadIdx.x;
  const Seq s = seq_of(P, b);
  unsigned st = 0;
  int a = 0, tc = -1, par = -2;
  if (c < s.n) {
    unsigned long long k = 0;
    for (int j = 0; j < nchunk_used; ++j) k = kmax(k, part[(size_t)(s.o + c) * NCHUNK + j]);
    unsigned idx = 0xffffffffu - (unsigned)(k & 0xffffffffu);
    if (k == 0 || idx >= (unsigned)V) {
      st |= DDT_ST_ARGMAX;
      idx = 0;
    }
    a = (int)idx;
    amax[s.o + c] = a;
    tc = tok[s.o + c];
    if (c > 0 && (tc < 0 || tc >= V)) st |= DDT_ST_TOKEN;
    par = (c == 0) ? -1 : P.parent[s.o + c];
  }
  am[c] = a;
  __syncthreads();
  int cur = 0, len = 1;
  if (c == 0 && s.n > 0) path[(size_t)b * P.n_max] = 0;
  for (int step = 1; step < s.n; ++step) {
    const int want = am[cur];
    unsigned long long m = __ballot(c < s.n && c > cur && par == cur && tc == want);
    if (!m) break;
    cur = __ffsll((long long)m) - 1;
    if (c == 0) path[(size_t)b * P.n_max + len] = cur;
    ++len;
  }
  for (int j = len + c; j < P.n_max; j += 64) path[(size_t)b * P.n_max + j] = -1;
  unsigned all = st;
  for (int off = 32; off > 0; off >>= 1) all |= __shfl_xor(all, off);
  if (c == 0) {
    L[b] = s.n > 0 ? len : 0;
    bonus[b] = am[cur];
    if (all) P.status[b] |= (int32_t)all;
  }
}

int check_plan(const ddt_plan *P);

// The walk over per-node tokens given as chunk keys (nchunk_used of them per
// node, stride NCHUNK): used by the greedy walk and by the sampled one.
int launch_walk(const ddt_plan *P, int V, int nchunk_used, const unsigned long long *part,
                const int32_t *draft_tok, int32_t *tokens, int32_t *path, int32_t *L, int32_t *bonus,
                hipStream_t st) {
  hipLaunchKernelGGL(walk_kernel, dim3(P->B), dim3(64), 0, st, *P, V, nchunk_used, part, draft_tok, tokens,
                     path, L, bonus);
  return launch_status();
}

}  // namespace ddt

using namespace ddt;

static int chunk_len(int V) { return ((V + NCHUNK - 1) / NCHUNK + 7) / 8 * 8; }

extern "C" size_t ddt_accept_walk_workspace(const ddt_plan *P, int32_t V) {
  (void)V;
  if (!P || P->n_total < 1) return 0;
  return (size_t)P->n_total * NCHUNK * sizeof(unsigned long long);
}

// The argmax and the walk with the chunk keys in `part` (n_total * NCHUNK
// keys): argmax_chunks writes every key the walk reads, so `part` needs no
// initialisation.
static int walk_with(const ddt_plan *P, const void *logits, int32_t dtype, int32_t V, const int32_t *draft_tok,
                     int32_t *argmax, int32_t *path, int32_t *L, int32_t *bonus, unsigned long long *part,
                     hipStream_t st) {
  const int chunk = chunk_len(V);
  const int used = (V + chunk - 1) / chunk;
  dim3 grid(used, P->n_total);
  if (dtype == DDT_BF16)
    hipLaunchKernelGGL(argmax_chunks<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)logits,
                       V, P->n_total, chunk, part);
  else if (dtype == DDT_F32)
    hipLaunchKernelGGL(argmax_chunks<float>, grid, dim3(256), 0, st, (const float *)logits, V,
                       P->n_total, chunk, part);
  else
    return DDT_E_DTYPE;
  const int r = launch_status();
  if (r) return r;
  return launch_walk(P, V, used, part, draft_tok, argmax, path, L, bonus, st);
}

extern "C" int ddt_accept_walk(const ddt_plan *P, const void *logits, int32_t dtype, int32_t V,
                               const int32_t *draft_tok, int32_t *argmax, int32_t *path,
                               int32_t *L, int32_t *bonus, void *ws, size_t ws_bytes,
                               void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!logits || !draft_tok || !argmax || !path || !L || !bonus || !ws) return DDT_E_ARG;
  if (V < 1) return DDT_E_SHAPE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  if (ws_bytes < ddt_accept_walk_workspace(P, V)) return DDT_E_WS;
  return walk_with(P, logits, dtype, V, draft_tok, argmax, path, L, bonus, (unsigned long long *)ws,
                   (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// The walk for callers that cannot allocate: its chunk keys live in a
// file-scope device array.  Each GPU holds its own copy of the array at its
// own address, found once per device with hipGetSymbolAddress while that
// device is current; host code passes that address, never the array's name
// (which on the host is only a stand-in, not a device address).
static __device__ __align__(256) unsigned long long scratch[DDT_NOALLOC_MAX_NODES * NCHUNK];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
unsigned long long *g_scratch[MAX_DEVICES] = {};

// address of this device's copy of `scratch` (NULL and a recorded HIP error
// if it cannot be had)
unsigned long long *scratch_of_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_hip_error(e);
    return nullptr;
  }
  if (dev < 0 || dev >= MAX_DEVICES) {
    set_hip_error(hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      set_hip_error(e);
      return nullptr;
    }
    g_scratch[dev] = (unsigned long long *)ptr;
  }
  return g_scratch[dev];
}
}  // namespace

extern "C" int ddt_accept_walk_noalloc(const ddt_plan *P, const void *logits, int32_t dtype, int32_t V,
                                       const int32_t *draft_tok, int32_t *argmax, int32_t *path, int32_t *L,
                                       int32_t *bonus, void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!logits || !draft_tok || !argmax || !path || !L || !bonus) return DDT_E_ARG;
  if (V < 1 || P->n_total > DDT_NOALLOC_MAX_NODES) return DDT_E_SHAPE;
  if (dtype != DDT_BF16 && dtype != DDT_F32) return DDT_E_DTYPE;
  unsigned long long *part = scratch_of_current_device();
  if (!part) return DDT_E_HIP;
  return walk_with(P, logits, dtype, V, draft_tok, argmax, path, L, bonus, part, (hipStream_t)stream);
}
