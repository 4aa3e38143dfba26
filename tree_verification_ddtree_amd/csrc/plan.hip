// Tree plan on the device and library-wide bits (the host plan is in host.cpp).
//
// The plan turns a parent-pointer draft tree (lucebox-hub README,
// "02 · DFlash DDtree", "Algorithms used": DDTree verifies a tree of draft
// tokens in one pass) into the index tables the other kernels read: depth,
// ancestor bitmask (the attention mask and the delta-net's root paths) and
// conv windows.  Parents precede their children, so index order is already
// topological and no visit order is needed.
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace ddt {

static thread_local char g_hip_msg[256] = "";

void set_hip_error(hipError_t e) {
  snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error %d: %s", (int)e, hipGetErrorString(e));
}

int launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_hip_error(e);
    return DDT_E_HIP;
  }
  return DDT_OK;
}

// the plan fields check (host.cpp)
int check_plan(const ddt_plan *P);

// ------------------------------------------------------------------ device plan
// One wavefront per sequence, lane c = node c, nothing through LDS.  The
// ancestor masks come from pointer jumping: after round k every lane holds
// the nodes within 2^k steps above it and a pointer 2^k steps up (the root
// points at itself), so six rounds cover any tree of up to 64 nodes.  The
// depth is the mask's population count less one.  Ancestors have smaller
// indices than their descendants, so the j-th previous token of a node is
// the j-th highest bit of its mask below its own.
__global__ __launch_bounds__(64) void plan_kernel(ddt_plan P, int max_levels) {
  const int b = blockIdx.x, c = threadIdx.x;
  unsigned st = 0;
  {
    const int o = P.tree_off[b], e = P.tree_off[b + 1];
    if (!(o >= 0 && e > o && e <= P.n_total && e - o <= P.n_max)) st |= DDT_ST_TREE;
    if (P.B == 1 && (o != 0 || e != P.n_total)) st |= DDT_ST_TREE;
  }
  const Seq s = seq_of(P, b);
  const int o = s.o, n = s.n;
  if (n == 0) {
    if (c == 0) P.status[b] = st | DDT_ST_TREE;
    return;
  }
  const bool on = c < n;
  int p = on ? P.parent[o + c] : 0;
  const bool ok = (c == 0) ? (p == -1) : (p >= 0 && p < c);
  if (__ballot(on && !ok)) st |= DDT_ST_TREE;
  if (on && !ok) p = (c == 0) ? -1 : 0;  // safe stand-in: hang it off the root
  // lanes past the tree point at themselves and hold no nodes
  int up = !on ? c : (c == 0 ? 0 : p);
  unsigned long long a = !on ? 0ull : ((1ull << c) | (1ull << up));
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const unsigned lo = __shfl((unsigned)a, up), hi = __shfl((unsigned)(a >> 32), up);
    a |= ((unsigned long long)hi << 32) | lo;
    up = __shfl(up, up);
  }
  const int d = on ? __popcll(a) - 1 : 0;
  int dmax = d;
  for (int off = 32; off > 0; off >>= 1) dmax = max(dmax, __shfl_xor(dmax, off));
  if (dmax + 1 > max_levels) st |= DDT_ST_LEVELS;
  if (on) {
    const int g = o + c;
    P.depth[g] = d;
    P.anc[g] = a;
    const int W1 = P.W - 1;
    unsigned long long m = a & ~(1ull << c);  // proper ancestors
    for (int j = 1; j <= W1; ++j) {
      int v;
      if (j <= d) {
        v = 63 - __clzll((long long)m);  // nearest remaining ancestor
        m &= ~(1ull << v);
      } else {
        v = -((W1 - (j - d)) + 1);  // committed prefix slot W1 - (j - d)
      }
      P.win[(size_t)g * W1 + (j - 1)] = v;
    }
    if (W1 == 0) P.win[g] = 0;
  }
  if (c == 0) P.status[b] = st;
}

}  // namespace ddt

using namespace ddt;

extern "C" int ddt_version(void) { return DDT_VERSION; }

// The build passes the sha256 of the sources it compiled (build.py,
// source_hash); a build that does not says so.
#ifndef DDT_SOURCE_HASH
#define DDT_SOURCE_HASH "unknown"
#endif
extern "C" const char *ddt_source_hash(void) { return DDT_SOURCE_HASH; }

extern "C" const char *ddt_status_str(int code) {
  switch (code) {
    case DDT_OK: return "ok";
    case DDT_E_ARG: return "null pointer or bad argument";
    case DDT_E_TREE: return "malformed tree";
    case DDT_E_SHAPE: return "unsupported or inconsistent sizes";
    case DDT_E_DTYPE: return "unsupported storage type";
    case DDT_E_RANGE: return "value out of range";
    case DDT_E_WS: return "workspace too small";
    case DDT_E_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
    default: return "unknown status";
  }
}

extern "C" int ddt_tree_plan(const ddt_plan *P, int32_t max_levels, void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (max_levels < 1) return DDT_E_RANGE;
  hipLaunchKernelGGL(plan_kernel, dim3(P->B), dim3(64), 0, (hipStream_t)stream, *P, max_levels);
  return launch_status();
}
