// Tree plan (host and device) and library-wide bits.
//
// The plan turns a parent-pointer draft tree (lucebox-hub README,
// "02 · DFlash DDtree", "Algorithms used": DDTree verifies a tree of draft
// tokens in one pass) into the index tables the other kernels read:
// depth, ancestor bitmask (the attention mask), conv windows, and a visit
// order with state slots for the tree recurrences.
//
// Visit order: a depth-first preorder in which the children of every node
// are visited by increasing (subtree size, index), so the largest subtree
// comes last.  A node's state must stay live until its last child has been
// computed; giving a node its parent's slot when it is that last child, and
// the parent's slot + 1 otherwise, never overwrites a live state, and each
// "+1" edge leads into a subtree at most half as large as its parent's, so
// floor(log2(n)) + 1 slots suffice for n nodes.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

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

static int plan_fields_ok(const ddt_plan *P) {
  if (!P) return DDT_E_ARG;
  if (P->B < 1 || P->n_total < 1 || P->n_max < 1 || P->n_max > DDT_MAX_NODES) return DDT_E_SHAPE;
  if (P->W < 1 || P->W > DDT_MAX_W) return DDT_E_SHAPE;
  if (!P->tree_off || !P->parent || !P->depth || !P->anc || !P->win || !P->order || !P->slot ||
      !P->status)
    return DDT_E_ARG;
  return DDT_OK;
}

int check_plan(const ddt_plan *P) { return plan_fields_ok(P); }

// ------------------------------------------------------------------ device plan
// One wavefront per sequence, lane c = node c.  After the parents are in LDS
// and each lane has chased its own root path, every table is built from
// loops over the nodes whose index is the same in all lanes, reading the
// other nodes' values out of their lanes (readlane) or as ballots, so no
// step waits on an LDS read.
__global__ __launch_bounds__(64) void plan_kernel(ddt_plan P, int max_levels) {
  __shared__ int par[64];
  const int b = blockIdx.x, c = threadIdx.x;
  unsigned st = 0;
  int o = P.tree_off[b], e = P.tree_off[b + 1];
  if (!(o >= 0 && e > o && e <= P.n_total && e - o <= P.n_max)) st |= DDT_ST_TREE;
  if (P.B == 1 && (o != 0 || e != P.n_total)) st |= DDT_ST_TREE;
  Seq s = seq_of(P, b);
  o = s.o;
  const int n = s.n;
  if (n == 0) {
    if (c == 0) P.status[b] = st | DDT_ST_TREE;
    return;
  }
  int p = (c < n) ? P.parent[o + c] : 0;
  bool ok = (c == 0) ? (p == -1) : (p >= 0 && p < c);
  if (c < n && !ok) p = (c == 0) ? -1 : 0;  // safe stand-in: hang it off the root
  if (__ballot(c < n && !ok)) st |= DDT_ST_TREE;
  const int pc = (c == 0) ? -1 : p;  // this node's parent
  par[c] = pc;
  __syncthreads();

  int d = 0;
  unsigned long long a = 0;
  if (c < n) {
    a = 1ull << c;
    for (int j = c; j > 0;) {
      j = par[j];
      a |= 1ull << j;
      ++d;
    }
  }
  int dmax = d;
  for (int off = 32; off > 0; off >>= 1) dmax = max(dmax, __shfl_xor(dmax, off));
  if (dmax + 1 > max_levels) st |= DDT_ST_LEVELS;

  // subtree sizes: the nodes whose root path holds x, one ballot per x
  int size = 0;
  for (int x = 0; x < n; ++x) {
    const unsigned long long m = __ballot(c < n && ((a >> x) & 1ull));
    if (c == x) size = __popcll(m);
  }
  // heaviest child = the one visited last: largest (size, index); and the
  // summed sizes of the siblings visited before this node (smaller (size,
  // index) under the same parent)
  int hv = -1, hvs = 0, sb = 0;
  for (int j = 1; j < n; ++j) {
    const int pj = __builtin_amdgcn_readlane(pc, j), sj = __builtin_amdgcn_readlane(size, j);
    if (pj == c && (hv < 0 || sj >= hvs)) {
      hv = j;
      hvs = sj;
    }
    if (pj == pc && j != c && (sj < size || (sj == size && j < c))) sb += sj;
  }
  // a node is light if it is not its parent's heaviest child
  int hpar = -1;
  for (int y = 0; y < n; ++y) {
    const int hy = __builtin_amdgcn_readlane(hv, y);
    if (y == pc) hpar = hy;
  }
  const int light1 = (c > 0 && hpar != c) ? 1 : 0;

  if (c < n) {
    const int g = o + c;
    // preorder position: the proper ancestors, plus for every node x on the
    // root path (root excluded) the subtrees of the siblings visited before x
    int pos = d, light = 0;
    for (int x = 1; x < n; ++x) {
      const int sbx = __builtin_amdgcn_readlane(sb, x), lx = __builtin_amdgcn_readlane(light1, x);
      if ((a >> x) & 1ull) {
        pos += sbx;
        light += lx;
      }
    }
    P.order[o + pos] = c;
    P.slot[g] = light;
    P.depth[g] = d;
    P.anc[g] = a;
    const int W1 = P.W - 1;
    int y = c, m = 0;  // walk up one ancestor per window entry
    for (int j = 1; j <= W1; ++j) {
      if (m < d) {
        y = par[y];
        ++m;
        P.win[(size_t)g * W1 + (j - 1)] = y;
      } else {
        int sl = W1 - (j - d);
        P.win[(size_t)g * W1 + (j - 1)] = -(sl + 1);
      }
    }
    if (W1 == 0) P.win[g] = 0;
  }
  if (c == 0) P.status[b] = st;
}

}  // namespace ddt

using namespace ddt;

extern "C" int ddt_version(void) { return DDT_VERSION; }

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

extern "C" int ddt_plan_slots(int32_t n_max) {
  if (n_max < 1) return 1;
  int s = 0;
  while ((2 << s) <= n_max) ++s;  // floor(log2(n_max))
  return s + 1;
}

extern "C" int ddt_tree_plan(const ddt_plan *P, int32_t max_levels, void *stream) {
  int r = plan_fields_ok(P);
  if (r) return r;
  if (max_levels < 1) return DDT_E_RANGE;
  hipLaunchKernelGGL(plan_kernel, dim3(P->B), dim3(64), 0, (hipStream_t)stream, *P, max_levels);
  return launch_status();
}

// ------------------------------------------------------------------ host plan
extern "C" int ddt_tree_plan_host(const ddt_plan *P, int32_t max_levels) {
  int r = plan_fields_ok(P);
  if (r) return r;
  if (max_levels < 1) return DDT_E_RANGE;
  const int B = P->B, W1 = P->W - 1;
  if (P->tree_off[0] != 0 || P->tree_off[B] != P->n_total) return DDT_E_TREE;
  // validate everything before writing anything
  for (int b = 0; b < B; ++b) {
    int o = P->tree_off[b], n = P->tree_off[b + 1] - o;
    if (n < 1 || n > P->n_max) return DDT_E_TREE;
    if (P->parent[o] != -1) return DDT_E_TREE;
    for (int i = 1; i < n; ++i)
      if (P->parent[o + i] < 0 || P->parent[o + i] >= i) return DDT_E_TREE;
    std::vector<int> d(n, 0);
    for (int i = 1; i < n; ++i) {
      d[i] = d[P->parent[o + i]] + 1;
      if (d[i] + 1 > max_levels) return DDT_E_RANGE;
    }
  }
  for (int b = 0; b < B; ++b) {
    const int o = P->tree_off[b], n = P->tree_off[b + 1] - o;
    const int32_t *par = P->parent + o;
    std::vector<int> d(n, 0), size(n, 1);
    std::vector<unsigned long long> a(n, 1ull);
    for (int i = 1; i < n; ++i) {
      d[i] = d[par[i]] + 1;
      a[i] = a[par[i]] | (1ull << i);
    }
    a[0] = 1ull;
    for (int i = n - 1; i > 0; --i) size[par[i]] += size[i];
    std::vector<std::vector<int>> ch(n);
    for (int i = 1; i < n; ++i) ch[par[i]].push_back(i);
    for (auto &v : ch)
      std::sort(v.begin(), v.end(), [&](int x, int y) {
        return size[x] != size[y] ? size[x] < size[y] : x < y;
      });
    std::vector<int> slot(n, 0), ord;
    std::vector<int> stack{0};
    while (!stack.empty()) {  // preorder, children by increasing (size, index)
      int u = stack.back();
      stack.pop_back();
      ord.push_back(u);
      for (int k = (int)ch[u].size() - 1; k >= 0; --k) stack.push_back(ch[u][k]);
      for (size_t k = 0; k < ch[u].size(); ++k)
        slot[ch[u][k]] = slot[u] + (k + 1 == ch[u].size() ? 0 : 1);
    }
    for (int i = 0; i < n; ++i) {
      P->depth[o + i] = d[i];
      P->anc[o + i] = a[i];
      P->order[o + i] = ord[i];
      P->slot[o + i] = slot[i];
      int y = i;
      for (int j = 1; j <= W1; ++j) {
        int v;
        if (j <= d[i]) {
          y = par[y];
          v = y;
        } else {
          v = -((W1 - (j - d[i])) + 1);
        }
        P->win[(size_t)(o + i) * W1 + (j - 1)] = v;
      }
      if (W1 == 0) P->win[o + i] = 0;
    }
    P->status[b] = 0;
  }
  return DDT_OK;
}
