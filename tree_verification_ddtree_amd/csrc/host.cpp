// Host-side half of the library: the plan fields check every entry point
// runs, the tree plan on the host, and the acceptance walk on the host.
//
// The walk on the host is the fall-back path of the verify step: the pages'
// GPU argmax is validated and the host takes over when it fails (codehub
// lucebox-hub@main, "GPU draft top-K & verify-argmax (DFlash)").  The device
// walk reports such failures in the plan's status word; a caller that sees
// one runs this walk on host copies of the logits and draft tokens.  It is
// plain C++ (no HIP), so it can also be built and run under the host
// sanitizers.
#include <string.h>

#include <vector>

#include "ddtree.h"

namespace ddt {

int check_plan(const ddt_plan *P) {
  if (!P) return DDT_E_ARG;
  if (P->B < 1 || P->n_total < 1 || P->n_max < 1 || P->n_max > DDT_MAX_NODES) return DDT_E_SHAPE;
  if (P->W < 1 || P->W > DDT_MAX_W) return DDT_E_SHAPE;
  if (!P->tree_off || !P->parent || !P->depth || !P->anc || !P->win || !P->status) return DDT_E_ARG;
  return DDT_OK;
}

// Every tree of a host plan well formed: offsets from 0 to n_total, each
// tree 1..n_max nodes, parent[0] = -1 and 0 <= parent[i] < i.
static int trees_ok(const ddt_plan *P) {
  const int B = P->B;
  if (P->tree_off[0] != 0 || P->tree_off[B] != P->n_total) return DDT_E_TREE;
  for (int b = 0; b < B; ++b) {
    const int o = P->tree_off[b], n = P->tree_off[b + 1] - o;
    if (o < 0 || n < 1 || n > P->n_max || o + n > P->n_total) return DDT_E_TREE;
    if (P->parent[o] != -1) return DDT_E_TREE;
    for (int i = 1; i < n; ++i)
      if (P->parent[o + i] < 0 || P->parent[o + i] >= i) return DDT_E_TREE;
  }
  return DDT_OK;
}

// Order-preserving key of a logit: larger value gives a larger key, NaN is
// keyed as -inf and -0 as +0, so equal keys are equal values.
static uint32_t logit_key(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (f != f) u = 0xff800000u;
  if (f == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

static float logit_at(const void *logits, int32_t dtype, size_t i) {
  if (dtype == DDT_F32) return static_cast<const float *>(logits)[i];
  const uint32_t u = (uint32_t) static_cast<const uint16_t *>(logits)[i] << 16;  // bf16: the high half
  float f;
  memcpy(&f, &u, 4);
  return f;
}

}  // namespace ddt

using namespace ddt;

extern "C" int ddt_tree_plan_host(const ddt_plan *P, int32_t max_levels) {
  int r = check_plan(P);
  if (r) return r;
  if (max_levels < 1) return DDT_E_RANGE;
  const int B = P->B, W1 = P->W - 1;
  // validate everything before writing anything
  r = trees_ok(P);
  if (r) return r;
  for (int b = 0; b < B; ++b) {
    const int o = P->tree_off[b], n = P->tree_off[b + 1] - o;
    std::vector<int> d(n, 0);
    for (int i = 1; i < n; ++i) {
      d[i] = d[P->parent[o + i]] + 1;
      if (d[i] + 1 > max_levels) return DDT_E_RANGE;
    }
  }
  for (int b = 0; b < B; ++b) {
    const int o = P->tree_off[b], n = P->tree_off[b + 1] - o;
    const int32_t *par = P->parent + o;
    std::vector<int> d(n, 0);
    std::vector<unsigned long long> a(n, 1ull);
    for (int i = 1; i < n; ++i) {
      d[i] = d[par[i]] + 1;
      a[i] = a[par[i]] | (1ull << i);
    }
    for (int i = 0; i < n; ++i) {
      P->depth[o + i] = d[i];
      P->anc[o + i] = a[i];
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

extern "C" int ddt_accept_walk_host(const ddt_plan *P, const void *logits, int32_t dtype, int32_t V,
                                    const int32_t *draft_tok, int32_t *argmax, int32_t *path, int32_t *L,
                                    int32_t *bonus) {
  if (!P || !P->tree_off || !P->parent || !P->status) return DDT_E_ARG;
  if (!logits || !draft_tok || !argmax || !path || !L || !bonus) return DDT_E_ARG;
  if (P->B < 1 || P->n_total < 1 || P->n_max < 1 || P->n_max > DDT_MAX_NODES) return DDT_E_SHAPE;
  if (dtype != DDT_F32 && dtype != DDT_BF16) return DDT_E_DTYPE;
  if (V < 1) return DDT_E_SHAPE;
  const int r = trees_ok(P);
  if (r) return r;
  // argmax of every row: the largest key at the smallest index
  for (int i = 0; i < P->n_total; ++i) {
    const size_t row = (size_t)i * (size_t)V;
    uint32_t best = logit_key(logit_at(logits, dtype, row));
    int arg = 0;
    for (int v = 1; v < V; ++v) {
      const uint32_t k = logit_key(logit_at(logits, dtype, row + (size_t)v));
      if (k > best) best = k, arg = v;
    }
    argmax[i] = arg;
  }
  for (int b = 0; b < P->B; ++b) {
    const int o = P->tree_off[b], n = P->tree_off[b + 1] - o;
    int32_t st = 0;
    for (int c = 1; c < n; ++c)
      if (draft_tok[o + c] < 0 || draft_tok[o + c] >= V) st |= (int32_t)DDT_ST_TOKEN;  // can never match
    int32_t *pb = path + (size_t)b * P->n_max;
    int cur = 0, len = 1;
    pb[0] = 0;
    for (;;) {
      // children of cur have larger indices; the smallest one whose draft
      // token is cur's argmax is taken
      int nxt = -1;
      for (int c = cur + 1; c < n && nxt < 0; ++c)
        if (P->parent[o + c] == cur && draft_tok[o + c] == argmax[o + cur]) nxt = c;
      if (nxt < 0) break;
      pb[len++] = nxt;
      cur = nxt;
    }
    for (int j = len; j < P->n_max; ++j) pb[j] = -1;
    L[b] = len;
    bonus[b] = argmax[o + cur];
    P->status[b] |= st;
  }
  return DDT_OK;
}
