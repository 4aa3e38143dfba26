// Test driver for the library's host-side code (csrc/host.cpp), built with
// the host sanitizers by tests/test_host_sanitize.py.  Reads cases from
// stdin, runs ddt_tree_plan_host / ddt_accept_walk_host on arrays of exactly
// the stated sizes (so a read past one is reported), and prints the return
// code and every output for the test to compare with the oracle.
//
//   plan  B n_total n_max W max_levels | tree_off[B+1] | parent[n_total]
//   walk  B n_total n_max V dtype | tree_off[B+1] | parent[n_total] |
//         draft_tok[n_total] | logits[n_total*V] as raw bits (u32 or u16)
#include <stdio.h>
#include <string.h>

#include <memory>
#include <string>

#include "ddtree.h"

template <typename T>
static std::unique_ptr<T[]> read_array(long n) {
  std::unique_ptr<T[]> a(new T[n > 0 ? n : 1]);
  for (long i = 0; i < n; ++i) {
    long long v;
    if (scanf("%lld", &v) != 1) return nullptr;
    a[i] = (T)v;
  }
  return a;
}

int main() {
  char what[16];
  int cases = 0;
  while (scanf("%15s", what) == 1) {
    int B, n_total, n_max, x, y;
    if (scanf("%d %d %d %d %d", &B, &n_total, &n_max, &x, &y) != 5) return 2;
    auto off = read_array<int32_t>(B + 1);
    auto par = read_array<int32_t>(n_total);
    if (!off || !par) return 2;
    ddt_plan P;
    memset(&P, 0, sizeof P);
    P.B = B, P.n_total = n_total, P.n_max = n_max, P.tree_off = off.get(), P.parent = par.get();
    std::unique_ptr<int32_t[]> status(new int32_t[B > 0 ? B : 1]());
    P.status = status.get();
    if (!strcmp(what, "plan")) {
      const int W = x, W1 = W - 1 > 1 ? W - 1 : 1;
      std::unique_ptr<int32_t[]> depth(new int32_t[n_total]()), win(new int32_t[(size_t)n_total * W1]());
      std::unique_ptr<uint64_t[]> anc(new uint64_t[n_total]());
      P.W = W, P.depth = depth.get(), P.anc = anc.get(), P.win = win.get();
      const int rc = ddt_tree_plan_host(&P, y);
      printf("rc %d\n", rc);
      if (rc == 0) {
        for (int i = 0; i < n_total; ++i) printf("%d%c", depth[i], i + 1 < n_total ? ' ' : '\n');
        for (int i = 0; i < n_total; ++i) printf("%llu%c", (unsigned long long)anc[i], i + 1 < n_total ? ' ' : '\n');
        for (long i = 0; i < (long)n_total * W1; ++i) printf("%d%c", win[i], i + 1 < (long)n_total * W1 ? ' ' : '\n');
      }
    } else if (!strcmp(what, "walk")) {
      const int V = x, dtype = y;
      auto tok = read_array<int32_t>(n_total);
      if (!tok) return 2;
      const long nl = (long)n_total * V;
      std::unique_ptr<uint32_t[]> l32;
      std::unique_ptr<uint16_t[]> l16;
      const void *logits;
      if (dtype == DDT_F32) {
        l32 = read_array<uint32_t>(nl);
        logits = l32.get();
      } else {
        l16 = read_array<uint16_t>(nl);
        logits = l16.get();
      }
      if (!logits) return 2;
      std::unique_ptr<int32_t[]> amax(new int32_t[n_total]), path(new int32_t[(size_t)B * n_max]),
          L(new int32_t[B]), bonus(new int32_t[B]);
      const int rc = ddt_accept_walk_host(&P, logits, dtype, V, tok.get(), amax.get(), path.get(), L.get(), bonus.get());
      printf("rc %d\n", rc);
      if (rc == 0) {
        for (int i = 0; i < n_total; ++i) printf("%d%c", amax[i], i + 1 < n_total ? ' ' : '\n');
        for (long i = 0; i < (long)B * n_max; ++i) printf("%d%c", path[i], i + 1 < (long)B * n_max ? ' ' : '\n');
        for (int b = 0; b < B; ++b) printf("%d %d %d\n", L[b], bonus[b], status[b]);
      }
    } else {
      return 2;
    }
    ++cases;
  }
  fprintf(stderr, "%d cases\n", cases);
  return 0;
}
