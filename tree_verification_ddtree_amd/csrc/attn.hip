// Tree-masked attention over a paged fp16 or 8-bit KV cache.
//
// Each tree node attends to all committed tokens of its sequence and to the
// draft tokens on its own root path (the whole tree is verified in one pass:
// lucebox-hub README, "02 · DFlash DDtree", "Algorithms used"); attention is
// full (codehub lucebox-hub@main, "Server flags", --fa-window 0) and the
// cache may be paged (Luce-Org/lucebox README, "Inference Engine
// Optimizations").  The pages call the verify step bandwidth bound
// (lucebox-hub README, "Retune per GPU"; "AMD Strix Halo (HIP backend)").
//
// Design for gfx950.  All G = Hq/Hkv query heads of all n tree nodes share
// one KV head, so a workgroup owns one KV head, one context split and up to
// 192 query rows (row = node * G + head): every K/V byte is read from HBM
// once per split and feeds 6*n rows (132 at budget 22).
//  - Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_f16: A = 16 keys x 32 channels (from LDS),
//    B = 32 channels x 16 rows (Q, resident in VGPRs for the whole split).
//    The accumulator then holds, per lane, 4 keys of ONE query row, so the
//    online-softmax statistics of a row live in one lane (replicated over
//    the 4 lane groups) and the probabilities are already in the B-operand
//    layout of the next product: O^T += V^T P^T (A = 16 channels x 32 keys
//    of V^T from LDS, B = P).  Keys are permuted inside a 32-key tile so
//    that lane group q holds keys 8q..8q+7 -- exactly the 8 consecutive
//    tokens that one 16-byte read of a channel-major V page provides.
//  - K and V pages go straight from HBM into a 4-stage LDS ring
//    (global_load_lds_dwordx4, up to three 32-key tiles in flight, no
//    staging registers); each direct load of a wavefront reads one page, at
//    a wave-uniform page base plus a lane offset fixed for the whole split.
//    16-byte chunks are XOR-swizzled so the operand reads of a wavefront
//    hit distinct banks.  The ragged last tile and the tree tiles go
//    through registers so keys past the end can be zero-filled.
//  - One wavefront per SIMD (the accumulators and resident Q take ~490
//    registers per lane), so a VALU instruction runs in the shadow of the
//    matrix pipe only when it sits between two MFMAs: the scores of the next
//    tile are issued with the tile's loads and block 0's probabilities
//    between them, and block j's value product with block j + 1's.
//  - Rows: 16-row blocks are dealt round-robin to the 4 wavefronts (NB
//    blocks each).  A wavefront skips blocks past the sequence's rows.
//  - The tree itself is one or two extra 32-key tiles (draft K/V of up to
//    64 nodes) processed by the last split of the sequence, masked by the
//    plan's ancestor bitmask; cache keys are never masked per row.  That
//    split stages its first tree tile in a fifth LDS stage before its main
//    loop (fp16 path), so at the end the tile costs it only its matrix work,
//    not a memory round trip.
//  - Online softmax without rescaling the accumulators and without a
//    cross-lane max per tile: a row's reference max is fixed by its first
//    tile and probabilities are formed against it (fp16 P has 15 binades
//    of headroom above 1); each lane only checks its own scores.  A split whose scores
//    outgrow that headroom is recomputed with the true maxima, so the
//    result is exact either way; on ordinary data the redo never happens.
//  - Each split writes its output rows divided by their row sums (fp16),
//    its reference max and the row sum; a combine kernel merges the splits
//    in fixed order (deterministic, no atomics).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace ddt {

// Cache policy of the loads of cache pages: non-temporal (the nt bit).  Each
// K/V byte is read once per call; with the hint the 128K, 22-node call measured
// 115.0 us against 121.8 us with the default policy.
constexpr int KV_STREAM_CPOL = 2;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 32;  // keys per pipeline stage (two pages)
constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
  ddt_plan P;
  const _Float16 *q, *Kc, *Vc, *Kt, *Vt;
  // 8-bit cache (Q8 path): Kq [P][Hkv][16][D], Vq [P][Hkv][D][16] int8 and one
  // fp16 scale per token, Ksc / Vsc [P][Hkv][16]; a value is fp16(q * scale)
  const int8_t *Kq, *Vq;
  const _Float16 *Ksc, *Vsc;
  const int32_t *pt;
  int max_pages;
  const int32_t *T;
  int T_max;
  int Hq, Hkv, G;
  float c;  // scale * log2(e)
  int n_splits, n_rg, rows_wg;
  // a split's output rows divided by their own row sums, in fp16 (values of
  // V's range; the rounding, 2^-11 relative, stays within the fp16 inputs'
  // own precision), and each row's reference max and sum
  _Float16 *Opart;  // [B][Hkv][n_rg][n_splits][rows_wg][D]
  float2 *ML;       // [B][Hkv][n_rg][n_splits][rows_wg]
  float *out;    // [n_total][Hq][D]
};

// committed length actually readable for sequence b (and whether it was cut)
__device__ __forceinline__ int ctx_len(const AttnArgs &A, int b, bool *cut) {
  int t = A.T[b];
  bool bad = false;
  if (t < 0) { t = 0; bad = true; }
  if (t > A.T_max) { t = A.T_max; bad = true; }
  if (A.pt && t > A.max_pages * DDT_PAGE) { t = A.max_pages * DDT_PAGE; bad = true; }
  if (cut) *cut = bad;
  return t;
}

// Keys per split of a sequence with Tb committed tokens and nb splits: the
// sequence's own length spread over its splits, in whole tiles, so every
// active split gets the same number of tiles (give or take one).
__device__ __forceinline__ int split_chunk(int Tb, int nb) {
  int c = (Tb + nb - 1) / nb;
  c = (c + TILE - 1) / TILE * TILE;
  return c < TILE ? TILE : c;
}

typedef __attribute__((address_space(4))) const int32_t cint32;

// Page of cache position t of sequence b, t the same in every lane (the
// first key of a tile).  The read goes through the scalar cache: waiting for
// it uses the scalar counter, so it never forces the wave to wait for the
// K/V tiles still in flight on the vector-memory counter.
__device__ __forceinline__ int page_uniform(const AttnArgs &A, int b, int t) {
  if (!A.pt) return t >> 4;
  const int pg = __builtin_amdgcn_readfirstlane(t >> 4);
  return *(const cint32 *)(A.pt + (size_t)b * A.max_pages + pg);
}

__device__ __forceinline__ int n_active_splits(int Tb, int nb) {
  const int chunk = split_chunk(Tb, nb);
  int n = (Tb + chunk - 1) / chunk;
  n = n < 1 ? 1 : n;
  return n > nb ? nb : n;
}

// The batch's sequences share the A.n_splits context splits of a (KV head,
// row group): every sequence with rows in the row group takes one, and the
// rest are dealt in proportion to each sequence's tiles (cache and tree),
// with at least 256 keys per split.  All splits stream at once, each at an
// equal share of the memory bandwidth, so a split's time is its tile count
// as long as its matrix work per tile hides under that share; beyond nine
// 16-row blocks in the row group (every wavefront then holds three) it does
// not, and a tile of such a sequence weighs 1 + (blocks - 9) / 12 (32 nodes
// at 6 query heads: 1.25).  The shares are rounded cumulatively (sequence b
// gets E S_(b+1) / W - E S_b / W, floors of its prefix sums of weights), so
// the whole pool is dealt.  A short context then no longer waits on a long
// one that has the same number of splits.  Every workgroup of the attention
// kernel and of the combine computes the same deal from the committed
// lengths (one lane per sequence).  A batch of one sequence launches the
// direct mapping instead.
struct PoolSlot {
  int b, j, nb, first;  // sequence, its split, its split count, its first pool split
};
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ long long wave_incl_scan_ll(long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// want_b >= 0: the deal of sequence want_b; otherwise the sequence that pool
// split s belongs to (b = -1 past the last dealt split).
__device__ PoolSlot pool_slot(const AttnArgs &A, int rg, int s, int want_b) {
  const int B = A.P.B;
  const int lane = threadIdx.x & 63;
  // per-lane sequence data: rows in this row group, weight, split cap
  auto seq_data = [&](int b, long long &w, int &cap) {
    w = 0;
    cap = 0;
    if (b >= B) return;
    const Seq q = seq_of(A.P, b);
    const int rows = min(max(A.G * q.n - rg * A.rows_wg, 0), A.rows_wg);
    if (rows == 0) return;
    const int Tb = ctx_len(A, b, nullptr);
    // weights in twelfths of a tile
    w = (long long)((Tb + TILE - 1) / TILE + (q.n + TILE - 1) / TILE) * (12 + max(0, (rows + 15) / 16 - 9));
    cap = max(1, (Tb + 255) / 256);
  };
  long long W = 0;
  int m = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    long long w;
    int cap;
    seq_data(b0 + lane, w, cap);
    m += __popcll(__ballot(cap > 0));
    W += wave_sum_ll(w);
  }
  const long long E = A.n_splits > m ? A.n_splits - m : 0;
  int base = 0;
  long long Sb = 0;  // weights of the sequences before this chunk
  for (int b0 = 0; b0 < B; b0 += 64) {
    long long w;
    int cap;
    seq_data(b0 + lane, w, cap);
    const long long Si = Sb + wave_incl_scan_ll(w), Se = Si - w;
    const int nb = cap > 0 ? min(cap, 1 + (int)(W > 0 ? E * Si / W - E * Se / W : 0)) : 0;
    const int incl = wave_incl_scan(nb);
    const int first = base + incl - nb;
    if (want_b >= 0) {
      if (want_b < b0 + 64) {
        const int l = want_b - b0;
        return {want_b, 0, __shfl(nb, l), __shfl(first, l)};
      }
    } else {
      const unsigned long long hit = __ballot(nb > 0 && first <= s && s < first + nb);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        const int f = __shfl(first, l);
        return {b0 + l, s - f, __shfl(nb, l), f};
      }
    }
    base += __shfl(incl, 63);
    Sb = __shfl(Si, 63);
  }
  return {-1, 0, 0, 0};
}

// Registers of N 16-byte K chunks and N V chunks of a tile being filled.
template <int N_>
struct TileRegs {
  static constexpr int N = N_;
  uint4 k[N_];
  half8 v[N_];
};

template <int D>
struct Lds {
  // K stage: [32 rows][D] halves; row r = 16*tt + m holds the key that the
  // score MFMA of key-half tt reads as A-row m; the 16-byte chunk c of a row
  // sits at chunk position c ^ ksw(r).
  // V stage: [2 page halves][D channels][2 groups][8 keys] halves: group q
  // (keys 8q .. 8q + 7 of the tile) of channel d sits in half q >> 1, slot
  // (q & 1) ^ bit 3 of d (vslot).  Every 1 KB piece of a stage then lies in
  // one page half, so each direct load of a wave reads from one page.
  // Both swizzles give the 16 lanes that read one 16-byte slot each in a
  // matrix-core operand load 16 different bank groups.
  static constexpr int K_HALVES = TILE * D;
  static constexpr int V_HALVES = TILE * D;
  static constexpr int STAGE = K_HALVES + V_HALVES;
};
constexpr int NSTAGE = 4;  // LDS ring depth: NSTAGE - 1 tiles in flight

// Q8 path: the 8-bit tiles land in their own ring (K [32 tokens][D], V [2
// pages][D][16], then the tile's 32 K and 32 V scales), and one pass per
// tile, between two workgroup barriers, turns the next tile's K and this
// tile's V into the fp16 stage layout above, in one fp16 stage.
template <int D>
struct LdsQ8 {
  static constexpr int K_BYTES = TILE * D, V_BYTES = TILE * D, S_BYTES = 4 * TILE;
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES + S_BYTES;
  // 8-bit ring: 96 KB of tiles in flight, as many bytes as the fp16 ring
  // keeps in flight (6 tiles at D = 256, 12 at D = 128)
  static constexpr int Q_STAGES = 1 + (96 * 1024) / (K_BYTES + V_BYTES);
  // one fp16 stage: K of the next tile in its K half, V of this tile in its V half
  static constexpr int FP_BYTES = Lds<D>::STAGE * 2;
  static constexpr int TOTAL = FP_BYTES + Q_STAGES * STAGE_BYTES;
};

// K rows are whole bank periods (256 B) long, so rows r and r + 8 collide
// without the low four row bits in the swizzle; V channel rows are an eighth
// of a period, so channels d and d + 8 share banks unless bit 3 of d enters.
__device__ __forceinline__ int ksw(int r) { return r & 15; }
template <int D>
__device__ __forceinline__ int vslot(int d, int q) {
  return (q >> 1) * (16 * D) + d * 16 + 8 * ((q & 1) ^ ((d >> 3) & 1));
}

// tile-local key tau (0..31) <-> K row in LDS
__device__ __forceinline__ int krow_of(int tau) {
  return 16 * ((tau >> 2) & 1) + 4 * (tau >> 3) + (tau & 3);
}
__device__ __forceinline__ int key_of_krow(int r) {
  const int tt = r >> 4, m = r & 15;
  return 8 * (m >> 2) + 4 * tt + (m & 3);
}

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier of the K/V ring: this wave's LDS and scalar-memory
// operations are complete (lgkmcnt(0)) and its direct-to-LDS tile loads are
// left in flight, since every wave has already waited for exactly the tile
// it needs (wait_tiles) before it arrives.  __syncthreads() would also drain
// every vector-memory load (the compiler puts vmcnt(0) before its barrier,
// because direct-to-LDS loads write LDS), which empties the ring at every
// tile and leaves one tile of lookahead instead of NSTAGE - 1.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most `later` tiles' direct loads (LPT per tile and wave) are
// outstanding, later in [0, L]: s_waitcnt takes an immediate, so one case
// per count, the deepest first.
template <int LPT, int L>
__device__ __forceinline__ void wait_vm_tiles(int later) {
  if constexpr (L > 0) {
    if (later >= L) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L * LPT) : "memory");
      return;
    }
    wait_vm_tiles<LPT, L - 1>(later);
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// POOL: the batch's sequences share the splits of a (KV head, row group)
// (pool_slot); otherwise the grid's z runs over sequences and row groups and
// every sequence has A.n_splits splits.
template <int D, int NB, bool Q8, bool POOL>
__global__ __launch_bounds__(256, 1) void attn_mfma_kernel(AttnArgs A) {
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int WAVE_CH = (TILE * CPR) / 256;  // direct loads per wave, per tensor and tile
  // direct loads per wave and tile: fp16 K and V; or 8-bit K and V (1 KB
  // pieces, D / 128 each per wave) plus one load of the tile's scales
  constexpr int LPT = Q8 ? 2 * (D / 128) + 1 : 2 * WAVE_CH;
  constexpr int KS = D / 32;               // k-steps of the score product
  constexpr int DB = D / 16;               // channel blocks of the value product
  extern __shared__ half8 lds_raw[];
  _Float16 *lds = reinterpret_cast<_Float16 *>(lds_raw);

  const int g = blockIdx.y;
  int b, rg, split, nbs;
  if constexpr (POOL) {
    rg = blockIdx.z;
    const PoolSlot ps = pool_slot(A, rg, blockIdx.x, -1);
    if (ps.b < 0) return;
    b = ps.b, split = ps.j, nbs = ps.nb;
  } else {
    b = blockIdx.z / A.n_rg, rg = blockIdx.z % A.n_rg, split = blockIdx.x, nbs = A.n_splits;
  }
  const Seq s = seq_of(A.P, b);
  const int rows_b = A.G * s.n;
  const int row0 = rg * A.rows_wg;
  if (row0 >= rows_b) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;

  // ---- resident Q fragments and per-row tree masks.  Rows past the
  // sequence's rows (padding of the last row block) load the last real row:
  // their results are never written out, and with every load unconditional
  // the compiler can count the loads in flight (a guarded load makes it wait
  // for all of them before the first matrix instruction).
  half8 qf[NB][KS];
  unsigned long long ancr[NB];
  bool blk_on[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int blk0 = row0 + 16 * (w + 4 * j);
    blk_on[j] = blk0 < rows_b;
    const int rho = min(blk0 + l16, rows_b - 1);
    const int node = rho / A.G;
    const int hq = g * A.G + rho % A.G;
    ancr[j] = A.P.anc[s.o + node];
    const _Float16 *qp = A.q + ((size_t)(s.o + node) * A.Hq + hq) * D + 8 * lq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[j][ks] = *reinterpret_cast<const half8 *>(qp + 32 * ks);
  }

  // ---- the split's keys: these need the committed length, read while the
  // Q fragments are on their way
  bool cut;
  const int Tb = ctx_len(A, b, &cut);
  const int nsp = n_active_splits(Tb, nbs);
  if (split >= nsp) return;
  if (cut && split == 0 && g == 0 && rg == 0 && threadIdx.x == 0) A.P.status[b] |= DDT_ST_CTX;
  const int chunk = split_chunk(Tb, nbs);
  const int t_beg = split * chunk;
  const int t_end = min(Tb, t_beg + chunk);
  const int n_keys = t_end > t_beg ? t_end - t_beg : 0;
  const int n_full = n_keys / TILE;                      // direct-load tiles
  const bool has_part = (n_keys % TILE) != 0;            // ragged last cache tile
  const int n_tree = (split == nsp - 1) ? (s.n + TILE - 1) / TILE : 0;

  f32x4 o[NB][DB];
  float mrow[NB], mseen[NB], lsum[NB];
  bool ovf = false;
#pragma unroll
  for (int j = 0; j < NB; ++j) mrow[j] = -INFINITY;

  auto page_of = [&](int t) -> int {
    return A.pt ? A.pt[(size_t)b * A.max_pages + (t >> 4)] : (t >> 4);
  };
  const size_t kv_head = (size_t)g;
  // pages of the two halves of full tile it (read ahead of the barrier that
  // precedes the tile's issue, so the barrier's own wait covers the read)
  auto tile_page = [&](int it, int half) { return page_uniform(A, b, t_beg + it * TILE + 16 * half); };

  // ---- full cache tile -> LDS stage, straight from HBM (global_load_lds).
  // Wave w fills 1 KB pieces w, w+4, ...; lane l of a piece lands at byte
  // 16*l, so each lane fetches whichever chunk belongs there.  A piece lies
  // in one page (the K rows of a piece are keys of one page half, and V
  // pieces are laid out by page half), so a load's address is the page's
  // base, the same for the whole wave, plus a lane offset that every tile
  // shares: khalf / vhalf say which page, koff / voff the offsets in halves.
  int koff[WAVE_CH], voff[WAVE_CH];
  bool khalf[WAVE_CH], vhalf[WAVE_CH];
#pragma unroll
  for (int k = 0; k < WAVE_CH; ++k) {
    const int piece = w + 4 * k;
    const int P = piece * 64 + lane;       // chunk position in the stage
    const int r = P / CPR, cpos = P % CPR;  // K row and chunk slot
    const int tau = key_of_krow(r);
    khalf[k] = __builtin_amdgcn_readfirstlane(tau >> 4);
    koff[k] = (tau & 15) * D + 8 * (cpos ^ ksw(r));
    constexpr int PPH = D / 32;  // V pieces per page half
    const int Pv = (piece % PPH) * 64 + lane;
    const int d = Pv >> 1, q1 = (Pv & 1) ^ ((d >> 3) & 1);
    vhalf[k] = piece >= PPH;
    voff[k] = d * DDT_PAGE + 8 * q1;
  }
  auto issue_tile = [&](int stage, int pg0, int pg1) {
    _Float16 *Ks = lds + stage * Lds<D>::STAGE;
    _Float16 *Vs = Ks + Lds<D>::K_HALVES;
    const _Float16 *kb0 = A.Kc + ((size_t)pg0 * A.Hkv + kv_head) * DDT_PAGE * D;
    const _Float16 *kb1 = A.Kc + ((size_t)pg1 * A.Hkv + kv_head) * DDT_PAGE * D;
    const _Float16 *vb0 = A.Vc + ((size_t)pg0 * A.Hkv + kv_head) * D * DDT_PAGE;
    const _Float16 *vb1 = A.Vc + ((size_t)pg1 * A.Hkv + kv_head) * D * DDT_PAGE;
#pragma unroll
    for (int k = 0; k < WAVE_CH; ++k)
      __builtin_amdgcn_global_load_lds((const void *)((khalf[k] ? kb1 : kb0) + koff[k]),
                                       (lds_void *)(Ks + (w + 4 * k) * 512), 16, 0, KV_STREAM_CPOL);
#pragma unroll
    for (int k = 0; k < WAVE_CH; ++k)
      __builtin_amdgcn_global_load_lds((const void *)((vhalf[k] ? vb1 : vb0) + voff[k]),
                                       (lds_void *)(Vs + (w + 4 * k) * 512), 16, 0, KV_STREAM_CPOL);
  };

  // ---- Q8: 8-bit tile -> its staging stage, straight from HBM.  A page of
  // one KV head is 16 * D contiguous bytes of K (token-major) and of V
  // (channel-major); the stage holds both pages of each back to back, so
  // wave w copies 1 KB pieces w, w + 4 of each, and then the 32-byte scale
  // run w (K page 0, K page 1, V page 0, V page 1) with eight lanes.
  char *const qbase = reinterpret_cast<char *>(lds) + (Q8 ? LdsQ8<D>::FP_BYTES : 0);
  auto issue_q8 = [&](int stage, int pg0, int pg1) {
    char *St = qbase + stage * LdsQ8<D>::STAGE_BYTES;
    constexpr int PPP = 16 * D / 1024;  // 1 KB pieces per page
#pragma unroll
    for (int k = 0; k < D / 128; ++k) {
      const int piece = w + 4 * k, half = piece / PPP, off = (piece % PPP) * 1024 + 16 * lane;
      const size_t pb = ((size_t)(half ? pg1 : pg0) * A.Hkv + kv_head) * 16 * D;
      __builtin_amdgcn_global_load_lds((const void *)(A.Kq + pb + off), (lds_void *)(St + piece * 1024), 16, 0, KV_STREAM_CPOL);
    }
#pragma unroll
    for (int k = 0; k < D / 128; ++k) {
      const int piece = w + 4 * k, half = piece / PPP, off = (piece % PPP) * 1024 + 16 * lane;
      const size_t pb = ((size_t)(half ? pg1 : pg0) * A.Hkv + kv_head) * 16 * D;
      __builtin_amdgcn_global_load_lds((const void *)(A.Vq + pb + off),
                                       (lds_void *)(St + LdsQ8<D>::K_BYTES + piece * 1024), 16, 0, KV_STREAM_CPOL);
    }
    const _Float16 *sc = (w < 2 ? A.Ksc : A.Vsc) + ((size_t)((w & 1) ? pg1 : pg0) * A.Hkv + kv_head) * 16;
    if (lane < 8)
      __builtin_amdgcn_global_load_lds((const void *)(sc + 2 * lane),
                                       (lds_void *)(St + LdsQ8<D>::K_BYTES + LdsQ8<D>::V_BYTES + 32 * w), 4, 0, 0);
  };
  // Q8: one pass turns a staged 8-bit tile into the fp16 stage layout (the
  // same rows, chunks and swizzles as a direct fp16 tile).  A value is
  // fp16(q * scale): q becomes fp16 exactly (0x6400 | (q + 128) is 1024 + q
  // + 128), and the product is rounded once, by the fp16 multiply.
  // Q8: a staged 8-bit tile's K (conv_k) or V (conv_v) -> the fp16 stage, in
  // the same rows, chunks and swizzles as a direct fp16 tile.  A value is
  // fp16(q * scale): q becomes fp16 exactly (0x6400 | (q + 128) is 1024 + q
  // + 128), and the product is rounded once, by the fp16 multiply.  Codes
  // are read as a vector type (not HIP's uint2): the compiler then leaves the
  // ring's direct-to-LDS loads in flight across the read.
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  auto dq8 = [](u32x2 q, half8 sc8) -> half8 {
    const unsigned x0 = q.x ^ 0x80808080u, x1 = q.y ^ 0x80808080u;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 hb = {__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u),
                      __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u),
                      __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u),
                      __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)};
    const half8 v = __builtin_bit_cast(half8, hb) - (half8)(_Float16)1152.0f;
    return v * sc8;
  };
  auto conv_k = [&](int qstage) {
    const char *St = qbase + qstage * LdsQ8<D>::STAGE_BYTES;
    const _Float16 *Sc = reinterpret_cast<const _Float16 *>(St + LdsQ8<D>::K_BYTES + LdsQ8<D>::V_BYTES);
#pragma unroll
    for (int k = 0; k < (TILE * CPR) / 256; ++k) {  // token tau, chunk cc
      const int idx = threadIdx.x + 256 * k, tau = idx / CPR, cc = idx % CPR;
      const u32x2 q = *reinterpret_cast<const u32x2 *>(St + tau * D + 8 * cc);
      const half8 v = dq8(q, (half8)Sc[tau]);
      const int r = krow_of(tau);
      *reinterpret_cast<half8 *>(lds + r * D + 8 * (cc ^ ksw(r))) = v;
    }
  };
  // V: thread idx writes slot idx & 1 of channel d of page half h, in the
  // order of the fp16 stage (a 16-lane phase writes 256 contiguous bytes);
  // the slot holds group q1 = slot ^ bit 3 of d, keys 8 q1 .. 8 q1 + 7
  auto conv_v = [&](int qstage) {
    const char *St = qbase + qstage * LdsQ8<D>::STAGE_BYTES;
    const _Float16 *Sc = reinterpret_cast<const _Float16 *>(St + LdsQ8<D>::K_BYTES + LdsQ8<D>::V_BYTES);
    _Float16 *Vf = lds + Lds<D>::K_HALVES;
#pragma unroll
    for (int k = 0; k < (4 * D) / 256; ++k) {
      const int idx = threadIdx.x + 256 * k, h = idx / (2 * D), d = (idx >> 1) % D;
      const int q1 = (idx & 1) ^ ((d >> 3) & 1), qg = 2 * h + q1;
      const u32x2 q = *reinterpret_cast<const u32x2 *>(St + LdsQ8<D>::K_BYTES + h * 16 * D + 16 * d + 8 * q1);
      const half8 sv = *reinterpret_cast<const half8 *>(Sc + TILE + 8 * qg);
      *reinterpret_cast<half8 *>(Vf + vslot<D>(d, qg)) = dq8(q, sv);
    }
  };

  // wait until at most `later` tiles' direct loads are outstanding (each
  // tile is LPT loads per wave); the counts are immediates
  auto wait_tiles = [&](int later) {
    static_assert(NSTAGE <= 5, "wait_tiles covers up to three later tiles");
    if (later >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LPT) : "memory");
    else if (later == 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPT) : "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPT) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // ---- a tree tile -> LDS stage through registers, zero-filling keys past
  // the tree.  Thread tid fills K chunks and V chunks tid + 256 u, each one
  // 16-byte slot of the stage: K chunk ci = key tau's channels 8 cc ..
  // 8 cc + 7 (tau = ci / CPR), V chunk ci = keys 8 qg .. 8 qg + 7 of channel
  // d (d = ci / 4, qg = ci % 4), so every LDS store is a whole slot on its
  // own banks.  Every load (at clamped addresses, so none is conditional)
  // is issued before the first store: a tile costs one memory round trip.
  constexpr int CPT = TILE * CPR / 256;  // K (and V) chunks per thread and tile
  static_assert(TILE * CPR == 4 * D, "as many V chunks as K chunks");
  auto load_tree_tile = [&](int kbase, int h, auto &R) {
    constexpr int HPT = std::remove_reference_t<decltype(R)>::N;
    const int nlast = s.n > 0 ? s.n - 1 : 0;
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
      const int ci = tid + 256 * (h * HPT + u);
      const int tau = ci / CPR, cc = ci % CPR;
      const int key = kbase + tau;
      const uint4 kx = *reinterpret_cast<const uint4 *>(
          A.Kt + ((size_t)(s.o + min(key, nlast)) * A.Hkv + kv_head) * D + 8 * cc);
      R.k[u] = key < s.n ? kx : make_uint4(0, 0, 0, 0);
      const int d = ci >> 2, k0 = kbase + 8 * (ci & 3);
      half8 vx;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vx[e] = A.Vt[((size_t)(s.o + min(k0 + e, nlast)) * A.Hkv + kv_head) * D + d];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k0 + e >= s.n) vx[e] = (_Float16)0.0f;
      R.v[u] = vx;
    }
  };
  auto store_tile = [&](const auto &R, int h, int stage) {
    constexpr int HPT = std::remove_reference_t<decltype(R)>::N;
    _Float16 *Ks = lds + stage * Lds<D>::STAGE;
    _Float16 *Vs = Ks + Lds<D>::K_HALVES;
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
      const int ci = tid + 256 * (h * HPT + u);
      const int tau = ci / CPR, cc = ci % CPR;
      const int r = krow_of(tau);
      *reinterpret_cast<uint4 *>(Ks + r * D + 8 * (cc ^ ksw(r))) = R.k[u];
      const int d = ci >> 2, qg = ci & 3;
      *reinterpret_cast<half8 *>(Vs + vslot<D>(d, qg)) = R.v[u];
    }
  };
  // a whole tree tile in one pass (one memory round trip)
  auto fill_tree_tile = [&](int kbase, int stage) {
    TileRegs<CPT> R;
    load_tree_tile(kbase, 0, R);
    store_tile(R, 0, stage);
  };
  // The epilogue's fill (a ragged cache tile, a second tree tile, or the
  // 8-bit path's tree tile), with the accumulators live: one chunk at a time.
  auto fill_tile_rolled = [&](bool tree, int kbase, int stage) {
    _Float16 *Ks = lds + stage * Lds<D>::STAGE;
    _Float16 *Vs = Ks + Lds<D>::K_HALVES;
    for (int ci = tid; ci < TILE * CPR; ci += 256) {
      const int tau = ci / CPR, cc = ci % CPR;
      const int key = kbase + tau;
      uint4 kx = make_uint4(0, 0, 0, 0);
      half8 vx = half8{0, 0, 0, 0, 0, 0, 0, 0};
      if (tree) {
        if (key < s.n) {
          const size_t src = ((size_t)(s.o + key) * A.Hkv + kv_head) * D + 8 * cc;
          kx = *reinterpret_cast<const uint4 *>(A.Kt + src);
          vx = *reinterpret_cast<const half8 *>(A.Vt + src);
        }
      } else if (key < t_end) {
        const size_t pg = (size_t)page_of(key) * A.Hkv + kv_head;
        if constexpr (Q8) {  // fp16(q * scale), the product rounded once
          const float ks = (float)A.Ksc[pg * DDT_PAGE + (key & 15)], vs = (float)A.Vsc[pg * DDT_PAGE + (key & 15)];
          const int8_t *kq = A.Kq + (pg * DDT_PAGE + (key & 15)) * D + 8 * cc;
          half8 kh;
#pragma unroll
          for (int x = 0; x < 8; ++x) kh[x] = (_Float16)((float)kq[x] * ks);
          kx = __builtin_bit_cast(uint4, kh);
#pragma unroll
          for (int x = 0; x < 8; ++x)
            vx[x] = (_Float16)((float)A.Vq[(pg * D + 8 * cc + x) * DDT_PAGE + (key & 15)] * vs);
        } else {
          kx = *reinterpret_cast<const uint4 *>(A.Kc + (pg * DDT_PAGE + (key & 15)) * D + 8 * cc);
#pragma unroll
          for (int x = 0; x < 8; ++x) vx[x] = A.Vc[(pg * D + 8 * cc + x) * DDT_PAGE + (key & 15)];
        }
      }
      const int r = krow_of(tau);
      *reinterpret_cast<uint4 *>(Ks + r * D + 8 * (cc ^ ksw(r))) = kx;
      const int qg = tau >> 3, e = tau & 7;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int d = 8 * cc + x;
        Vs[vslot<D>(d, qg) + e] = vx[x];
      }
    }
  };
  // fp16 cache: the split that takes the tree stages its first tree tile in
  // the spare LDS stage now, before the loop; the epilogue computes on it
  // directly (the 8-bit path has no spare stage and fills it afterwards).
  constexpr int TREE_STAGE = NSTAGE;
  if constexpr (!Q8) {
    if (n_tree > 0) fill_tree_tile(0, TREE_STAGE);
  }
  // Every load so far (the Q fragments, issued together with the read of
  // the committed length) is complete before the first tiles go out: the
  // compiler then sees no load pending on a register when the first matrix
  // instruction runs and leaves the tiles in flight (vmcnt(0) only).
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- scores of one 32-key tile: S^T = K Q^T (two 16-key halves)
  auto qk = [&](int stage, f32x4 (&S)[2][NB]) {
    const _Float16 *Ks = lds + stage * Lds<D>::STAGE;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < NB; ++j) S[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int r = 16 * tt + l16;
        const int cc = 4 * ks + lq;
        const half8 kf = *reinterpret_cast<const half8 *>(Ks + r * D + 8 * (cc ^ ksw(r)));
#pragma unroll
        for (int j = 0; j < NB; ++j)
          S[tt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[j][ks], S[tt][j], 0, 0, 0);
      }
    }
  };

  // ---- probabilities of one tile against each row's reference max.
  // This lane holds keys kbase + 8*lq + e (e = 4*tt + i) of row l16.
  // mask = 1: ragged cache tile; 2: tree tile.  Row blocks past the
  // sequence's rows compute harmless values that are never written out.
  auto softmax = [&](const f32x4 (&S)[2][NB], int mask, int kbase, half8 (&pf)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      float sv[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kbase + 8 * lq + e;
        const bool valid = mask == 2 ? (key < s.n && ((ancr[j] >> key) & 1ull)) : (key < t_end);
        sv[e] = valid ? S[e >> 2][j][e & 3] : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      if (__ballot(mrow[j] == -INFINITY)) {
        // a row's first tile with valid keys fixes its reference max
        float mloc = fmaxf(tmax, __shfl_xor(tmax, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        if (mrow[j] == -INFINITY) mrow[j] = mloc;
      }
      mseen[j] = fmaxf(mseen[j], tmax);
      ovf |= (tmax - mrow[j]) * A.c > 15.0f;  // fp16 P keeps 15 binades above 1
      const float mc = mrow[j] == -INFINITY ? 0.f : mrow[j] * A.c;
      float p[8], ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], A.c, -mc));  // masked keys: exp2(-inf) = 0
        ps += p[e];
      }
      lsum[j] += ps;
      pf[j] = half8{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                    (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
    }
  };
  // full cache tile, every reference already fixed: no masks, no branches
  auto softmax_blk = [&](const f32x4 (&S)[2][NB], int j, half8 &pfj) {
    float sv[8], p[8], ps = 0.f, tmax = -INFINITY;
    const float mc = mrow[j] * A.c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = S[e >> 2][j][e & 3];
      tmax = fmaxf(tmax, sv[e]);
      p[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], A.c, -mc));
      ps += p[e];
    }
    mseen[j] = fmaxf(mseen[j], tmax);
    ovf |= (tmax - mrow[j]) * A.c > 15.0f;
    lsum[j] += ps;
    pfj = half8{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
  };
  // K fragment (tile stage, key half tt, k-step ks) and V fragment (channel block n)
  auto kfrag = [&](const _Float16 *Ks, int tt, int ks) -> half8 {
    const int r = 16 * tt + l16;
    const int cc = 4 * ks + lq;
    return *reinterpret_cast<const half8 *>(Ks + r * D + 8 * (cc ^ ksw(r)));
  };
  auto vfrag = [&](const _Float16 *Vs, int n) -> half8 {
    const int d = 16 * n + l16;
    return *reinterpret_cast<const half8 *>(Vs + vslot<D>(d, lq));
  };
  // The 8-bit path's tile step: the same work in batches, no loads (the
  // fp16 path's step below measured slower here, behind the conversion pass
  // and its second barrier).  Scores of the next tile (Ks1) while the
  // probabilities and value product of this tile (S, Vs0) are formed, for
  // the first NBA row blocks of this wave (the others are padding past the
  // sequence's rows and are skipped).  sched_barrier fences keep each batch
  // of LDS reads one batch ahead of the MFMAs that consume it and put the
  // softmax next to the score MFMAs.
  auto tile_step_ahead = [&](auto NBA_c, const _Float16 *Ks1, const _Float16 *Vs0, const f32x4 (&S)[2][NB],
                             f32x4 (&Sn)[2][NB]) {
    constexpr int NBA = decltype(NBA_c)::value;
    constexpr int KH = KS / 2;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < NBA; ++j) Sn[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    half8 ka[2][KH], kb[2][KH], pf[NB];
    if constexpr (NBA > 0) {
#pragma unroll
      for (int ks = 0; ks < KH; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) ka[tt][ks] = kfrag(Ks1, tt, ks);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NBA > 0) {
#pragma unroll
      for (int ks = 0; ks < KH; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) kb[tt][ks] = kfrag(Ks1, tt, KH + ks);
#pragma unroll
      for (int ks = 0; ks < KH; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < NBA; ++j)
            Sn[tt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[tt][ks], qf[j][ks], Sn[tt][j], 0, 0, 0);
      softmax_blk(S, 0, pf[0]);
      __builtin_amdgcn_sched_barrier(0);
      constexpr int VH = DB / 2;
      half8 va[VH], vb[VH];
#pragma unroll
      for (int n = 0; n < VH; ++n) va[n] = vfrag(Vs0, n);
#pragma unroll
      for (int ks = 0; ks < KH; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < NBA; ++j)
            Sn[tt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[tt][ks], qf[j][KH + ks], Sn[tt][j], 0, 0, 0);
#pragma unroll
      for (int j = 1; j < NBA; ++j) softmax_blk(S, j, pf[j]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < VH; ++n) vb[n] = vfrag(Vs0, VH + n);
#pragma unroll
      for (int n = 0; n < VH; ++n)
#pragma unroll
        for (int j = 0; j < NBA; ++j)
          o[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[n], pf[j], o[j][n], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < VH; ++n)
#pragma unroll
        for (int j = 0; j < NBA; ++j)
          o[j][VH + n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vb[n], pf[j], o[j][VH + n], 0, 0, 0);
    }
  };

  // One full tile of the main loop: scores of the next tile (Ks1) while the
  // probabilities and value product of this tile (S, Vs0) are formed, for
  // the first NBA row blocks of this wave (the others are padding past the
  // sequence's rows and are skipped).  With one wavefront per SIMD, a VALU
  // instruction runs in the shadow of the matrix pipe only when it sits
  // between two MFMAs, a few per MFMA; so the VALU work is spread over all
  // of them: the score MFMAs carry the tile's loads (`issue`, straight-line
  // code) and block 0's probabilities, and block j's value product carries
  // block j + 1's probabilities (sched_group_barrier pairs each MFMA with a
  // few other instructions).
  auto tile_step = [&](auto NBA_c, const _Float16 *Ks1, const _Float16 *Vs0, const f32x4 (&S)[2][NB],
                       f32x4 (&Sn)[2][NB], auto &&issue) {
    constexpr int NBA = decltype(NBA_c)::value;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < NBA; ++j) Sn[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NBA == 0) {
      issue();
    } else {
      half8 kf[2][KS], pf[NB];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) kf[tt][ks] = kfrag(Ks1, tt, ks);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < NBA; ++j)
            Sn[tt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[tt][ks], qf[j][ks], Sn[tt][j], 0, 0, 0);
      issue();
      softmax_blk(S, 0, pf[0]);
#pragma unroll
      for (int i = 0; i < 2 * KS * NBA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x416, 3, 0);  // VALU, SALU, VMEM, transcendental
      }
      __builtin_amdgcn_sched_barrier(0);
      half8 vf[DB];
#pragma unroll
      for (int n = 0; n < DB; ++n) vf[n] = vfrag(Vs0, n);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NBA; ++j) {
#pragma unroll
        for (int n = 0; n < DB; ++n)
          o[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[n], pf[j], o[j][n], 0, 0, 0);
        if (j + 1 < NBA) {
          softmax_blk(S, j + 1, pf[j + 1]);
#pragma unroll
          for (int n = 0; n < DB; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x406, 4, 1);  // VALU, SALU, transcendental
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- O^T += V^T P^T for one tile
  auto pv = [&](int stage, const half8 (&pf)[NB]) {
    const _Float16 *Vs = lds + stage * Lds<D>::STAGE + Lds<D>::K_HALVES;
#pragma unroll
    for (int n = 0; n < DB; ++n) {
      const int d = 16 * n + l16;
      const half8 vf = *reinterpret_cast<const half8 *>(Vs + vslot<D>(d, lq));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        o[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[j], o[j][n], 0, 0, 0);
    }
  };

  // The split normally runs once.  If some score exceeded its row's
  // reference by more than fp16 P can hold, it runs again with every
  // reference set to the true maximum seen, which cannot overflow.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      mseen[j] = -INFINITY;
      lsum[j] = 0.f;
#pragma unroll
      for (int n = 0; n < DB; ++n) o[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // ---- main loop over full tiles: NSTAGE-stage LDS ring with up to
    // NSTAGE - 1 tiles in flight; the scores of tile it+1 are formed while the
    // probabilities and value product of tile it are worked on.
    if (n_full > 0) {
      // row blocks are dealt round-robin, so a wave's active blocks are a
      // prefix of its NB and number NB or NB - 1
      f32x4 Sn[2][NB];
      auto fix_refs = [&]() {  // the first full tile fixes every row's reference max (pass 0 only)
        if (__ballot(mrow[0] == -INFINITY)) {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            float t = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) t = fmaxf(t, Sn[e >> 2][j][e & 3]);
            t = fmaxf(t, __shfl_xor(t, 16));
            mrow[j] = fmaxf(t, __shfl_xor(t, 32));
          }
        }
      };
      auto copy_S = [&](f32x4 (&Sc)[2][NB]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < NB; ++j) Sc[tt][j] = Sn[tt][j];
      };
      if constexpr (!Q8) {
        // the first NSTAGE - 1 tiles, all issued: a split with fewer tiles
        // reads its last tile again into stages it never uses, so that the
        // number of loads in flight is fixed and the first wait can leave
        // them all but tile 0 outstanding
#pragma unroll
        for (int t = 0; t < NSTAGE - 1; ++t) {
          const int tc = min(t, n_full - 1);
          issue_tile(t, tile_page(tc, 0), tile_page(tc, 1));
        }
        // wait for tile 0: the loads of the later tiles may stay outstanding
        wait_tiles(NSTAGE - 2);
        ring_barrier();
        qk(0, Sn);
        fix_refs();
        auto main_loop = [&](auto NBA_c) {
          // while tiles are left to issue: one goes out per iteration, and
          // exactly one more is in flight behind tile it + 1
          int it = 0;
          for (; it + NSTAGE - 1 < n_full; ++it) {
            const int nt = it + NSTAGE - 1;  // tile issued in this iteration
            const int npg0 = tile_page(nt, 0), npg1 = tile_page(nt, 1);
            wait_tiles(NSTAGE - 3);  // tile it + 1 landed
            ring_barrier();  // ... for every wave; every wave is past tile it - 1
            f32x4 Sc[2][NB];
            copy_S(Sc);
            tile_step(NBA_c, lds + ((it + 1) % NSTAGE) * Lds<D>::STAGE,
                      lds + (it % NSTAGE) * Lds<D>::STAGE + Lds<D>::K_HALVES, Sc, Sn,
                      [&]() { issue_tile(nt % NSTAGE, npg0, npg1); });
          }
          // the last tiles: nothing left to issue (past the last tile the
          // scores read a stale stage and are dropped)
          for (; it < n_full; ++it) {
            if (it + 1 < n_full) wait_tiles(n_full - it - 2);
            ring_barrier();
            f32x4 Sc[2][NB];
            copy_S(Sc);
            tile_step(NBA_c, lds + ((it + 1) % NSTAGE) * Lds<D>::STAGE,
                      lds + (it % NSTAGE) * Lds<D>::STAGE + Lds<D>::K_HALVES, Sc, Sn, [&]() {});
          }
        };
        if (blk_on[NB - 1])
          main_loop(std::integral_constant<int, NB>{});
        else
          main_loop(std::integral_constant<int, NB - 1>{});
      } else {
        // K of tile t is converted in iteration t - 1 and its V in
        // iteration t, so a tile's 8-bit stage is free once iteration t has
        // passed its first barrier; up to QS - 2 tiles are in flight behind
        // the one converted next
        constexpr int QS = LdsQ8<D>::Q_STAGES;
        auto wait_q8 = [&](int later) { wait_vm_tiles<LPT, QS - 2>(later); };
#pragma unroll
        for (int t = 0; t < QS - 1; ++t)
          if (t < n_full) issue_q8(t, tile_page(t, 0), tile_page(t, 1));
        wait_q8(min(n_full, QS - 1) - 1);  // tile 0 landed
        ring_barrier();
        conv_k(0);
        ring_barrier();
        qk(0, Sn);
        fix_refs();
        auto main_loop = [&](auto NBA_c) {
          for (int it = 0; it < n_full; ++it) {
            const int nt = it + QS - 1;  // 8-bit tile issued in this iteration
            const int npg0 = nt < n_full ? tile_page(nt, 0) : 0, npg1 = nt < n_full ? tile_page(nt, 1) : 0;
            if (it + 1 < n_full) wait_q8(min(n_full, it + QS - 1) - (it + 2));  // tile it + 1 landed
            ring_barrier();  // ... for every wave; every wave is past tile it - 1
            // the next 8-bit tile goes out first, into the stage of tile
            // it - 1 (its V was converted in the last iteration)
            if (nt < n_full) issue_q8(nt % QS, npg0, npg1);
            if (it + 1 < n_full) conv_k((it + 1) % QS);
            conv_v(it % QS);
            ring_barrier();
            f32x4 Sc[2][NB];
            copy_S(Sc);
            tile_step_ahead(NBA_c, lds, lds + Lds<D>::K_HALVES, Sc, Sn);
          }
        };
        if (blk_on[NB - 1])
          main_loop(std::integral_constant<int, NB>{});
        else
          main_loop(std::integral_constant<int, NB - 1>{});
      }
    }
    // ---- epilogue: ragged cache tile, then the tree tiles
    const int n_ep = (has_part ? 1 : 0) + n_tree;
    for (int e = 0; e < n_ep; ++e) {
      const bool tree = !(has_part && e == 0);
      const int kbase = tree ? (e - (has_part ? 1 : 0)) * TILE : t_beg + n_full * TILE;
      const int stage = (!Q8 && tree && kbase == 0) ? TREE_STAGE : 0;
      __syncthreads();  // the stage is no longer read
      if (stage == 0) fill_tile_rolled(tree, kbase, 0);
      __syncthreads();
      f32x4 S[2][NB];
      half8 pf[NB];
      qk(stage, S);
      softmax(S, tree ? 2 : 1, kbase, pf);
      pv(stage, pf);
    }
    // any overflow in the workgroup?  The flags go through the first ring
    // stage, idle by now (a block-wide vote would take static LDS, and the
    // ring fills all of it)
    __syncthreads();  // every wave is done reading the ring
    int *flag = reinterpret_cast<int *>(lds);
    const bool wave_ovf = __ballot(ovf) != 0ull;  // every lane votes, outside the branch
    if (lane == 0) flag[w] = wave_ovf;
    __syncthreads();
    const bool redo = (flag[0] | flag[1] | flag[2] | flag[3]) != 0;
    __syncthreads();  // flags read before the ring is refilled
    if (!redo) break;
    ovf = false;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      float m = fmaxf(mseen[j], __shfl_xor(mseen[j], 16));
      mrow[j] = fmaxf(m, __shfl_xor(m, 32));
    }
  }

  // ---- partial results of this split
  const size_t base =
      POOL ? (((size_t)g * A.n_rg + rg) * A.n_splits + blockIdx.x) * A.rows_wg
           : (((size_t)(b * A.Hkv + g) * A.n_rg + rg) * A.n_splits + split) * A.rows_wg;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (!blk_on[j]) continue;
    float l = lsum[j];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int rl = 16 * (w + 4 * j) + l16;  // row within the workgroup
    if (row0 + rl >= rows_b) continue;
    if (lq == 0) A.ML[base + rl] = make_float2(mrow[j], l);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    _Float16 *op = A.Opart + (base + rl) * D + 4 * lq;
#pragma unroll
    for (int n = 0; n < DB; ++n)
      *reinterpret_cast<half4 *>(op + 16 * n) = half4{(_Float16)(o[j][n][0] * inv), (_Float16)(o[j][n][1] * inv),
                                                      (_Float16)(o[j][n][2] * inv), (_Float16)(o[j][n][3] * inv)};
  }
}

// Merge the splits of one query row: one workgroup per row.  Every thread
// first issues the loads of its share of the partial outputs (8 channels,
// one 16-byte load, x splits sg, sg + SG, ...; with 8-byte loads of 4
// channels the call measured ~1.5 us longer); meanwhile wavefront 0 turns the split maxima
// and sums into weights l_s 2^((m_s - M) c) (the partials are normalised by
// their own sums l_s) and their total L.  The weighted sums
// are then added in a fixed order, so the result does not depend on timing.
constexpr int MAX_SPLITS = 1024;

// The combine for a batch of one sequence (n1 nodes), whose splits are all
// its own: one workgroup per row.  The fields of A that the first loads need
// lead the arguments, which the library preloads into scalar registers at
// dispatch (14 dwords).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const _Float16 *__restrict__ a_Opart,
                                                           const float2 *__restrict__ a_ML,
                                                           const int32_t *__restrict__ a_T, const int32_t *a_pt,
                                                           int n1, int a_G, int a_rows_wg, int a_n_rg,
                                                           int a_n_splits, int a_T_max, AttnArgs A) {
  constexpr int TPR = D / 8;     // threads per channel sweep (8 channels, one 16-byte load each)
  constexpr int SG = 256 / TPR;  // split groups
  constexpr int BATCH = 64 / SG; // partial loads in flight per thread
  __shared__ float wts[MAX_SPLITS];
  __shared__ float Lsh;
  __shared__ float4 part[SG][TPR][2];
  A.Opart = const_cast<_Float16 *>(a_Opart);
  A.ML = const_cast<float2 *>(a_ML);
  A.T = a_T;
  A.pt = a_pt;
  A.G = a_G;
  A.rows_wg = a_rows_wg;
  A.n_rg = a_n_rg;
  A.n_splits = a_n_splits;
  A.T_max = a_T_max;
  const int rl = blockIdx.x, g = blockIdx.y, b = 0, rg = blockIdx.z;
  const Seq s{0, n1};
  const int rho = rg * A.rows_wg + rl;
  if (rho >= A.G * s.n) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const size_t base = (((size_t)g * A.n_rg + rg) * A.n_splits) * A.rows_wg + rl;
  const int nw = A.n_splits;
  const int dc = tid % TPR, sg = tid / TPR;
  const _Float16 *src = A.Opart + base * D + 8 * dc;
  const size_t sstride = (size_t)A.rows_wg * D;
  // Every load that depends on no other goes out first: the context length,
  // wave 0's split statistics and each thread's first BATCH partials.  Split
  // indices are clamped to the sequence's split count, which bounds the
  // active count; a split that turns out inactive is skipped after its load
  // and never multiplied, since its slot may hold anything.
  float2 ml0 = make_float2(-INFINITY, 0.f);
  if (tid < 64) ml0 = A.ML[base + (size_t)min(lane, nw - 1) * A.rows_wg];
  half8 v[BATCH];
#pragma unroll
  for (int t = 0; t < BATCH; ++t) v[t] = *reinterpret_cast<const half8 *>(src + min(sg + t * SG, nw - 1) * sstride);
  // the context length is read after the partials are requested (left to
  // itself the scheduler clamps it first and so waits for it before them);
  // the arguments not preloaded are fetched in the same round
  __builtin_amdgcn_sched_barrier(0);
  const int nsp = n_active_splits(ctx_len(A, b, nullptr), nw);
  asm volatile("" ::"s"(A.c), "s"(A.out), "s"(A.Hq));
  if (tid < 64) {
    float m = lane < nsp ? fmaxf(-INFINITY, ml0.x) : -INFINITY;
    for (int sp = lane + 64; sp < nsp; sp += 64) m = fmaxf(m, A.ML[base + (size_t)sp * A.rows_wg].x);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float l = 0.f;
    for (int sp = lane; sp < nsp; sp += 64) {
      const float2 ml = sp == lane ? ml0 : A.ML[base + (size_t)sp * A.rows_wg];
      const float wgt = (ml.x == -INFINITY) ? 0.f : ml.y * exp2f((ml.x - m) * A.c);
      wts[sp] = wgt;
      l += wgt;
    }
    // fixed-order total: lane partials gathered in lane order
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_down(l, o);
      if ((lane & (2 * o - 1)) == 0) l += t;
    }
    if (lane == 0) Lsh = l;
  }
  __syncthreads();
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < BATCH; ++t) {
    const int sp = sg + t * SG;
    if (sp < nsp) {
      const float wgt = wts[sp];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf((float)v[t][e], wgt, acc[e]);
    }
  }
  for (int sp = sg + BATCH * SG; sp < nsp; sp += SG) {
    const float wgt = wts[sp];
    const half8 x = *reinterpret_cast<const half8 *>(src + sp * sstride);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf((float)x[e], wgt, acc[e]);
  }
  part[sg][dc][0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  part[sg][dc][1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  if (sg == 0) {
    for (int k = 1; k < SG; ++k) {
      const float4 x0 = part[k][dc][0], x1 = part[k][dc][1];
      acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
      acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
    }
    const float inv = 1.f / Lsh;
    const int node = rho / A.G, hq = g * A.G + rho % A.G;
    float4 *dst = reinterpret_cast<float4 *>(A.out + ((size_t)(s.o + node) * A.Hq + hq) * D + 8 * dc);
    dst[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    dst[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
}

// The combine for a batch sharing pooled splits: one wavefront per row,
// four rows of one sequence per workgroup.  A sequence has a few splits
// each (its share of the pool), so a whole workgroup per row, as above,
// would mostly wait; here each wave computes the sequence's deal, its
// splits' weights (lane sp holds split sp, 64 at a time, then LDS makes
// them visible to the whole wave) and its row's channels, CPL per lane,
// with every partial load of a batch of 16 splits issued before any is
// used.  Same fixed merge order as above, so results are deterministic.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_rows_kernel(AttnArgs A) {
  constexpr int CPL = D / 64;  // channels per lane
  constexpr int BATCH = 16;
  typedef _Float16 hcpl __attribute__((ext_vector_type(CPL)));
  __shared__ float wts[4][MAX_SPLITS];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = blockIdx.y, b = blockIdx.z / A.n_rg, rg = blockIdx.z % A.n_rg;
  const int rl = 4 * blockIdx.x + wv;
  const Seq s = seq_of(A.P, b);
  const int rho = rg * A.rows_wg + rl;
  if (rl >= A.rows_wg || rho >= A.G * s.n) return;  // the same in every lane of the wave
  const PoolSlot ps = pool_slot(A, rg, 0, b);        // the sequence's pool splits
  const size_t base = (((size_t)g * A.n_rg + rg) * A.n_splits + ps.first) * A.rows_wg + rl;
  const int nsp = n_active_splits(ctx_len(A, b, nullptr), ps.nb);
  const size_t sstride = (size_t)A.rows_wg * D;
  const _Float16 *src = A.Opart + base * D + CPL * lane;
  float *wt = wts[wv];
  // reference maximum over the active splits, then the weights
  float m = -INFINITY;
  for (int sp = lane; sp < nsp; sp += 64) m = fmaxf(m, A.ML[base + (size_t)sp * A.rows_wg].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float l = 0.f;
  for (int sp = lane; sp < nsp; sp += 64) {
    const float2 ml = A.ML[base + (size_t)sp * A.rows_wg];
    const float wgt = (ml.x == -INFINITY) ? 0.f : ml.y * exp2f((ml.x - m) * A.c);
    wt[sp] = wgt;
    l += wgt;
  }
  // fixed-order total: lane partials gathered in lane order
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_down(l, o);
    if ((lane & (2 * o - 1)) == 0) l += t;
  }
  l = __shfl(l, 0);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes are done (lgkmcnt(0))
  __builtin_amdgcn_wave_barrier();
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int sp0 = 0; sp0 < nsp; sp0 += BATCH) {
    hcpl v[BATCH];
#pragma unroll
    for (int t = 0; t < BATCH; ++t) v[t] = *reinterpret_cast<const hcpl *>(src + min(sp0 + t, nsp - 1) * sstride);
#pragma unroll
    for (int t = 0; t < BATCH; ++t) {
      if (sp0 + t < nsp) {
        const float wgt = wt[sp0 + t];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = fmaf((float)v[t][c], wgt, acc[c]);
      }
    }
  }
  const float inv = 1.f / l;
  const int node = rho / A.G, hq = g * A.G + rho % A.G;
  float *o = A.out + ((size_t)(s.o + node) * A.Hq + hq) * D + CPL * lane;
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[c] = acc[c] * inv;
}

// Small head dims (D <= 64) and fp32 caches: one workgroup per (node, q
// head); each thread keeps an online softmax over a strided subset of the
// keys, then the 64 partial states are merged in LDS.
template <typename E, int D>
__global__ __launch_bounds__(64) void attn_small_kernel(ddt_plan P, const E *__restrict__ q,
                                                        const E *__restrict__ Kc,
                                                        const E *__restrict__ Vc,
                                                        const int32_t *pt, int max_pages,
                                                        const int32_t *T, int T_max,
                                                        const E *__restrict__ Kt,
                                                        const E *__restrict__ Vt, int Hq, int Hkv,
                                                        float scale, float *__restrict__ out) {
  const int hq = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const Seq s = seq_of(P, b);
  if (i >= s.n) return;
  const int g = hq / (Hq / Hkv), gi = s.o + i;
  int Tb = T[b];
  bool cut = false;
  if (Tb < 0) { Tb = 0; cut = true; }
  if (Tb > T_max) { Tb = T_max; cut = true; }
  if (pt && Tb > max_pages * DDT_PAGE) { Tb = max_pages * DDT_PAGE; cut = true; }
  if (cut && hq == 0 && i == 0 && threadIdx.x == 0) P.status[b] |= DDT_ST_CTX;
  float qv[D];
  for (int d = 0; d < D; ++d) qv[d] = (float)q[((size_t)gi * Hq + hq) * D + d];
  const unsigned long long anc = P.anc[gi];
  float m = -INFINITY, l = 0.f, acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  const int nkeys = Tb + s.n;
  for (int key = threadIdx.x; key < nkeys; key += 64) {
    const E *kp, *vp;
    int vstride;
    if (key < Tb) {
      const int page = pt ? pt[(size_t)b * max_pages + key / DDT_PAGE] : key / DDT_PAGE;
      const size_t pg = (size_t)page * Hkv + g;
      kp = Kc + (pg * DDT_PAGE + key % DDT_PAGE) * D;
      vp = Vc + pg * D * DDT_PAGE + key % DDT_PAGE;
      vstride = DDT_PAGE;
    } else {
      const int j = key - Tb;
      if (!((anc >> j) & 1ull)) continue;
      kp = Kt + ((size_t)(s.o + j) * Hkv + g) * D;
      vp = Vt + ((size_t)(s.o + j) * Hkv + g) * D;
      vstride = 1;
    }
    float sc = 0.f;
    for (int d = 0; d < D; ++d) sc = fmaf(qv[d], (float)kp[d], sc);
    sc *= scale;
    const float mn = fmaxf(m, sc);
    const float corr = __expf(m - mn), p = __expf(sc - mn);
    l = l * corr + p;
    for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], corr, p * (float)vp[d * vstride]);
    m = mn;
  }
  __shared__ float sm[64], sl[64], so[64][D + 1];
  sm[threadIdx.x] = m;
  __syncthreads();
  float M = -INFINITY;
  for (int t = 0; t < 64; ++t) M = fmaxf(M, sm[t]);
  const float wgt = (m == -INFINITY) ? 0.f : __expf(m - M);
  sl[threadIdx.x] = l * wgt;
  for (int d = 0; d < D; ++d) so[threadIdx.x][d] = acc[d] * wgt;
  __syncthreads();
  if (threadIdx.x < D) {
    float L = 0.f, O = 0.f;
    for (int t = 0; t < 64; ++t) {
      L += sl[t];
      O += so[t][threadIdx.x];
    }
    out[((size_t)gi * Hq + hq) * D + threadIdx.x] = O / L;
  }
}

int check_plan(const ddt_plan *P);

struct Cfg {
  bool mfma;
  int nb, rows_wg, n_rg, n_splits, chunk;
};

static Cfg attn_cfg(const ddt_plan *P, int Hq, int Hkv, int D, int T_max, int n_splits, int dtype) {
  Cfg c{};
  const int G = Hq / Hkv;
  c.mfma = (dtype == DDT_F16) && (D == 128 || D == 256);
  if (!c.mfma) return c;
  const int rows = G * P->n_max;
  const int blocks = (rows + 15) / 16;
  c.nb = (blocks + 3) / 4;
  if (c.nb > 3) c.nb = 3;
  c.rows_wg = 64 * c.nb;
  c.n_rg = (rows + c.rows_wg - 1) / c.rows_wg;
  int tmax = T_max > 0 ? T_max : 1;
  if (P->B > 1) {
    // a pool of splits per (KV head, row group) that the sequences share
    // (pool_slot): about one workgroup per compute unit, at least one split
    // per sequence, at most one per 256 keys of the longest context each
    if (n_splits <= 0) {
      const long long units = (long long)Hkv * c.n_rg;
      const long long want = (256 + units - 1) / units;
      const long long by_len = (long long)P->B * ((tmax + 255) / 256);
      n_splits = (int)(want < by_len ? want : by_len);
    }
    if (n_splits < P->B) n_splits = P->B;
    c.n_splits = n_splits < MAX_SPLITS ? n_splits : MAX_SPLITS;
    c.chunk = 0;
    return c;
  }
  if (n_splits <= 0) {
    // about one workgroup per compute unit
    const long long units = (long long)Hkv * c.n_rg;
    long long want = (256 + units - 1) / units;
    long long by_len = (tmax + 255) / 256;  // keep splits >= 256 keys
    n_splits = (int)(want < by_len ? want : by_len);
    if (n_splits < 1) n_splits = 1;
  }
  int chunk = (tmax + n_splits - 1) / n_splits;
  chunk = (chunk + TILE - 1) / TILE * TILE;
  c.chunk = chunk;
  c.n_splits = (tmax + chunk - 1) / chunk;
  if (c.n_splits < 1) c.n_splits = 1;
  if (c.n_splits > MAX_SPLITS) {  // the combine keeps one weight per split in LDS
    chunk = (tmax + MAX_SPLITS - 1) / MAX_SPLITS;
    c.chunk = chunk = (chunk + TILE - 1) / TILE * TILE;
    c.n_splits = (tmax + chunk - 1) / chunk;
  }
  return c;
}

static AttnArgs attn_args(const ddt_plan *P, const void *q, const int32_t *page_table, int32_t max_pages,
                          const int32_t *T, int32_t T_max, const void *Kt, const void *Vt, int32_t Hq,
                          int32_t Hkv, int32_t D, float scale, const Cfg &c, float *out, void *ws) {
  AttnArgs A{};
  A.P = *P;
  A.q = (const _Float16 *)q;
  A.Kt = (const _Float16 *)Kt;
  A.Vt = (const _Float16 *)Vt;
  A.pt = page_table;
  A.max_pages = max_pages;
  A.T = T;
  A.T_max = T_max;
  A.Hq = Hq;
  A.Hkv = Hkv;
  A.G = Hq / Hkv;
  A.c = scale * LOG2E;
  A.n_splits = c.n_splits;
  A.n_rg = c.n_rg;
  A.rows_wg = c.rows_wg;
  const size_t rows = (size_t)Hkv * c.n_rg * c.n_splits * c.rows_wg;
  A.Opart = (_Float16 *)ws;
  A.ML = (float2 *)((char *)ws + rows * D * sizeof(_Float16));
  A.out = out;
  return A;
}

// The matrix-core path: the split kernel, then the combine.
template <bool Q8>
static int launch_attn_mfma(const ddt_plan &P, const AttnArgs &A, const Cfg &c, int D, hipStream_t st) {
  // one sequence: its splits directly; several: the shared pool
  const bool pool = P.B > 1;
  dim3 grid(c.n_splits, A.Hkv, c.n_rg);
  // fp16: the ring and one spare stage for the tree tile (160 KiB at D = 256)
  const size_t lds = Q8 ? (size_t)(D == 256 ? LdsQ8<256>::TOTAL : LdsQ8<128>::TOTAL)
                        : (size_t)(NSTAGE + 1) * (D == 256 ? Lds<256>::STAGE : Lds<128>::STAGE) * sizeof(_Float16);
#define DDT_ATTN(DD, NBB)                                                                       \
  do {                                                                                          \
    const void *k_ = pool ? (const void *)attn_mfma_kernel<DD, NBB, Q8, true>                   \
                          : (const void *)attn_mfma_kernel<DD, NBB, Q8, false>;                 \
    hipError_t e_ = hipFuncSetAttribute(k_, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e_ != hipSuccess) {                                                                     \
      set_hip_error(e_);                                                                        \
      return DDT_E_HIP;                                                                         \
    }                                                                                           \
    if (pool)                                                                                   \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, NBB, Q8, true>), grid, dim3(256), lds, st, A);   \
    else                                                                                        \
      hipLaunchKernelGGL((attn_mfma_kernel<DD, NBB, Q8, false>), grid, dim3(256), lds, st, A);  \
  } while (0)
  if (D == 256) {
    if (c.nb == 1) DDT_ATTN(256, 1); else if (c.nb == 2) DDT_ATTN(256, 2); else DDT_ATTN(256, 3);
  } else {
    if (c.nb == 1) DDT_ATTN(128, 1); else if (c.nb == 2) DDT_ATTN(128, 2); else DDT_ATTN(128, 3);
  }
#undef DDT_ATTN
  const int r = launch_status();
  if (r) return r;
  if (pool) {
    dim3 rgrid((c.rows_wg + 3) / 4, A.Hkv, P.B * c.n_rg);
    if (D == 256)
      hipLaunchKernelGGL(attn_combine_rows_kernel<256>, rgrid, dim3(256), 0, st, A);
    else
      hipLaunchKernelGGL(attn_combine_rows_kernel<128>, rgrid, dim3(256), 0, st, A);
    return launch_status();
  }
  dim3 cgrid(c.rows_wg, A.Hkv, c.n_rg);
  const int n1 = std::max(0, std::min(P.n_total, P.n_max));  // the one sequence's nodes (seq_of)
#define DDT_COMBINE(DD)                                                                                   \
  hipLaunchKernelGGL(attn_combine_kernel<DD>, cgrid, dim3(256), 0, st, A.Opart, A.ML, A.T, A.pt, n1, A.G,   \
                     A.rows_wg, A.n_rg, A.n_splits, A.T_max, A)
  if (D == 256)
    DDT_COMBINE(256);
  else
    DDT_COMBINE(128);
#undef DDT_COMBINE
  return launch_status();
}

}  // namespace ddt

using namespace ddt;

extern "C" size_t ddt_tree_attn_workspace(const ddt_plan *P, int32_t Hq, int32_t Hkv, int32_t D,
                                          int32_t T_max, int32_t n_splits) {
  if (!P || Hkv < 1 || Hq < Hkv || Hq % Hkv || D < 1) return 0;
  Cfg c = attn_cfg(P, Hq, Hkv, D, T_max, n_splits, DDT_F16);
  if (!c.mfma) return 0;
  const size_t rows = (size_t)Hkv * c.n_rg * c.n_splits * c.rows_wg;
  return rows * (size_t)D * sizeof(_Float16) + rows * sizeof(float2);
}

extern "C" int ddt_tree_attn(const ddt_plan *P, const void *q, const void *Kc, const void *Vc,
                             const int32_t *page_table, int32_t max_pages, const int32_t *T,
                             int32_t T_max, const void *Kt, const void *Vt, int32_t Hq,
                             int32_t Hkv, int32_t D, float scale, int32_t dtype,
                             int32_t n_splits, float *out, void *ws, size_t ws_bytes,
                             void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!q || !Kc || !Vc || !T || !Kt || !Vt || !out) return DDT_E_ARG;
  if (!page_table && P->B != 1) return DDT_E_ARG;
  if (page_table && max_pages < 1) return DDT_E_SHAPE;
  if (Hkv < 1 || Hq < Hkv || Hq % Hkv) return DDT_E_SHAPE;
  if (T_max < 0 || n_splits < 0) return DDT_E_RANGE;
  if (dtype != DDT_F16 && dtype != DDT_F32) return DDT_E_DTYPE;
  hipStream_t st = (hipStream_t)stream;
  Cfg c = attn_cfg(P, Hq, Hkv, D, T_max, n_splits, dtype);
  if (!c.mfma) {
    if (D != 16 && D != 32 && D != 64) return DDT_E_SHAPE;
    dim3 grid(Hq, P->n_max, P->B);
#define DDT_SMALL(E, DD)                                                                          \
  hipLaunchKernelGGL((attn_small_kernel<E, DD>), grid, dim3(64), 0, st, *P, (const E *)q,         \
                     (const E *)Kc, (const E *)Vc, page_table, max_pages, T, T_max, (const E *)Kt, \
                     (const E *)Vt, Hq, Hkv, scale, out)
    if (dtype == DDT_F32) {
      if (D == 16) DDT_SMALL(float, 16); else if (D == 32) DDT_SMALL(float, 32); else DDT_SMALL(float, 64);
    } else {
      if (D == 16) DDT_SMALL(_Float16, 16); else if (D == 32) DDT_SMALL(_Float16, 32); else DDT_SMALL(_Float16, 64);
    }
#undef DDT_SMALL
    return launch_status();
  }
  if (P->B > MAX_SPLITS) return DDT_E_SHAPE;  // a split per sequence at least
  if (!ws || ws_bytes < ddt_tree_attn_workspace(P, Hq, Hkv, D, T_max, n_splits)) return DDT_E_WS;
  AttnArgs A = attn_args(P, q, page_table, max_pages, T, T_max, Kt, Vt, Hq, Hkv, D, scale, c, out, ws);
  A.Kc = (const _Float16 *)Kc;
  A.Vc = (const _Float16 *)Vc;
  return launch_attn_mfma<false>(*P, A, c, D, st);
}

extern "C" int ddt_tree_attn_q8(const ddt_plan *P, const void *q, const int8_t *Kq, const void *Ksc,
                                const int8_t *Vq, const void *Vsc, const int32_t *page_table,
                                int32_t max_pages, const int32_t *T, int32_t T_max, const void *Kt,
                                const void *Vt, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                                int32_t n_splits, float *out, void *ws, size_t ws_bytes, void *stream) {
  int r = check_plan(P);
  if (r) return r;
  if (!q || !Kq || !Ksc || !Vq || !Vsc || !T || !Kt || !Vt || !out) return DDT_E_ARG;
  if (!page_table && P->B != 1) return DDT_E_ARG;
  if (page_table && max_pages < 1) return DDT_E_SHAPE;
  if (Hkv < 1 || Hq < Hkv || Hq % Hkv) return DDT_E_SHAPE;
  if (D != 128 && D != 256) return DDT_E_SHAPE;
  if (T_max < 0 || n_splits < 0) return DDT_E_RANGE;
  const Cfg c = attn_cfg(P, Hq, Hkv, D, T_max, n_splits, DDT_F16);
  if (P->B > MAX_SPLITS) return DDT_E_SHAPE;  // a split per sequence at least
  if (!ws || ws_bytes < ddt_tree_attn_workspace(P, Hq, Hkv, D, T_max, n_splits)) return DDT_E_WS;
  AttnArgs A = attn_args(P, q, page_table, max_pages, T, T_max, Kt, Vt, Hq, Hkv, D, scale, c, out, ws);
  A.Kq = Kq;
  A.Vq = Vq;
  A.Ksc = (const _Float16 *)Ksc;
  A.Vsc = (const _Float16 *)Vsc;
  return launch_attn_mfma<true>(*P, A, c, D, (hipStream_t)stream);
}
