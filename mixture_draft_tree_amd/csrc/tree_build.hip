// Common cut-off and tree construction for the mixture draft tree.
//
// The tree is the B best prefixes by best-mode score, which is the union of
// the per-mode trees at the common cut-off (project page, "In one minute" and
// "How it works" step 3).  Both calls here run the same level-synchronous
// search over prefix depth, one 1024-thread workgroup per tree:
//
//   level d:  every kept (node, mode) entry of depth d-1 expands into the
//             candidates of row (mode, d) whose score reaches the threshold.
//             Candidates are sorted by rank, so the expansion of one entry is
//             a prefix of its row, found by binary search (scores only fall
//             with depth: log-probabilities are <= 0).  The children of all
//             entries are written as 64-bit keys (parent node, token, mode,
//             slot) into LDS and bitonic-sorted, so the copies of one prefix
//             produced by different modes become adjacent: each run is one
//             node (a prefix kept by several modes is one node), its score
//             is the run's maximum and its best mode the first mode attaining
//             it.  The run members become the node's per-mode entries for the
//             next level.
//
// mfd_mixture_threshold starts from a lower bound on the cut-off (any single
// mode's B-th depth-1 candidate) and, after every level, raises the threshold
// to the B-th best score among the unique nodes found so far -- a valid lower
// bound on the final cut-off, since those nodes are distinct prefixes.  Every
// prefix scoring at least the final cut-off is still generated (its parent
// scores at least as much under the same mode), so the B-th best found node
// is the exact cut-off.  If one level would overflow the LDS sort, the
// threshold is first raised by bisection on a lower bound of the unique count
// (each parent counts only its largest per-mode child set).
//
// mfd_tree_build runs the same search at the fixed cut-off, so it materialises
// exactly the prefixes that reach it (the per-mode keeps and their union),
// breaks the ties at the cut-off by (best mode, token sequence), and lays the
// selection out by (depth, token sequence).
#include <math.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {

namespace {

constexpr int kNT = 1024;
constexpr int kMaxSort = 16384;
constexpr size_t kTreeLdsMax = 156 * 1024;  // LDS one workgroup may use (of 160 KB per CU)
constexpr int kFirstQ = 64;  // depth-1 candidates per mode behind the threshold call's starting bound
// Leading candidates of every (mode, position) row staged in LDS when they fit
// (the searches mostly look at a row's first few candidates).
constexpr int kPreQ = 16;

// Per-tree workspace layout (offsets in bytes from the tree's base).
struct WsLayout {
  size_t node_parent, node_token, node_depth, node_S, node_mu, node_aux;
  size_t ent_node, ent_mode, ent_raw, ent_s;
  size_t fr, fr_off;
  size_t ch_raw, ch_s, ch_mode, ch_pnode, ch_tok, grp;
  size_t total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline WsLayout ws_layout(int sort_cap, int ent_cap, int node_cap) {
  WsLayout w;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o = align256(o + bytes);
    return r;
  };
  w.node_parent = take((size_t)node_cap * 4);
  w.node_token = take((size_t)node_cap * 4);
  w.node_depth = take((size_t)node_cap * 4);
  w.node_S = take((size_t)node_cap * 8);
  w.node_mu = take((size_t)node_cap * 4);
  w.node_aux = take((size_t)node_cap * 4);
  w.ent_node = take((size_t)ent_cap * 4);
  w.ent_mode = take((size_t)ent_cap * 4);
  w.ent_raw = take((size_t)ent_cap * 8);
  w.ent_s = take((size_t)ent_cap * 8);
  w.fr = take((size_t)ent_cap * 4);
  w.fr_off = take((size_t)ent_cap * 4);
  w.ch_raw = take((size_t)sort_cap * 8);
  w.ch_s = take((size_t)sort_cap * 8);
  w.ch_mode = take((size_t)sort_cap * 4);
  w.ch_pnode = take((size_t)sort_cap * 4);
  w.ch_tok = take((size_t)sort_cap * 4);
  w.grp = take((size_t)sort_cap * 4);
  w.total = o;
  return w;
}

struct TreeArgs {
  const int32_t* topk_id;
  const float* topk_raw;
  const double* lse;
  int K, L, k, B;
  int sort_cap, ent_cap, node_cap, tie_cap;
  int nk_lds;  // threshold call: the nodes' 16-bit score keys are kept in LDS
  int pre_q;   // leading candidates per row staged in LDS (0: none)
  int pre_off; // their byte offset in LDS: raw values [K * L * pre_q], then ids
  int ch_lds;  // a level's children (raw sums [sort_cap], then node offsets [sort_cap]) live in LDS
  int ch_off;  //   at this byte offset
  int f_cap;   // frontier entries whose data an LDS cache holds (0: none)
  int fc_off;  //   at this byte offset: raw [f_cap], offsets [f_cap], nodes [f_cap], modes [f_cap]
  unsigned char* ws;
  size_t ws_stride;
  int32_t* status;
  // per-tree number of active modes (modes 0..K_n-1), or null for K everywhere
  const int32_t* modes;
  // threshold outputs
  double* cutoff_out;
  int32_t* n_select_out;
  int32_t* per_mode_kept;
  // build inputs / outputs
  const double* cutoff_in;
  const int32_t* n_select_in;
  const int32_t* anchor;
  int32_t* node_token;
  int32_t* parent;
  int32_t* depth;
  double* score;
  int32_t* best_mode;
  int32_t* n_nodes;
};

struct Tree {
  int32_t *node_parent, *node_token, *node_depth, *node_mu, *node_aux;
  double* node_S;
  int32_t *ent_node, *ent_mode;
  double *ent_raw, *ent_s;
  int32_t *fr, *fr_off;
  double *ch_raw, *ch_s;
  int32_t *ch_mode, *ch_pnode, *ch_tok, *grp;
};

struct Ctl {
  double tau;
  int node_count, ent_count, fsize, fail;
  int C;
  int level_start[34];
  int sh[8];
  int scan[kNT / kWave];
  uint32_t hist[256];
  int kept[32];
  int fcount[kNT / kWave];
  int small;  // children of a level built by small_level, -1 if it did not fit
  int up;     // a node of this level has a 16-bit score key above the threshold's
};

// LDS cache of the current frontier's entries (mode, accumulated raw logit,
// node) and of their child offsets, valid while the frontier has at most
// TreeArgs::f_cap entries (every writer of a frontier fills it).
struct FrontierCache {
  double* raw;
  int32_t* off;
  uint16_t* node;
  uint8_t* mode;
};

// Bytes of LDS before the optional node-key array: sort keys, norms, Ctl.
__host__ __device__ inline size_t tree_lds_base(int sort_cap, int K, int L) {
  return (size_t)sort_cap * 8 + (size_t)K * (L + 1) * 8 + sizeof(Ctl);
}

__device__ __forceinline__ Tree tree_ptrs(const TreeArgs& a, int n) {
  const WsLayout w = ws_layout(a.sort_cap, a.ent_cap, a.node_cap);
  unsigned char* b = a.ws + (size_t)n * a.ws_stride;
  Tree t;
  t.node_parent = (int32_t*)(b + w.node_parent);
  t.node_token = (int32_t*)(b + w.node_token);
  t.node_depth = (int32_t*)(b + w.node_depth);
  t.node_S = (double*)(b + w.node_S);
  t.node_mu = (int32_t*)(b + w.node_mu);
  t.node_aux = (int32_t*)(b + w.node_aux);
  t.ent_node = (int32_t*)(b + w.ent_node);
  t.ent_mode = (int32_t*)(b + w.ent_mode);
  t.ent_raw = (double*)(b + w.ent_raw);
  t.ent_s = (double*)(b + w.ent_s);
  t.fr = (int32_t*)(b + w.fr);
  t.fr_off = (int32_t*)(b + w.fr_off);
  t.ch_raw = (double*)(b + w.ch_raw);
  t.ch_s = (double*)(b + w.ch_s);
  t.ch_mode = (int32_t*)(b + w.ch_mode);
  t.ch_pnode = (int32_t*)(b + w.ch_pnode);
  t.ch_tok = (int32_t*)(b + w.ch_tok);
  t.grp = (int32_t*)(b + w.grp);
  return t;
}

// Number of leading candidates j of a rank-sorted row with
// (raw + x_j) - norm >= tau and x_j > -inf.
__device__ __forceinline__ int count_children(const float* vals, int k, double raw, double norm, double tau) {
  int lo = 0, hi = k;  // answer in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const float x = vals[mid];
    const bool ok = (x != -INFINITY) && ((raw + (double)x) - norm >= tau);
    if (ok) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// count_children when the row's first q candidates (q <= k) are also in LDS
// (pre): the search stays there unless all q of them qualify.
__device__ __forceinline__ int count_children_pre(const float* pre, int q, const float* vals, int k, double raw,
                                                  double norm, double tau) {
  auto ok = [&](float x) { return (x != -INFINITY) && ((raw + (double)x) - norm >= tau); };
  if (q > 0 && !ok(pre[q - 1])) {
    int lo = 0, hi = q - 1;  // answer in [lo, hi]
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (ok(pre[mid])) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  }
  int lo = q, hi = k;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ok(vals[mid])) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// count_children by one wave: the condition holds on a prefix of the row
// (ranks are in descending order and the score is monotone in the logit), so
// the count is the number of positions where it holds; all loads of a block
// of 4 * 64 positions are issued together.
__device__ __forceinline__ int wave_count_children(const float* vals, int k, double raw, double norm, double tau) {
  const int lane = lane_id();
  int total = 0;
  for (int b = 0; b < k; b += 4 * kWave) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = b + u * kWave + lane;
      x[u] = j < k ? vals[j] : -INFINITY;
    }
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = (x[u] != -INFINITY) && ((raw + (double)x[u]) - norm >= tau);
      cnt += __popcll(__ballot(ok));
    }
    total += cnt;
    const int valid = k - b < 4 * kWave ? k - b : 4 * kWave;
    if (cnt < valid) break;
  }
  return total;
}

// A lower bound of the rank-th largest of the doubles score(i), i in [0, n),
// for which use(i) holds (the caller guarantees at least `rank` of them):
// the rank-th largest of their ordered keys with the low 48 bits cleared,
// which is at or below every key it stands for.  Two radix passes.
template <typename Score, typename Use>
__device__ __forceinline__ double kth_lower_bound(int n, int rank, Score score, Use use, Ctl& ctl) {
  auto get = [&](int i, uint64_t* key) -> bool {
    if (!use(i)) return false;
    *key = f64_key(score(i)) >> 48;
    return true;
  };
  const uint64_t kb = block_kth_largest<kNT, 16>(n, rank, get, ctl.hist, ctl.sh);
  return f64_from_key(kb << 48);
}

// The rank-th largest 16-bit score key among the items scoring at least t0,
// as a lower bound of their rank-th best score; -inf when fewer than rank
// items reach t0.  Their keys are at least t0's key kt, and the scores in
// play span far fewer than 255 keys above it (16 per binade), so one pass
// histograms key - kt (255 and above share the top bin), counting the items
// as it goes, and the two radix passes of kth_lower_bound run only when the
// rank-th key falls in the top bin.  Barriers inside.
template <typename Score>
__device__ __forceinline__ double kth_lower_bound_above(int n, int rank, Score score, double t0, Ctl& ctl) {
  const int tid = threadIdx.x;
  const uint32_t kt = (uint32_t)(f64_key(t0) >> 48);
  for (int i = tid; i < 256; i += kNT) ctl.hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kNT) {
    const double sc = score(i);
    if (sc >= t0) atomicAdd(&ctl.hist[min((uint32_t)(f64_key(sc) >> 48) - kt, 255u)], 1u);
  }
  __syncthreads();
  if (tid < kWave) {
    int tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) tot += (int)ctl.hist[4 * tid + j];
    tot = wave_allreduce(tot, [](int x, int y) { return x + y; });
    int digit = -1, above = 0;
    if (tot >= rank && rank > 0) wave_pick_digit(ctl.hist, rank, &digit, &above);
    digit = wave_allreduce(digit, [](int x, int y) { return x > y ? x : y; });
    if (tid == 0) ctl.sh[0] = tot >= rank && rank > 0 ? digit : -1;
  }
  __syncthreads();
  const int dg = ctl.sh[0];
  __syncthreads();
  if (dg < 0) return -INFINITY;
  if (dg < 255) return f64_from_key((uint64_t)(kt + (uint32_t)dg) << 48);
  return kth_lower_bound(n, rank, score, [&](int i) { return score(i) >= t0; }, ctl);
}

// The exact rank-th largest (rank >= 1, at most n) of the doubles score(i),
// i in [0, n).  The 16-bit lower bound first fixes the bucket of keys that
// holds the answer; the members of that bucket (listed in `buf`, capacity
// `cap`) then rank themselves by direct comparison.  Falls back to the full
// 64-bit radix select if the bucket does not fit.  Barriers inside.
template <typename Score>
__device__ __forceinline__ double exact_kth(int n, int rank, Score score, Ctl& ctl, uint64_t* buf, int cap) {
  const int tid = threadIdx.x;
  const double lb = kth_lower_bound(n, rank, score, [](int) { return true; }, ctl);
  const uint64_t b16 = f64_key(lb) >> 48;
  if (tid == 0) {
    ctl.sh[4] = 0;  // members of the bucket
    ctl.sh[5] = 0;  // keys above the bucket
  }
  __syncthreads();
  int above = 0;
  for (int i = tid; i < n; i += kNT) {
    const uint64_t key = f64_key(score(i));
    if ((key >> 48) > b16) ++above;
    else if ((key >> 48) == b16) {
      const int slot = atomicAdd(&ctl.sh[4], 1);
      if (slot < cap) buf[slot] = key;
    }
  }
  above = block_sum<kNT>(above, ctl.scan);
  const int nb = ctl.sh[4];
  const int need = rank - above;  // 1 <= need <= nb
  if (nb > cap) {
    auto get = [&](int i, uint64_t* key) -> bool {
      *key = f64_key(score(i));
      return true;
    };
    return f64_from_key(block_kth_largest<kNT, 64>(n, rank, get, ctl.hist, ctl.sh));
  }
  // the member with fewer than `need` members above it and at least `need`
  // at or above it holds the answer
  for (int q = tid; q < nb; q += kNT) {
    const uint64_t mine = buf[q];
    int gt = 0, ge = 0;
    for (int r = 0; r < nb; ++r) {
      const uint64_t o = buf[r];
      gt += o > mine ? 1 : 0;
      ge += o >= mine ? 1 : 0;
    }
    if (gt < need && need <= ge) ctl.sh[6] = (int)(uint32_t)(mine >> 32), ctl.sh[7] = (int)(uint32_t)mine;
  }
  __syncthreads();
  const uint64_t ans = ((uint64_t)(uint32_t)ctl.sh[6] << 32) | (uint64_t)(uint32_t)ctl.sh[7];
  __syncthreads();
  return f64_from_key(ans);
}

// One wave builds a whole level when the frontier has at most 64 entries and
// each of them at most 8 children reaching tau (so at most 64 children): the
// counts come from the first 8 candidates of every entry's row (one round of
// loads), the children are gathered by shuffles, sorted by (parent, token,
// mode, index) with a wave sort and split into runs with ballots.  It writes
// exactly what the block path writes (same node and entry order) and keeps
// each child's score in `my_s` (lane = the child's position in that order).
// Returns the number of children, or -1, writing nothing, if the level does
// not fit.  Wave 0 only, no block barrier.
__device__ __forceinline__ int small_level(const TreeArgs& a, const Tree& t, int n, int d, int fsize, double tau,
                                           const double* norm, Ctl& ctl, uint16_t* nk, const float* pre_raw,
                                           const int32_t* pre_id, const FrontierCache& fc, bool cached, double& my_s,
                                           int& my_mode, double& my_raw, int& my_node) {
  const int lane = lane_id();
  const int K = a.K, L = a.L, k = a.k, Lp1 = L + 1;
  int m = 0, pnode = 0, cnt = 0;
  double raw = 0.0, nrm = 0.0;
  float v[8];
  int id[8];
  bool more = false;
  if (lane < fsize) {
    if (cached) {
      m = fc.mode[lane];
      raw = fc.raw[lane];
      pnode = fc.node[lane];
    } else {
      const int e = t.fr[lane];
      m = t.ent_mode[e];
      raw = t.ent_raw[e];
      pnode = t.ent_node[e];
    }
    nrm = norm[m * Lp1 + d];
    const size_t row = ((size_t)(n * K + m) * L + (d - 1)) * k;
    if (a.pre_q >= 8) {
      const int pr = (m * L + (d - 1)) * a.pre_q;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = pre_raw[pr + j];
        id[j] = pre_id[pr + j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = j < k ? a.topk_raw[row + j] : -INFINITY;
        id[j] = j < k ? a.topk_id[row + j] : 0;
      }
    }
    bool run = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      run = run && (v[j] != -INFINITY) && ((raw + (double)v[j]) - nrm >= tau);
      cnt += run ? 1 : 0;
    }
    more = cnt == 8 && k > 8;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = -INFINITY;
      id[j] = 0;
    }
  }
  if (__ballot(more) != 0ull) return -1;
  const int incl = wave_inclusive_scan(cnt);
  const int off = incl - cnt;
  const int C = __shfl(incl, kWave - 1, kWave);
  if (C > kWave) return -1;
  if (C == 0) return 0;
  if (ctl.ent_count + C > a.ent_cap || ctl.node_count + C > a.node_cap) return -1;

  // child c = lane: its entry f is the last one whose offset is at most c
  const int c = lane;
  int lo = 0, hi = fsize - 1;
#pragma unroll
  for (int it = 0; it < 6; ++it) {
    const int mid = (lo + hi + 1) >> 1;
    const int om = __shfl(off, mid, kWave);
    if (lo < hi) {
      if (om <= c) lo = mid;
      else hi = mid - 1;
    }
  }
  const int f = lo;
  const int j = c - __shfl(off, f, kWave);
  float x = -INFINITY;
  int tok = 0;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const float xv = __shfl(v[jj], f, kWave);
    const int tv = __shfl(id[jj], f, kWave);
    if (jj == j) {
      x = xv;
      tok = tv;
    }
  }
  const double craw = __shfl(raw, f, kWave) + (double)x;
  const double cs = craw - __shfl(nrm, f, kWave);
  const int cm = __shfl(m, f, kWave);
  const int cp = __shfl(pnode, f, kWave);
  const bool valid = c < C;
  const uint64_t key =
      valid ? (((uint64_t)cp << 40) | ((uint64_t)tok << 20) | ((uint64_t)cm << 15) | (uint64_t)c) : ~0ull;
  // ascending order of the keys (the descending sort of their complements)
  const uint64_t sk = ~wave_sort_desc(~key);
  const bool sv = lane < C;
  const int sc = sv ? (int)(sk & 0x7FFFu) : 0;
  const double sraw = __shfl(craw, sc, kWave);
  const double ss = __shfl(cs, sc, kWave);
  const int smode = __shfl(cm, sc, kWave);
  // runs of equal (parent, token) are one node; members are in mode order
  const uint64_t prefix = sk >> 20;
  const uint64_t prev = __shfl_up(prefix, 1, kWave);
  const bool head = sv && (lane == 0 || prefix != prev);
  const uint64_t hb = __ballot(head);
  const int g = __popcll(hb & (lanemask_lt() | (1ull << lane))) - 1;
  const int G = __popcll(hb);
  // run length of a head: up to the next head or C
  const uint64_t after = lane == kWave - 1 ? 0ull : (hb & ~((2ull << lane) - 1ull));
  const int nexth = after ? __builtin_ctzll(after) : C;
  int runlen = head ? nexth - lane : 0;
  int maxlen = runlen;
  maxlen = wave_allreduce(maxlen, [](int x, int y) { return x > y ? x : y; });
  double best = -INFINITY;
  int mu = -1;
  for (int q = 0; q < maxlen; ++q) {
    const int src = lane + q < kWave ? lane + q : kWave - 1;
    const double sq = __shfl(ss, src, kWave);
    const int mq = __shfl(smode, src, kWave);
    if (q < runlen && (mu < 0 || sq > best)) {
      best = sq;
      mu = mq;
    }
  }
  const int node0 = ctl.node_count, ent0 = ctl.ent_count;
  const uint64_t kt = f64_key(tau) >> 48;
  const bool up = __ballot(head && (f64_key(best) >> 48) > kt) != 0ull;
  if (head) {
    const int node = node0 + g;
    t.node_parent[node] = (int)(sk >> 40);
    t.node_token[node] = (int)((sk >> 20) & 0xFFFFFu);
    t.node_depth[node] = d;
    t.node_S[node] = best;
    t.node_mu[node] = mu;
    if (nk) nk[node] = (uint16_t)(f64_key(best) >> 48);
  }
  if (sv) {
    const int e = ent0 + lane;
    t.ent_node[e] = node0 + g;
    t.ent_mode[e] = smode;
    t.ent_raw[e] = sraw;
    t.ent_s[e] = ss;
  }
  if (lane == 0) {
    ctl.node_count = node0 + G;
    ctl.ent_count = ent0 + C;
    ctl.up = up ? 1 : 0;
  }
  my_s = sv ? ss : -INFINITY;
  my_mode = smode;
  my_raw = sraw;
  my_node = node0 + g;
  return C;
}

// Chunked exclusive scan of `val(i)` for i in [0, n) writing out[i]; returns the total.
template <typename Val, typename Out>
__device__ __forceinline__ int block_scan_range(int n, Val val, Out out, int* scan_smem) {
  int carry = 0;
  for (int base = 0; base < n; base += kNT) {
    const int i = base + (int)threadIdx.x;
    const int v = (i < n) ? val(i) : 0;
    int tot;
    const int ex = block_exclusive_scan<kNT>(v, scan_smem, &tot);
    if (i < n) out(i, carry + ex, v);
    carry += tot;
  }
  __syncthreads();  // outputs visible to the whole block
  return carry;
}

// The search.  Returns with ctl.node_count nodes (node 0 = root) and
// ctl.ent_count entries; ctl.fail set on capacity overflow.
template <bool BUILD>
__device__ __forceinline__ void level_search(const TreeArgs& a, const Tree& t, int n, Ctl& ctl, uint64_t* keys,
                                             const double* norm, uint16_t* nk, const float* pre_raw,
                                             const int32_t* pre_id, double* chr, int32_t* cg,
                                             const FrontierCache& fc) {
  const int K = a.K, L = a.L, k = a.k, B = a.B;
  const int tid = threadIdx.x;
  const int Lp1 = L + 1;

  for (int d = 1; d <= L; ++d) {
    if (tid == 0) {
      ctl.level_start[d] = ctl.node_count;
      ctl.up = 0;
    }
    __syncthreads();
    const int fsize = ctl.fsize;
    if (fsize == 0 || ctl.fail) break;
    double tau = ctl.tau;
    // the frontier's entries are in the LDS cache (every writer fills it up
    // to f_cap entries), else in the workspace through fr
    const bool cached = fsize <= a.f_cap;
    int32_t* froff = cached ? fc.off : t.fr_off;
    auto fe_mode = [&](int f) -> int { return cached ? (int)fc.mode[f] : t.ent_mode[t.fr[f]]; };
    auto fe_raw = [&](int f) -> double { return cached ? fc.raw[f] : t.ent_raw[t.fr[f]]; };
    auto fe_node = [&](int f) -> int { return cached ? (int)fc.node[f] : t.ent_node[t.fr[f]]; };

    // (threshold call) raise tau to the B-th best unique node so far.  The
    // raise works on 16-bit score keys; if no node of this level has a key
    // above tau's, no key above tau's is among the B best either (the older
    // nodes above it are fewer than B after the last raise, and a bisection
    // only lifts tau), so the bound it would find is at most tau: skipped.
    auto raise_tau = [&]() {
      if (!ctl.up) return;
      if (nk) {
        // on the 16-bit keys in LDS: the B-th largest key among those at or
        // above tau's stands for B distinct nodes scoring at least its value.
        // One pass first: a histogram of key - kt (255 and above share the
        // top bin), which also counts the keys at or above kt; keys of the
        // scores in play span far fewer than 255 values above tau's, so the
        // B-th largest is found there unless it falls in the top bin.
        const uint32_t kt = (uint32_t)(f64_key(tau) >> 48);
        for (int i = tid; i < 256; i += kNT) ctl.hist[i] = 0u;
        __syncthreads();
        for (int i = 1 + tid; i < ctl.node_count; i += kNT) {
          const uint32_t kk = nk[i];
          if (kk >= kt) atomicAdd(&ctl.hist[min(kk - kt, 255u)], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
          int tot = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) tot += (int)ctl.hist[4 * tid + j];
          tot = wave_allreduce(tot, [](int x, int y) { return x + y; });
          int digit = -1, above = 0;
          if (tot >= B && B > 0) wave_pick_digit(ctl.hist, B, &digit, &above);
          digit = wave_allreduce(digit, [](int x, int y) { return x > y ? x : y; });
          if (tid == 0) ctl.sh[0] = tot >= B && B > 0 ? digit : -1;
        }
        __syncthreads();
        const int dg = ctl.sh[0];
        __syncthreads();
        if (dg < 0) return;  // fewer than B keys at or above tau's
        if (dg < 255) {
          const double nt = f64_from_key((uint64_t)(kt + (uint32_t)dg) << 48);
          if (nt > tau) tau = nt;
          if (tid == 0) ctl.tau = tau;
          __syncthreads();
          return;
        }
        int local = 0;
        for (int i = 1 + tid; i < ctl.node_count; i += kNT) local += nk[i] >= kt ? 1 : 0;
        const int alive = block_sum<kNT>(local, ctl.scan);
        if (alive >= B && B > 0) {
          auto get = [&](int i, uint64_t* key) -> bool {
            *key = nk[i + 1];
            return nk[i + 1] >= kt;
          };
          const uint64_t kb = block_kth_largest<kNT, 16>(ctl.node_count - 1, B, get, ctl.hist, ctl.sh);
          const double nt = f64_from_key(kb << 48);
          if (nt > tau) tau = nt;
          if (tid == 0) ctl.tau = tau;
        }
        __syncthreads();
        return;
      }
      // any lower bound of the B-th best node score is a valid threshold;
      // a 16-bit one (-inf when fewer than B nodes reach tau)
      const double tcur = tau;
      const double nt =
          kth_lower_bound_above(ctl.node_count - 1, B, [&](int i) { return t.node_S[i + 1]; }, tcur, ctl);
      if (nt > tau) tau = nt;
      if (tid == 0) ctl.tau = tau;
      __syncthreads();
    };

    if (fsize <= kWave) {
      // a small level: one wave builds it (or finds that it does not fit)
      const int ent0 = ctl.ent_count;
      double my_s = -INFINITY, my_raw = 0.0;
      int my_mode = 0, my_node = 0;
      if (tid < kWave) {
        const int cs = small_level(a, t, n, d, fsize, tau, norm, ctl, nk, pre_raw, pre_id, fc, cached, my_s, my_mode,
                                   my_raw, my_node);
        if (tid == 0) ctl.small = cs;
      }
      __syncthreads();
      const int Cs = ctl.small;
      if (Cs == 0) break;
      if (Cs > 0) {
        if (!BUILD) raise_tau();
        if (tid < kWave) {
          const double tnext = ctl.tau;
          const bool keep = tid < Cs && my_s >= tnext;
          const uint64_t kb = __ballot(keep);
          const int pos = __popcll(kb & lanemask_lt());
          if (keep) {
            t.fr[pos] = ent0 + tid;
            if (pos < a.f_cap) {
              fc.mode[pos] = (uint8_t)my_mode;
              fc.raw[pos] = my_raw;
              fc.node[pos] = (uint16_t)my_node;
            }
          }
          if (tid == 0) ctl.fsize = __popcll(kb);
        }
        __syncthreads();
        continue;
      }
    }

    // 1. per frontier entry: number of children reaching tau; exclusive offsets
    auto count_at = [&](int f, double th) -> int {
      const int m = fe_mode(f);
      const float* vals = a.topk_raw + ((size_t)(n * K + m) * L + (d - 1)) * k;
      if (a.pre_q)
        return count_children_pre(pre_raw + (m * L + (d - 1)) * a.pre_q, a.pre_q, vals, k, fe_raw(f),
                                  norm[m * Lp1 + d], th);
      return count_children(vals, k, fe_raw(f), norm[m * Lp1 + d], th);
    };
    int C;
    if (fsize <= kNT / kWave) {
      // a few entries (the first level): one wave per entry
      const int w = tid / kWave;
      if (w < fsize) {
        const int m = fe_mode(w);
        const float* vals = a.topk_raw + ((size_t)(n * K + m) * L + (d - 1)) * k;
        const int cnt = wave_count_children(vals, k, fe_raw(w), norm[m * Lp1 + d], tau);
        if (lane_id() == 0) ctl.fcount[w] = cnt;
      }
      __syncthreads();
      C = block_scan_range(
          fsize, [&](int f) { return ctl.fcount[f]; }, [&](int f, int off, int) { froff[f] = off; }, ctl.scan);
    } else {
      C = block_scan_range(
          fsize, [&](int f) { return count_at(f, tau); }, [&](int f, int off, int) { froff[f] = off; }, ctl.scan);
    }

    const bool too_big = (C > a.sort_cap) || (ctl.ent_count + C > a.ent_cap) || (ctl.node_count + C > a.node_cap);
    if (!BUILD && too_big) {
      // Raise tau by bisection on a lower bound of the unique prefixes
      // reaching it: nodes already found plus, per parent node, its largest
      // per-mode child count.
      uint64_t lo = f64_key(tau == -INFINITY ? -INFINITY : tau), hi = f64_key(INFINITY);
      for (int it = 0; it < 70 && hi - lo > 1; ++it) {
        const uint64_t mid = lo + (hi - lo) / 2;
        const double th = f64_from_key(mid);
        int local = 0;
        for (int f = tid; f < fsize; f += kNT) {
          const int node = fe_node(f);
          if (f > 0 && fe_node(f - 1) == node) continue;  // group head only
          int best = 0;
          for (int g = f; g < fsize && fe_node(g) == node; ++g) best = max(best, count_at(g, th));
          local += best;
        }
        for (int i = 1 + tid; i < ctl.node_count; i += kNT) local += (t.node_S[i] >= th) ? 1 : 0;
        const int cnt = block_sum<kNT>(local, ctl.scan);
        if (cnt >= B) lo = mid;
        else hi = mid;
      }
      tau = f64_from_key(lo);
      if (tid == 0) ctl.tau = tau;
      C = block_scan_range(
          fsize, [&](int f) { return count_at(f, tau); }, [&](int f, int off, int) { froff[f] = off; }, ctl.scan);
    }
    if ((C > a.sort_cap) || (ctl.ent_count + C > a.ent_cap) || (ctl.node_count + C > a.node_cap)) {
      if (tid == 0) ctl.fail = 1;
      __syncthreads();
      break;
    }
    if (C == 0) break;

    // 2. materialise children: the accumulated raw logit (chr), and the sort
    // key, which carries the parent node, token and mode
    for (int c = tid; c < C; c += kNT) {
      int lo = 0, hi = fsize - 1;  // largest f with froff[f] <= c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (froff[mid] <= c) lo = mid;
        else hi = mid - 1;
      }
      const int f = lo;
      const int m = fe_mode(f);
      const int j = c - froff[f];
      const size_t row = ((size_t)(n * K + m) * L + (d - 1)) * k;
      const bool staged = j < a.pre_q;
      const int pr = (m * L + (d - 1)) * a.pre_q + j;
      const float x = staged ? pre_raw[pr] : a.topk_raw[row + j];
      const int tok = staged ? pre_id[pr] : a.topk_id[row + j];
      const int pnode = fe_node(f);
      chr[c] = fe_raw(f) + (double)x;
      keys[c] = ((uint64_t)pnode << 40) | ((uint64_t)tok << 20) | ((uint64_t)m << 15) | (uint64_t)c;
    }
    const int P = next_pow2(C);
    for (int c = C + tid; c < P; c += kNT) keys[c] = ~0ull;
    __syncthreads();
    block_sort_keys<kNT>(keys, P);

    // 3. runs of equal (parent, token) are one node; cg[i] = the node offset
    // of sorted entry i
    const int node0 = ctl.node_count, ent0 = ctl.ent_count;
    const int G = block_scan_range(
        C, [&](int i) { return (i == 0 || (keys[i] >> 20) != (keys[i - 1] >> 20)) ? 1 : 0; },
        [&](int i, int off, int head) { cg[i] = head ? off : off - 1; }, ctl.scan);
    auto child_s = [&](uint64_t key) -> double {
      const int m = (int)((key >> 15) & 31u);
      return chr[key & 0x7FFFu] - norm[m * Lp1 + d];
    };
    // each entry is recorded; each run head builds its node
    for (int i = tid; i < C; i += kNT) {
      const uint64_t key = keys[i];
      const int m = (int)((key >> 15) & 31u);
      const double raw = chr[key & 0x7FFFu];
      const int node = node0 + cg[i];
      const int e = ent0 + i;
      t.ent_node[e] = node;
      t.ent_mode[e] = m;
      t.ent_raw[e] = raw;
      t.ent_s[e] = raw - norm[m * Lp1 + d];
      if (i > 0 && (keys[i - 1] >> 20) == (key >> 20)) continue;  // run heads only
      const uint64_t prefix = key >> 20;
      double best = -INFINITY;
      int mu = -1;
      for (int j = i; j < C && (keys[j] >> 20) == prefix; ++j) {
        const double s = child_s(keys[j]);
        if (mu < 0 || s > best) {
          best = s;
          mu = (int)((keys[j] >> 15) & 31u);
        }
      }
      if ((f64_key(best) >> 48) > (f64_key(tau) >> 48)) ctl.up = 1;
      t.node_parent[node] = (int)(key >> 40);
      t.node_token[node] = (int)((key >> 20) & 0xFFFFFu);
      t.node_depth[node] = d;
      t.node_S[node] = best;
      t.node_mu[node] = mu;
      if (nk) nk[node] = (uint16_t)(f64_key(best) >> 48);
    }
    __syncthreads();
    if (tid == 0) {
      ctl.node_count = node0 + G;
      ctl.ent_count = ent0 + C;
    }
    __syncthreads();

    // 4. (threshold call) raise tau to the B-th best unique node so far
    if (!BUILD) raise_tau();

    // 5. next frontier: this level's entries still reaching tau (their data
    // also into the LDS cache, up to f_cap of them)
    const double tnext = ctl.tau;
    const int fs = block_scan_range(
        C, [&](int i) { return child_s(keys[i]) >= tnext ? 1 : 0; },
        [&](int i, int off, int v) {
          if (!v) return;
          t.fr[off] = ent0 + i;
          if (off < a.f_cap) {
            const uint64_t key = keys[i];
            fc.mode[off] = (uint8_t)((key >> 15) & 31u);
            fc.raw[off] = chr[key & 0x7FFFu];
            fc.node[off] = (uint16_t)(node0 + cg[i]);
          }
        },
        ctl.scan);
    if (tid == 0) ctl.fsize = fs;
    __syncthreads();
  }
  if (tid == 0) {
    for (int d = 1; d <= L + 1; ++d)
      if (ctl.level_start[d] < 0) ctl.level_start[d] = ctl.node_count;
  }
  __syncthreads();
}

// What one launch of tree_kernel does: find the cut-off (mfd_mixture_threshold),
// build the tree at a given cut-off (mfd_tree_build), or both from one search
// (mfd_mixture_tree).
enum TreeMode { kThreshold = 0, kBuild = 1, kFused = 2 };

template <int MODE>
__global__ void __launch_bounds__(kNT) tree_kernel(TreeArgs a) {
  // the search raises its threshold as nodes are found (cut-off wanted), and
  // a tree is laid out (from the same nodes, in the fused mode)
  constexpr bool kRaise = MODE != kBuild;
  constexpr bool kEmit = MODE != kThreshold;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int K = a.K, L = a.L, k = a.k, B = a.B, Lp1 = L + 1;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem_raw);
  double* norm = reinterpret_cast<double*>(keys + a.sort_cap);
  Ctl& ctl = *reinterpret_cast<Ctl*>(norm + K * Lp1);
  uint16_t* nk = (kRaise && a.nk_lds)
                     ? reinterpret_cast<uint16_t*>(smem_raw + ((tree_lds_base(a.sort_cap, K, L) + 15) & ~size_t(15)))
                     : nullptr;
  float* pre_raw = a.pre_q ? reinterpret_cast<float*>(smem_raw + a.pre_off) : nullptr;
  int32_t* pre_id = a.pre_q ? reinterpret_cast<int32_t*>(pre_raw + (size_t)K * L * a.pre_q) : nullptr;
  const Tree t = tree_ptrs(a, n);
  // a level's children (accumulated raw logits, node offsets): LDS when they fit
  double* chr = a.ch_lds ? reinterpret_cast<double*>(smem_raw + a.ch_off) : t.ch_raw;
  int32_t* cg = a.ch_lds ? reinterpret_cast<int32_t*>(smem_raw + a.ch_off + (size_t)a.sort_cap * sizeof(double))
                         : t.grp;
  FrontierCache fc = {};
  if (a.f_cap) {
    unsigned char* f0 = smem_raw + a.fc_off;
    fc.raw = reinterpret_cast<double*>(f0);
    fc.off = reinterpret_cast<int32_t*>(f0 + (size_t)a.f_cap * 8);
    fc.node = reinterpret_cast<uint16_t*>(f0 + (size_t)a.f_cap * 12);
    fc.mode = f0 + (size_t)a.f_cap * 14;
  }
  // a tree built from its first K_n futures only: the inactive modes' rows
  // are never read (the strides keep the full K)
  int Kn = K;
  if (a.modes) {
    Kn = a.modes[n];
    if (Kn < 1 || Kn > K) {
      if (a.status && tid == 0) atomicOr(&a.status[n], MFD_TREE_BAD_MODES);
      Kn = Kn < 1 ? 1 : K;
    }
  }

  // norm[m][d] = sum_{i<d} lse[m][i], fp64, from i = 0 upward (all Kn*L
  // values loaded at once, then one running sum per mode).  A row's
  // normaliser is taken no lower than its top logit: the true one never is,
  // and a positive log-probability from rounding would let a child outscore
  // its parent (the comparison keeps a NaN normaliser NaN).
  for (int q = tid; q < Kn * L; q += kNT) {
    const int m = q / L, i = q - m * L;
    const double l = a.lse[(size_t)n * K * L + q];
    const double top = (double)a.topk_raw[((size_t)n * K * L + q) * k];
    norm[m * Lp1 + i + 1] = l < top ? top : l;
  }
  // the rows' leading candidates (past k: -inf), loaded with the norms
  for (int q = tid; q < Kn * L * a.pre_q; q += kNT) {
    const int r = q / a.pre_q, j = q - r * a.pre_q;  // r = m * L + position
    const size_t at = ((size_t)n * K * L + r) * k + j;
    pre_raw[q] = j < k ? a.topk_raw[at] : -INFINITY;
    pre_id[q] = j < k ? a.topk_id[at] : 0;
  }
  __syncthreads();
  for (int m = tid; m < Kn; m += kNT) {
    double acc = 0.0;
    norm[m * Lp1] = 0.0;
    for (int i = 0; i < L; ++i) {
      acc = acc + norm[m * Lp1 + i + 1];
      norm[m * Lp1 + i + 1] = acc;
    }
  }
  for (int i = tid; i < 32; i += kNT) ctl.kept[i] = 0;
  if (tid == 0) {
    ctl.node_count = 1;
    ctl.ent_count = Kn;
    ctl.fsize = Kn;
    ctl.fail = 0;
    for (int d = 0; d < 34; ++d) ctl.level_start[d] = -1;
    t.node_parent[0] = -1;
    t.node_token[0] = -1;
    t.node_depth[0] = 0;
    t.node_S[0] = 0.0;
    t.node_mu[0] = -1;
  }
  for (int m = tid; m < Kn; m += kNT) {
    t.ent_node[m] = 0;
    t.ent_mode[m] = m;
    t.ent_raw[m] = 0.0;
    t.ent_s[m] = 0.0;
    t.fr[m] = m;
    if (m < a.f_cap) {
      fc.mode[m] = (uint8_t)m;
      fc.raw[m] = 0.0;
      fc.node[m] = 0;
    }
  }
  __syncthreads();

  double cutoff_in = 0.0;
  int nsel_in = 0;
  if (!kRaise) {
    cutoff_in = a.cutoff_in[n];
    nsel_in = a.n_select_in[n];
    if (nsel_in > B) nsel_in = B;
    if (nsel_in < 0) nsel_in = 0;
    if (tid == 0) {
      ctl.tau = cutoff_in;
      if (nsel_in == 0) ctl.fsize = 0;
    }
  } else {
    if (tid == 0) {
      double t0 = -INFINITY;
      if (B == 0) ctl.fsize = 0;
      else if (k >= B) {
        for (int m = 0; m < Kn; ++m) {
          const float x = a.topk_raw[((size_t)(n * K + m) * L) * k + (B - 1)];
          if (x != -INFINITY) {
            const double s0 = (0.0 + (double)x) - norm[m * Lp1 + 1];
            if (s0 > t0) t0 = s0;
          }
        }
      }
      ctl.tau = t0;
    }
  }
  __syncthreads();

  if (kRaise && B > 0) {
    // A tighter start: pool each mode's first kFirstQ depth-1 candidates, give
    // each distinct token the best of its pooled scores, and take (a 16-bit
    // lower bound of) the B-th largest.  Those are B distinct prefixes whose
    // node scores are at least their pooled scores, so it is a lower bound on
    // the final cut-off too, and far above the single-mode one when the modes
    // disagree.  Scores use the search's own expression.
    const int q = k < kFirstQ ? k : kFirstQ;
    const int np = Kn * q;
    // the distinct tokens: an LDS hash table in the (free) sort area, slot h
    // holding a token and the ordered key of its best pooled score (a NaN
    // score takes the largest key, so the token's best is NaN, as below)
    int H = 1;
    while (H * 2 * 12 <= a.sort_cap * 8) H *= 2;  // 12 bytes per slot
    if (np >= B && H >= 2 * np) {
      uint64_t* hkey = keys;
      uint32_t* htok = reinterpret_cast<uint32_t*>(keys + H);
      constexpr uint32_t kEmpty = 0xFFFFFFFFu;
      for (int c = tid; c < H; c += kNT) {
        hkey[c] = 0ull;
        htok[c] = kEmpty;
      }
      __syncthreads();
      for (int c = tid; c < np; c += kNT) {
        const int m = c / q, j = c - m * q;
        const size_t at = ((size_t)(n * K + m) * L) * k + j;
        const int tok = a.topk_id[at];
        const float x = a.topk_raw[at];
        if (tok < 0 || x == -INFINITY) continue;  // no candidate: its score is -inf
        const double sc = (0.0 + (double)x) - norm[m * Lp1 + 1];
        // Fibonacci hashing, linear probing; H > np slots, so a probe ends
        uint32_t h = ((uint32_t)tok * 0x9E3779B1u) & (uint32_t)(H - 1);
        while (true) {
          const uint32_t prev = atomicCAS(&htok[h], kEmpty, (uint32_t)tok);
          if (prev == kEmpty || prev == (uint32_t)tok) break;
          h = (h + 1u) & (uint32_t)(H - 1);
        }
        atomicMax(reinterpret_cast<unsigned long long*>(&hkey[h]), (unsigned long long)(sc != sc ? ~0ull : f64_key(sc)));
      }
      __syncthreads();
      const double t0 = ctl.tau;
      auto best = [&](int i) { return htok[i] == kEmpty ? (double)NAN : f64_from_key(hkey[i]); };
      const double nb = kth_lower_bound_above(H, B, best, t0, ctl);  // -inf: fewer than B reach t0
      if (tid == 0 && nb > t0) ctl.tau = nb;
      __syncthreads();
    } else if (np >= B) {
      // keys[0, P) are sorted; the pooled scores wait in keys[P, 2P)
      // (2P <= sort_cap: sort_cap >= 2 K k, or 16384)
      const int P = next_pow2(np);
      double* pooled = reinterpret_cast<double*>(keys + P);
      for (int c = tid; c < P; c += kNT) {
        uint64_t key = ~0ull;
        if (c < np) {
          const int m = c / q, j = c - m * q;
          const size_t at = ((size_t)(n * K + m) * L) * k + j;
          const int tok = a.topk_id[at];
          const float x = a.topk_raw[at];
          key = ((uint64_t)(uint32_t)tok << 32) | (uint64_t)c;
          pooled[c] = (0.0 + (double)x) - norm[m * Lp1 + 1];
        }
        keys[c] = key;
      }
      __syncthreads();
      block_sort_keys<kNT>(keys, P);
      // runs of equal token: the head holds the best score, the rest NaN
      for (int i = tid; i < np; i += kNT) {
        double best = NAN;
        const uint64_t tk = keys[i] >> 32;
        if (i == 0 || (keys[i - 1] >> 32) != tk) {
          best = -INFINITY;
          bool bad = false;
          for (int r = i; r < np && (keys[r] >> 32) == tk; ++r) {
            const double sc = pooled[(uint32_t)keys[r]];
            if (sc != sc) bad = true;
            else if (sc > best) best = sc;
          }
          if (bad) best = NAN;
        }
        t.ch_s[i] = best;
      }
      __syncthreads();
      const double t0 = ctl.tau;
      const double nb = kth_lower_bound_above(np, B, [&](int i) { return t.ch_s[i]; }, t0, ctl);
      if (tid == 0 && nb > t0) ctl.tau = nb;
      __syncthreads();
    }
  }

  level_search<!kRaise>(a, t, n, ctl, keys, norm, nk, pre_raw, pre_id, chr, cg, fc);

  const int nc = ctl.node_count;
  const int fail = ctl.fail;
  if (fail && a.status && tid == 0) atomicOr(&a.status[n], MFD_TREE_CAPACITY);

  if (kRaise) {
    // ---------------------------------------------------------- cut-off
    const int total = nc - 1;
    int nsel = 0;
    double cut = INFINITY;
    if (!fail && B > 0 && total > 0) {
      nsel = total >= B ? B : total;
      cut = exact_kth(total, nsel, [&](int i) { return t.node_S[i + 1]; }, ctl, keys, a.sort_cap);
    }
    if (fail) cut = NAN;
    if (a.per_mode_kept) {
      for (int e = Kn + tid; e < ctl.ent_count; e += kNT)
        if (!fail && nsel > 0 && t.ent_s[e] >= cut) atomicAdd(&ctl.kept[t.ent_mode[e]], 1);
      __syncthreads();
      for (int m = tid; m < K; m += kNT) a.per_mode_kept[(size_t)n * K + m] = ctl.kept[m];
    }
    if (tid == 0) {
      a.cutoff_out[n] = cut;
      a.n_select_out[n] = nsel;
    }
    if (!kEmit) return;
    // Fused: the search materialised every prefix with some per-mode score at
    // or above its running threshold, which never exceeded the cut-off, so
    // every prefix at or above the cut-off is a node, with all the modes that
    // reach the cut-off among its entries: its score and best mode are those
    // the build call would find.  Nodes below the cut-off are never selected.
    cutoff_in = cut;
    nsel_in = nsel;
    __syncthreads();
  }

  // ------------------------------------------------------------ tree build
  const int Bp1 = B + 1;
  const int M = nc - 1;
  int nsel = fail ? 0 : (nsel_in < M ? nsel_in : M);
  // node_aux: 1 = selected, then the canonical row index
  if (M > nsel && nsel > 0) {
    // The nsel-th best node score.  It is the given cut-off itself when fewer
    // than nsel nodes lie above it and at least nsel at or above it, as for
    // the threshold call's own cut-off; otherwise it is selected exactly.
    int lgt = 0, lge = 0;
    for (int i = 1 + tid; i < nc; i += kNT) {
      const double sc = t.node_S[i];
      lgt += (sc > cutoff_in) ? 1 : 0;
      lge += (sc >= cutoff_in) ? 1 : 0;
    }
    const int gt_in = block_sum<kNT>(lgt, ctl.scan);
    const int ge_in = block_sum<kNT>(lge, ctl.scan);
    double cstar = cutoff_in;
    int gt = gt_in;
    const bool exact_in = gt_in < nsel && ge_in >= nsel;
    if (exact_in && ge_in == nsel) {
      // exactly nsel nodes reach the cut-off: no ties to break
      for (int i = 1 + tid; i < nc; i += kNT) t.node_aux[i] = (t.node_S[i] >= cutoff_in) ? 1 : 0;
      __syncthreads();
    } else {
      if (!exact_in) {
        cstar = exact_kth(M, nsel, [&](int i) { return t.node_S[i + 1]; }, ctl, keys, a.sort_cap);
        lgt = 0;
        for (int i = 1 + tid; i < nc; i += kNT) lgt += (t.node_S[i] > cstar) ? 1 : 0;
        gt = block_sum<kNT>(lgt, ctl.scan);
      }
      const int need = nsel - gt;
      // collect the ties at cstar (node ids in node_aux order via keys[] as int list)
      int32_t* tied = reinterpret_cast<int32_t*>(keys);
      const int T = block_scan_range(
          M, [&](int i) { return (t.node_S[i + 1] == cstar) ? 1 : 0; },
          [&](int i, int off, int v) {
            if (v && off < a.tie_cap) tied[off] = i + 1;
          },
          ctl.scan);
      for (int i = 1 + tid; i < nc; i += kNT) t.node_aux[i] = (t.node_S[i] > cstar) ? 1 : 0;
      __syncthreads();
      if (T > a.tie_cap) {
        if (tid == 0) {
          if (a.status) atomicOr(&a.status[n], MFD_TREE_CAPACITY);
          ctl.fail = 1;
        }
      } else {
        // token paths of the tied nodes, then rank by (best mode, tokens)
        int32_t* paths = tied + a.tie_cap;
        for (int q = tid; q < T; q += kNT) {
          int node = tied[q];
          const int dq = t.node_depth[node];
          for (int x = 0; x < L; ++x) paths[q * L + x] = -1;
          while (node > 0) {
            paths[q * L + t.node_depth[node] - 1] = t.node_token[node];
            node = t.node_parent[node];
          }
          (void)dq;
        }
        __syncthreads();
        for (int q = tid; q < T; q += kNT) {
          const int nq = tied[q];
          const int mq = t.node_mu[nq], dq = t.node_depth[nq];
          int rank = 0;
          for (int r = 0; r < T; ++r) {
            if (r == q) continue;
            const int nr = tied[r];
            const int mr = t.node_mu[nr], dr = t.node_depth[nr];
            bool less;
            if (mr != mq) less = mr < mq;
            else {
              int x = 0;
              const int dm = dr < dq ? dr : dq;
              while (x < dm && paths[r * L + x] == paths[q * L + x]) ++x;
              if (x < dm) less = paths[r * L + x] < paths[q * L + x];
              else less = dr < dq;
            }
            rank += less ? 1 : 0;
          }
          if (rank < need) t.node_aux[nq] = 1;
        }
      }
      __syncthreads();
    }
  } else {
    for (int i = 1 + tid; i < nc; i += kNT) t.node_aux[i] = (i - 1 < nsel) ? 1 : 0;
    __syncthreads();
  }
  const int fail2 = ctl.fail;

  // Canonical layout.  The search created nodes level by level, and within a
  // level in ascending (parent node, token) order: a level's children are
  // sorted by that key before its runs become nodes.  By induction over depth
  // this is the order (depth, token sequence) of the prefixes -- at depth d
  // two prefixes compare as their parents do, or by their last token under
  // one parent -- and it stays so among the selected nodes, since a selected
  // node's parent is selected.  A selected node's row is therefore one plus
  // the number of selected nodes created before it: one scan, no sort.
  int base = 1;
  if (!fail2) {
    // node_aux: 1 = selected; after the scan, row + 2 for selected nodes
    const int cnt = block_scan_range(
        nc - 1, [&](int i) { return t.node_aux[i + 1] == 1 ? 1 : 0; },
        [&](int i, int off, int v) {
          if (v) t.node_aux[i + 1] = off + 3;
        },
        ctl.scan);
    for (int node = 1 + tid; node < nc; node += kNT) {
      const int aux = t.node_aux[node];
      if (aux < 3) continue;
      const int rowi = aux - 2;
      const int p = t.node_parent[node];
      const int prow = (p == 0) ? 0 : (t.node_aux[p] - 2);
      const size_t o = (size_t)n * Bp1 + rowi;
      a.node_token[o] = t.node_token[node];
      a.parent[o] = prow;
      a.depth[o] = t.node_depth[node];
      a.score[o] = t.node_S[node];
      a.best_mode[o] = t.node_mu[node];
    }
    base = 1 + cnt;
  }
  const int rows = fail2 ? 1 : base;
  for (int i = tid; i < Bp1; i += kNT) {
    const size_t o = (size_t)n * Bp1 + i;
    if (i == 0) {
      a.node_token[o] = a.anchor[n];
      a.parent[o] = -1;
      a.depth[o] = 0;
      a.score[o] = 0.0;
      a.best_mode[o] = -1;
    } else if (i >= rows) {
      a.node_token[o] = -1;
      a.parent[o] = -1;
      a.depth[o] = -1;
      a.score[o] = -INFINITY;
      a.best_mode[o] = -1;
    }
  }
  if (tid == 0) a.n_nodes[n] = rows;
}

}  // namespace

TreeCaps tree_caps(int K, int L, int k, int B) {
  TreeCaps c;
  long long want = 2LL * K * k;
  if (want < 2LL * (B + 1)) want = 2LL * (B + 1);
  if (want < 2048) want = 2048;  // small trees: room for ~4096 / (1 + L) exact ties at the cut-off
  if (want > kMaxSort) want = kMaxSort;
  c.sort_cap = next_pow2((int)want);
  c.ent_cap = 4 * c.sort_cap;
  c.node_cap = 4 * c.sort_cap;
  if (c.node_cap > 65535) c.node_cap = 65535;  // node ids fit 16 bits in the layout keys
  const WsLayout w = ws_layout(c.sort_cap, c.ent_cap, c.node_cap);
  c.ws_bytes_per_tree = w.total;
  c.lds_bytes = tree_lds_base(c.sort_cap, K, L) + 64;
  return c;
}

static int tie_cap_for(const TreeCaps& c, int L) {
  // tied ids + paths share the sort buffer: cap * (1 + L) ints <= sort_cap * 2 ints
  int t = (c.sort_cap * 2) / (1 + L);
  return t < 1 ? 1 : t;
}

static hipError_t launch_tree(int mode, TreeArgs& a, int N, hipStream_t stream) {
  const TreeCaps c = tree_caps(a.K, a.L, a.k, a.B);
  a.sort_cap = c.sort_cap;
  a.ent_cap = c.ent_cap;
  a.node_cap = c.node_cap;
  a.tie_cap = tie_cap_for(c, a.L);
  a.ws_stride = c.ws_bytes_per_tree;
  const void* fn = mode == kBuild  ? reinterpret_cast<const void*>(&tree_kernel<kBuild>)
                   : mode == kFused ? reinterpret_cast<const void*>(&tree_kernel<kFused>)
                                    : reinterpret_cast<const void*>(&tree_kernel<kThreshold>);
  // the searches that raise their threshold keep a 16-bit score key per node
  // in LDS when it fits
  size_t lds = c.lds_bytes;
  const size_t nk_off = (tree_lds_base(c.sort_cap, a.K, a.L) + 15) & ~size_t(15);
  const size_t nk_end = nk_off + (size_t)c.node_cap * sizeof(uint16_t);
  a.nk_lds = (mode != kBuild && nk_end <= kTreeLdsMax) ? 1 : 0;
  if (a.nk_lds && nk_end > lds) lds = nk_end;
  // the rows' leading candidates after that, when they fit
  const size_t pre_off = (lds + 15) & ~size_t(15);
  const size_t pre_end = pre_off + (size_t)a.K * a.L * kPreQ * (sizeof(float) + sizeof(int32_t));
  a.pre_q = pre_end <= kTreeLdsMax ? kPreQ : 0;
  a.pre_off = (int)pre_off;
  if (a.pre_q) lds = pre_end;
  // then a level's children (raw sums and node offsets, 12 bytes per key)
  const size_t ch_off = (lds + 15) & ~size_t(15);
  const size_t ch_end = ch_off + (size_t)c.sort_cap * (sizeof(double) + sizeof(int32_t));
  a.ch_lds = ch_end <= kTreeLdsMax ? 1 : 0;
  a.ch_off = (int)ch_off;
  if (a.ch_lds) lds = ch_end;
  // and a cache of the frontier's entries, as many as fit (15 bytes each; a
  // frontier of more entries reads them from the workspace)
  const size_t fc_off = (lds + 15) & ~size_t(15);
  long long f_cap = fc_off < kTreeLdsMax ? (long long)((kTreeLdsMax - fc_off) / 15) : 0;
  f_cap = f_cap / 64 * 64;
  if (f_cap > c.ent_cap) f_cap = c.ent_cap;
  if (f_cap < a.K) f_cap = 0;  // the root entries must fit
  a.f_cap = (int)f_cap;
  a.fc_off = (int)fc_off;
  if (a.f_cap) lds = fc_off + (size_t)f_cap * 15;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (N == 0) return hipSuccess;
  if (mode == kBuild) hipLaunchKernelGGL(tree_kernel<kBuild>, dim3(N), dim3(kNT), lds, stream, a);
  else if (mode == kFused) hipLaunchKernelGGL(tree_kernel<kFused>, dim3(N), dim3(kNT), lds, stream, a);
  else hipLaunchKernelGGL(tree_kernel<kThreshold>, dim3(N), dim3(kNT), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_mixture_threshold(const int32_t* topk_id, const float* topk_raw, const double* lse, int N, int K,
                                    int L, int k, int B, const int32_t* modes, double* cutoff, int32_t* n_select,
                                    int32_t* per_mode_kept, int32_t* status, void* ws, hipStream_t stream) {
  TreeArgs a = {};
  a.modes = modes;
  a.topk_id = topk_id;
  a.topk_raw = topk_raw;
  a.lse = lse;
  a.K = K;
  a.L = L;
  a.k = k;
  a.B = B;
  a.ws = static_cast<unsigned char*>(ws);
  a.status = status;
  a.cutoff_out = cutoff;
  a.n_select_out = n_select;
  a.per_mode_kept = per_mode_kept;
  return launch_tree(kThreshold, a, N, stream);
}

hipError_t launch_tree_build(const int32_t* topk_id, const float* topk_raw, const double* lse, const double* cutoff,
                             const int32_t* n_select, const int32_t* anchor, int N, int K, int L, int k, int B,
                             const int32_t* modes, int32_t* node_token, int32_t* parent, int32_t* depth,
                             double* score, int32_t* best_mode, int32_t* n_nodes, int32_t* status, void* ws,
                             hipStream_t stream) {
  TreeArgs a = {};
  a.modes = modes;
  a.topk_id = topk_id;
  a.topk_raw = topk_raw;
  a.lse = lse;
  a.K = K;
  a.L = L;
  a.k = k;
  a.B = B;
  a.ws = static_cast<unsigned char*>(ws);
  a.status = status;
  a.cutoff_in = cutoff;
  a.n_select_in = n_select;
  a.anchor = anchor;
  a.node_token = node_token;
  a.parent = parent;
  a.depth = depth;
  a.score = score;
  a.best_mode = best_mode;
  a.n_nodes = n_nodes;
  return launch_tree(kBuild, a, N, stream);
}

hipError_t launch_mixture_tree(const int32_t* topk_id, const float* topk_raw, const double* lse, const int32_t* anchor,
                               int N, int K, int L, int k, int B, const int32_t* modes, double* cutoff,
                               int32_t* n_select, int32_t* per_mode_kept, int32_t* node_token, int32_t* parent,
                               int32_t* depth, double* score, int32_t* best_mode, int32_t* n_nodes, int32_t* status,
                               void* ws, hipStream_t stream) {
  TreeArgs a = {};
  a.modes = modes;
  a.topk_id = topk_id;
  a.topk_raw = topk_raw;
  a.lse = lse;
  a.K = K;
  a.L = L;
  a.k = k;
  a.B = B;
  a.ws = static_cast<unsigned char*>(ws);
  a.status = status;
  a.cutoff_out = cutoff;
  a.n_select_out = n_select;
  a.per_mode_kept = per_mode_kept;
  a.anchor = anchor;
  a.node_token = node_token;
  a.parent = parent;
  a.depth = depth;
  a.score = score;
  a.best_mode = best_mode;
  a.n_nodes = n_nodes;
  return launch_tree(kFused, a, N, stream);
}

}  // namespace mfd
