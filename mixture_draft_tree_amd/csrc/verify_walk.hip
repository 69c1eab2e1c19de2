// Tree-verification walk over the target's per-node logits.
//
// The target keeps the future it actually takes (project page, "How it works"
// step 3): starting at the root, take the target's token at the current node
// and move to the child holding that token while one exists.  The accepted
// drafted tokens plus the last (bonus) token give tau = depth + 1 (project
// page, Figure 2: six drafted tokens plus the bonus).  At T = 0 the token is
// the argmax; at T > 0 it is a Gumbel-max sample, which draws exactly from
// softmax(R / T), so decoding stays lossless (model card summary).  The noise
// is counter-based (Philox4x64-10) and keyed by (seed, depth, token), so a
// given seed samples the same tokens whatever the tree's shape.
//
// Work layout: the token chosen at a node depends only on that node's row,
// T, the seed and its depth, so the only order the walk imposes is one row
// after the other within a tree.  Every row is cut into S slices, and a round
// is one row (or its exact re-evaluation, below) of one tree.  The launch's
// workgroups, all resident at once (cooperative launch), form G groups of S:
// tree n belongs to group n mod G, and workgroup s of a group always reduces
// slice s of its trees' rows.  A workgroup serves every tree of its group, in
// whatever order their rounds open, so one waiting tree does not idle it.
// After its slice a workgroup publishes a top-two and counts itself in; the
// one that completes the round merges the S results, finds the child (tree
// nodes sit in LDS) and opens the tree's next round with one packed word, or
// ends the tree.  Waits are polls of those words, bounded; a workgroup leaves
// once all its trees have ended.  Only the rows on the walked path are read.
//
// At T > 0 the noise is first estimated in fp32 (two v_log_f32, error below
// kGumbelTol, see gumbel_estimate) and y = x / T + g is formed in fp64 from
// it, so every estimate lies within kGumbelTol (plus a few ulp of |y|) of the
// exact y.  Each round keeps the best estimate and the second best value.
// When they are further apart than twice that the best one is the exact
// winner; otherwise a second round evaluates the exact fp64 noise for every
// element whose estimate comes that close to the best, and takes the exact
// maximum.
#include <math.h>

#include <mutex>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {

// Walk workspace of mfd_verify_walk_noalloc, for callers that cannot
// allocate: one copy per GPU, held until the process ends.  Host code never
// uses this name as an address: it is a host-side stand-in, and a kernel
// handed it would fault.  The device address comes from hipGetSymbolAddress,
// once per device, below.
constexpr size_t kWalkScratchBytes = size_t(2) << 20;
static __device__ __align__(256) unsigned char scratch[kWalkScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

}  // namespace

size_t walk_scratch_bytes() { return kWalkScratchBytes; }

hipError_t walk_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy (the device is current)
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

namespace {

constexpr int kWalkThreads = 256;
constexpr int kWalkWaves = kWalkThreads / kWave;
constexpr int kSlices = 64;                  // slices per row, at most
constexpr int kMaxRounds = 2 * (32 + 1);     // two rounds per depth, L <= 32
constexpr int kMaxServed = kWave;            // trees one workgroup serves, at most
constexpr long long kIdleLimit = 1LL << 22;  // polls without work before giving up (seconds; never in practice)
constexpr int kPollSleep = 2;                // s_sleep units (64 clocks each) between polls
constexpr double kGumbelTol = 1e-4;
constexpr float kLn2f = 0.693147180559945309f;
constexpr int kSliceVec = 2;                 // 16-byte vectors per thread per round of loads
constexpr int kNodesLds = 2048;              // node (parent, token) pairs of the served trees kept in LDS

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t lane_word(const Philox4& r, int l) {
  return l == 0 ? r.v[0] : (l == 1 ? r.v[1] : (l == 2 ? r.v[2] : r.v[3]));
}

// (y, index) with larger y first, then lower index.
__device__ __forceinline__ bool better(double y, int i, double by, int bi) {
  return (y > by) || (y == by && i < bi);
}

// fp32 estimate of the noise g = -ln(-ln U), U = ((w >> 12) + 0.5) 2^-52.
// With t = -ln U:
//  * 1 - U < 2^-8 (m = 2^52 - (w >> 12) < 2^44): u = 1 - U = (m - 0.5) 2^-52
//    is formed with relative error <= 2^-23 and t ~ u (1 + u / 2), whose
//    truncation error is below u^2 / 3 <= 2^-16 / 3 relative;
//  * otherwise U is formed with relative error <= 2^-23, which moves ln U by
//    at most 2^-23, i.e. by at most 2^-23 / |ln U| <= 2^-15 relative to t
//    (|ln U| >= 2^-8 here); v_log_f32 adds a few ulp of |log2 U| <= 53.
// A relative error e of t moves g by about e, and the final v_log_f32 and
// scaling add at most ~1e-5, so |estimate - g| < 5e-5 < kGumbelTol.
__device__ __forceinline__ float gumbel_estimate(uint64_t w) {
  const uint64_t hi = w >> 12;
  const uint64_t m = (1ull << 52) - hi;  // in [1, 2^52]
  const float u = ((float)m - 0.5f) * 0x1.0p-52f;
  const float U = ((float)hi + 0.5f) * 0x1.0p-52f;
  const float t_small = u * (1.f + 0.5f * u);
  const float t_big = -__builtin_amdgcn_logf(U) * kLn2f;
  const float t = m < (1ull << 44) ? t_small : t_big;
  return -__builtin_amdgcn_logf(t) * kLn2f;
}

// Best (value, index) and the second best value seen.
struct Top2 {
  double y1;
  int i1;
  double y2;
};

__device__ __forceinline__ void top2_add(Top2& t, double y, int i) {
  if (better(y, i, t.y1, t.i1)) {
    t.y2 = t.y1;
    t.y1 = y;
    t.i1 = i;
  } else if (y > t.y2) {
    t.y2 = y;
  }
}

__device__ __forceinline__ void top2_merge(Top2& a, const Top2& b) {
  top2_add(a, b.y1, b.i1);
  if (b.y2 > a.y2) a.y2 = b.y2;
}

__device__ __forceinline__ Top2 top2_shfl_xor(const Top2& t, int o) {
  Top2 r;
  r.y1 = __shfl_xor(t.y1, o, kWave);
  r.i1 = __shfl_xor(t.i1, o, kWave);
  r.y2 = __shfl_xor(t.y2, o, kWave);
  return r;
}

// Per-tree round word: 0 = no round open, kEnded = the tree has ended, else
// (round + 1) | kind << 7 | step << 8 | node << 14, where kind 1 marks an
// exact re-evaluation of the row (its cut-off is in `cut`) and step is the
// number of moves from the root (the output position of the round's token).
constexpr uint32_t kEnded = 0xFFFFFFFFu;
__host__ __device__ __forceinline__ uint32_t round_word(int r, int kind, int step, int u) {
  return (uint32_t)(r + 1) | ((uint32_t)kind << 7) | ((uint32_t)step << 8) | ((uint32_t)u << 14);
}

struct WalkArgs {
  const void* target;
  int N, Bp1, L, S, G;
  long long V;
  const int32_t* node_token;
  const int32_t* parent;
  const int32_t* depth;
  const int32_t* n_nodes;
  const float* temperature;
  const uint64_t* seed;
  int32_t* tau;
  int32_t* out_tokens;
  int32_t* path_nodes;
  int32_t* status;
  uint32_t* word;  // [N] round words
  double* cut;     // [N] cut-off of an exact round
  int32_t* done;   // [N][kMaxRounds] slices finished per round
  double* py1;     // [N][kSlices] slice results of the open round
  double* py2;
  int32_t* pi;
};

// Ordering between workgroups.  Everything one workgroup hands to another
// (slice results, cut-offs, counters, round words) is written and read with
// agent-scope atomic stores, loads and RMWs; on this device family those
// loads and stores carry the sc1 (device-scope) cache policy and act at the
// device's coherence point, as do the RMWs.  In the LLVM AMDGPU memory model
// for this family an agent-scope release is "write back L2 (buffer_wbl2 sc1),
// then wait for every earlier access to complete (s_waitcnt vmcnt(0))" and an
// acquire is "wait, then invalidate (buffer_inv sc1)"; the writeback and the
// invalidate exist for non-atomic data, and the kernel hands over none (the
// rows and nodes it reads are never written by it).  What remains of a
// release or an acquire is the wait, which `drain` issues: every access
// before it has completed at the coherence point before any access after it
// is issued.  The signal fences around it stop the compiler from moving
// memory accesses across it (s_waitcnt alone is no compiler barrier), so
// program order is the order the hardware sees.
__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename T>
__device__ __forceinline__ T ld(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct WalkShared {
  Top2 w[kWalkWaves];
  Top2 g;  // merged result of a round
  int child;
  int j, quit, last;
  uint32_t word;
  double cut;
  int seen[kMaxServed];   // last round this workgroup reduced, per served tree
  int node0[kMaxServed];  // first LDS slot of the tree's nodes, -1 if not in LDS
};

// Element value as float (bf16 or fp32 storage).
template <bool BF16>
__device__ __forceinline__ float elem_at(const void* row, long long i) {
  return BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(row)[i]) : static_cast<const float*>(row)[i];
}

// Calls f(i, x) for every element i of [e0, e1): scalars before and after the
// 16-byte aligned part, then the aligned vectors kSliceVec per thread at a
// time (all loads of a round issued before any is used).
template <bool BF16, typename F>
__device__ __forceinline__ void for_slice(const void* row, long long e0, long long e1, F f) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  const int tid = threadIdx.x;
  const uintptr_t base = reinterpret_cast<uintptr_t>(row);
  long long a = e0;
  while (a < e1 && ((base + (uintptr_t)a * ESZ) & 15u)) ++a;
  const long long nv = (e1 - a) / VEC;
  const long long b = a + nv * VEC;
  for (long long i = e0 + tid; i < a; i += kWalkThreads) f(i, elem_at<BF16>(row, i));
  for (long long i = b + tid; i < e1; i += kWalkThreads) f(i, elem_at<BF16>(row, i));
  if (nv <= 0) return;
  const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + a * ESZ);
  for (long long q0 = 0; q0 < nv; q0 += kSliceVec * kWalkThreads) {
    u32x4 v[kSliceVec];
#pragma unroll
    for (int u = 0; u < kSliceVec; ++u) {
      long long q = q0 + u * kWalkThreads + tid;
      q = q < nv ? q : nv - 1;  // clamped; only q < nv is used
      v[u] = __builtin_nontemporal_load(vp + q);
    }
#pragma unroll
    for (int u = 0; u < kSliceVec; ++u) {
      const long long q = q0 + u * kWalkThreads + tid;
      if (q < nv) {
        const long long i0 = a + q * VEC;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const uint32_t w = v[u][BF16 ? (j >> 1) : j];
          const float x = BF16 ? __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w);
          f(i0 + j, x);
        }
      }
    }
  }
}

// Element range [e0, e1) of slice s of S of a row: the row's aligned vectors
// are split evenly; slice 0 also takes the unaligned head, slice S-1 the tail.
template <bool BF16>
__device__ __forceinline__ void slice_range(const void* row, long long V, int S, int s, long long& e0,
                                            long long& e1) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(row) & 15u;
  long long a = mis ? (long long)((16u - mis) / ESZ) : 0;
  if (a > V) a = V;
  const long long nv = (V - a) / VEC;
  e0 = s == 0 ? 0 : a + (nv * s / S) * VEC;
  e1 = s == S - 1 ? V : a + (nv * (s + 1) / S) * VEC;
}

// Philox block of element i (four words per counter), cached across calls.
struct NoiseCache {
  long long blk = -1;
  Philox4 r;
  __device__ __forceinline__ uint64_t word(long long i, uint64_t seed, int d) {
    const long long bk = i >> 2;
    if (bk != blk) {
      r = philox4x64_10((uint64_t)bk, (uint64_t)d, 0, 0, seed, 0);
      blk = bk;
    }
    return lane_word(r, (int)(i & 3));
  }
};

// Block-wide Top2 of the per-thread values (barriers inside); every thread gets it.
__device__ __forceinline__ Top2 block_top2(Top2 t, WalkShared& sh) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) top2_merge(t, top2_shfl_xor(t, o));
  if (lane_id() == 0) sh.w[wave_id()] = t;
  __syncthreads();
  Top2 r = sh.w[0];
  for (int w = 1; w < kWalkWaves; ++w) top2_merge(r, sh.w[w]);
  __syncthreads();  // sh.w may be reused
  return r;
}

// Opens round 0 (the root) of every tree with a valid temperature and ends
// the others; clears the per-round counters.
__global__ void walk_init_kernel(WalkArgs a) {
  const int N = a.N, Lp1 = a.L + 1;
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x, stride = gridDim.x * blockDim.x;
  for (int i = i0; i < N * kMaxRounds; i += stride) a.done[i] = 0;
  for (int n = i0; n < N; n += stride) {
    const float T = a.temperature[n];
    a.cut[n] = 0.0;
    if (!(T >= 0.f) || isinf(T)) {
      for (int i = 0; i < Lp1; ++i) {
        a.out_tokens[(size_t)n * Lp1 + i] = -1;
        a.path_nodes[(size_t)n * Lp1 + i] = -1;
      }
      a.tau[n] = 0;
      if (a.status) atomicOr(&a.status[n], MFD_TREE_BAD_TEMPERATURE);
      a.word[n] = kEnded;
    } else {
      a.word[n] = round_word(0, 0, 0, 0);
    }
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kWalkThreads, 4) verify_walk_kernel(WalkArgs a) {
  __shared__ WalkShared sh;
  __shared__ int32_t lpar[kNodesLds];
  __shared__ int32_t ltok[kNodesLds];
  const int tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const int N = a.N, S = a.S, G = a.G, L = a.L, Lp1 = L + 1, Bp1 = a.Bp1;
  const long long V = a.V;
  const size_t esz = BF16 ? 2 : 4;
  const int grp = blockIdx.x / S, s = blockIdx.x - grp * S;
  // served trees: n = grp + j * G
  const int served = grp < N ? (N - 1 - grp) / G + 1 : 0;
  if (tid < kMaxServed) sh.seen[tid] = 0;
  if (tid == 0) {
    int slot = 0;
    for (int j = 0; j < served; ++j) {
      const int n = grp + j * G;
      int nn = a.n_nodes[n];
      nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
      sh.node0[j] = slot + nn <= kNodesLds ? slot : -1;
      if (slot + nn <= kNodesLds) slot += nn;
    }
  }
  __syncthreads();
  for (int j = 0; j < served; ++j) {
    const int o = sh.node0[j];
    if (o < 0) continue;
    const int n = grp + j * G;
    int nn = a.n_nodes[n];
    nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
    for (int q = tid; q < nn; q += kWalkThreads) {
      lpar[o + q] = a.parent[(size_t)n * Bp1 + q];
      ltok[o + q] = a.node_token[(size_t)n * Bp1 + q];
    }
  }
  long long idle = 0;
  int backoff = 1;

  while (true) {
    __syncthreads();  // everyone is done with the previous iteration's shared fields
    // ------------------------------------------------ find an open round (wave 0)
    if (wid == 0) {
      int quit = 0, pick = -1;
      uint32_t w = kEnded;
      if (lane < served) w = ld(&a.word[grp + lane * G]);
      const bool ended = w == kEnded;
      const bool ready = !ended && w != 0u && (int)(w & 0x7Fu) > sh.seen[lane < kMaxServed ? lane : 0];
      const uint64_t rm = __ballot(lane < served && ready);
      if (rm != 0ull) {
        pick = __builtin_ctzll(rm);
        backoff = 1;
        idle = 0;
      } else if (__ballot(lane < served && !ended) == 0ull) {
        quit = 1;  // every served tree has ended
      } else if (++idle > kIdleLimit) {
        quit = 2;
      } else {
        // back off while nothing is ready (up to ~1 us between polls)
        backoff = backoff < 16 ? backoff * 2 : 16;
        for (int z = 0; z < backoff; ++z) __builtin_amdgcn_s_sleep(kPollSleep);
      }
      w = __shfl(w, pick < 0 ? 0 : pick, kWave);
      if (lane == 0) {
        sh.quit = quit;
        sh.j = pick;
        sh.word = w;
        sh.child = 0x7FFFFFFF;
        if (pick >= 0 && ((w >> 7) & 1u)) {
          drain();  // the word was read before the cut-off it announces
          sh.cut = ld(&a.cut[grp + pick * G]);
        }
      }
    }
    __syncthreads();
    const int quit = sh.quit, j = sh.j;
    if (quit) {
      if (quit == 2 && tid == 0) {
        // gave up waiting: flag every served tree that has not ended
        for (int q = 0; q < served; ++q) {
          const int n = grp + q * G;
          if (ld(&a.word[n]) != kEnded) {
            if (a.status) atomicOr(&a.status[n], MFD_TREE_CAPACITY);
            a.tau[n] = 0;
          }
        }
      }
      break;
    }
    if (j < 0) continue;
    const uint32_t word = sh.word;
    const int r = (int)(word & 0x7Fu) - 1, kind = (int)((word >> 7) & 1u), step = (int)((word >> 8) & 0x3Fu),
              u = (int)(word >> 14);
    const double cut = sh.cut;
    const int n = grp + j * G;
    if (tid == 0) sh.seen[j] = r + 1;

    // ------------------------------------------------ reduce this workgroup's slice
    const size_t tb = (size_t)n * Bp1;
    const double T = (double)a.temperature[n];
    const double invT = T > 0.0 ? 1.0 / T : 0.0;
    const uint64_t sd = a.seed[n];
    const int d = a.depth[tb + u];
    const void* row = static_cast<const char*>(a.target) + ((tb + u) * (size_t)V) * esz;
    long long e0, e1;
    slice_range<BF16>(row, V, S, s, e0, e1);
    Top2 t = {-INFINITY, 0x7FFFFFFF, -INFINITY};
    NoiseCache nc;
    if (T == 0.0) {
      for_slice<BF16>(row, e0, e1, [&](long long i, float x) { top2_add(t, (double)x, (int)i); });
    } else if (kind == 0) {
      for_slice<BF16>(row, e0, e1, [&](long long i, float x) {
        const float g = gumbel_estimate(nc.word(i, sd, d));
        top2_add(t, (double)x * invT + (double)g, (int)i);
      });
    } else {
      // exact fp64 noise for every element whose estimate comes within the
      // slack of the best estimate
      for_slice<BF16>(row, e0, e1, [&](long long i, float x) {
        const uint64_t w = nc.word(i, sd, d);
        if ((double)x * invT + (double)gumbel_estimate(w) >= cut)
          top2_add(t, (double)x / T + gumbel_from_word(w), (int)i);
      });
    }
    const Top2 mine = block_top2(t, sh);
    double* py1 = a.py1 + (size_t)n * kSlices;
    double* py2 = a.py2 + (size_t)n * kSlices;
    int32_t* pi = a.pi + (size_t)n * kSlices;
    int32_t* done = a.done + (size_t)n * kMaxRounds + r;
    if (tid == 0) {
      st(&py1[s], mine.y1);
      st(&py2[s], mine.y2);
      st(&pi[s], mine.i1);
      drain();  // the result is in place before the slice counts as done
      const int old = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      drain();  // the count is in before the merge below reads the other slices' results
      sh.last = old == S - 1;
    }
    __syncthreads();
    if (!sh.last) continue;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    // ------------------------------------------------ finish the round
    if (wid == 0) {
      // every slice stored its result before counting itself done, and the
      // count has reached S: the S results are in place
      Top2 g = {-INFINITY, 0x7FFFFFFF, -INFINITY};
      for (int q = lane; q < S; q += kWave) {
        Top2 o;
        o.y1 = ld(&py1[q]);
        o.y2 = ld(&py2[q]);
        o.i1 = ld(&pi[q]);
        top2_merge(g, o);
      }
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) top2_merge(g, top2_shfl_xor(g, o));
      if (lane == 0) sh.g = g;
    }
    __syncthreads();
    const Top2 g = sh.g;
    // the estimates also carry the rounding of x / T (a few ulp of |y|)
    const double slack = 2.0 * kGumbelTol + (fabs(g.y1) + fabs(g.y2)) * 0x1.0p-48;
    if (T != 0.0 && kind == 0 && !(g.y1 - g.y2 > slack) && r + 1 < kMaxRounds) {
      // too close to call from the estimates: the same row once more, exactly
      if (tid == 0) {
        st(&a.cut[n], g.y1 - slack);
        drain();
        st(&a.word[n], round_word(r + 1, 1, step, u));
      }
      continue;
    }
    const int tstar = g.i1 == 0x7FFFFFFF ? 0 : g.i1;
    int nn = a.n_nodes[n];
    nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
    const int o = sh.node0[j];
    if (o >= 0) {
      for (int q = 1 + tid; q < nn; q += kWalkThreads)
        if (lpar[o + q] == u && ltok[o + q] == tstar) atomicMin(&sh.child, q);
    } else {
      for (int q = 1 + tid; q < nn; q += kWalkThreads)
        if (a.parent[tb + q] == u && a.node_token[tb + q] == tstar) atomicMin(&sh.child, q);
    }
    __syncthreads();
    const int child = sh.child;
    int32_t* ot = a.out_tokens + (size_t)n * Lp1;
    int32_t* pn = a.path_nodes + (size_t)n * Lp1;
    if (child != 0x7FFFFFFF && step < L && r + 1 < kMaxRounds) {
      if (tid == 0) {
        ot[step] = tstar;
        pn[step] = u;
        st(&a.word[n], round_word(r + 1, 0, step + 1, child));
      }
    } else {
      for (int i = step + 1 + tid; i < Lp1; i += kWalkThreads) {
        ot[i] = -1;
        pn[i] = -1;
      }
      if (tid == 0) {
        ot[step] = tstar;
        pn[step] = u;
        a.tau[n] = d + 1;
        st(&a.word[n], kEnded);
      }
    }
  }
}

template <size_t A>
constexpr size_t round_up(size_t x) {
  return (x + A - 1) / A * A;
}

struct WalkWsLayout {
  size_t word, cut, done, py1, py2, pi, total;
};

WalkWsLayout walk_ws_layout(int N) {
  WalkWsLayout w;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = round_up<128>(o + bytes);
    return r;
  };
  w.word = take((size_t)N * sizeof(uint32_t));
  w.cut = take((size_t)N * sizeof(double));
  w.done = take((size_t)N * kMaxRounds * sizeof(int32_t));
  w.py1 = take((size_t)N * kSlices * sizeof(double));
  w.py2 = take((size_t)N * kSlices * sizeof(double));
  w.pi = take((size_t)N * kSlices * sizeof(int32_t));
  w.total = o + 128;  // room to align the base
  return w;
}

}  // namespace

size_t walk_ws_bytes(int N) { return walk_ws_layout(N).total; }

hipError_t launch_verify_walk(const void* target, bool bf16, int N, int Bp1, long long V, int L,
                              const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                              const int32_t* n_nodes, const float* temperature, const uint64_t* seed, int32_t* tau,
                              int32_t* out_tokens, int32_t* path_nodes, int32_t* status, void* ws,
                              hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const void* fn = bf16 ? reinterpret_cast<const void*>(&verify_walk_kernel<true>)
                        : reinterpret_cast<const void*>(&verify_walk_kernel<false>);
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kWalkThreads, 0);
  if (e != hipSuccess) return e;
  long long resident = (long long)cus * (per_cu < 1 ? 1 : per_cu);
  // slices per row: about kSliceVec vectors per thread, at most kSlices and
  // at most the resident workgroups
  const long long nvec = V / (bf16 ? 8 : 4);
  long long S = (nvec + (long long)kSliceVec * kWalkThreads - 1) / ((long long)kSliceVec * kWalkThreads);
  if (S > kSlices) S = kSlices;
  if (S > resident) S = resident;
  if (S < 1) S = 1;
  // groups: as many as fit and at most one per tree; each group serves at
  // most kMaxServed trees, so a larger batch is walked in several launches
  long long Gmax = resident / S;
  if (Gmax < 1) Gmax = 1;
  const long long per_launch = Gmax * kMaxServed;

  const WalkWsLayout l = walk_ws_layout(N);
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 127) & ~uintptr_t(127));
  for (long long n0 = 0; n0 < N; n0 += per_launch) {
    const int nb = (int)(N - n0 < per_launch ? N - n0 : per_launch);
    long long G = Gmax < nb ? Gmax : nb;
    WalkArgs a;
    a.target = static_cast<const char*>(target) + (size_t)n0 * Bp1 * V * (bf16 ? 2 : 4);
    a.N = nb;
    a.Bp1 = Bp1;
    a.L = L;
    a.S = (int)S;
    a.G = (int)G;
    a.V = V;
    a.node_token = node_token + (size_t)n0 * Bp1;
    a.parent = parent + (size_t)n0 * Bp1;
    a.depth = depth + (size_t)n0 * Bp1;
    a.n_nodes = n_nodes + n0;
    a.temperature = temperature + n0;
    a.seed = seed + n0;
    a.tau = tau + n0;
    a.out_tokens = out_tokens + (size_t)n0 * (L + 1);
    a.path_nodes = path_nodes + (size_t)n0 * (L + 1);
    a.status = status ? status + n0 : nullptr;
    a.word = reinterpret_cast<uint32_t*>(w + l.word) + n0;
    a.cut = reinterpret_cast<double*>(w + l.cut) + n0;
    a.done = reinterpret_cast<int32_t*>(w + l.done) + (size_t)n0 * kMaxRounds;
    a.py1 = reinterpret_cast<double*>(w + l.py1) + (size_t)n0 * kSlices;
    a.py2 = reinterpret_cast<double*>(w + l.py2) + (size_t)n0 * kSlices;
    a.pi = reinterpret_cast<int32_t*>(w + l.pi) + (size_t)n0 * kSlices;
    hipLaunchKernelGGL(walk_init_kernel, dim3((nb * kMaxRounds + 255) / 256), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    void* args[] = {&a};
    e = hipLaunchCooperativeKernel(fn, dim3((unsigned)(G * S)), dim3(kWalkThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mfd
