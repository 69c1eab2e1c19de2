// Tree-verification walk over the target's per-node logits.
//
// The target keeps the future it actually takes (project page, "How it works"
// step 3): starting at the root, take the target's token at the current node
// and move to the child holding that token while one exists.  The accepted
// drafted tokens plus the last (bonus) token give tau = depth + 1 (project
// page, Figure 2: six drafted tokens plus the bonus).  At T = 0 the token is
// the argmax; at T > 0 it is a Gumbel-max sample, which draws exactly from
// softmax(R / T), so decoding stays lossless (model card summary).  The noise
// is counter-based (Philox4x32-10, one 32-bit word per token) and keyed by
// (seed, depth, token), so a given seed samples the same tokens whatever the
// tree's shape.
//
// Work layout: the token chosen at a node depends only on that node's row,
// T, the seed and its depth, so the only order the walk imposes is one row
// after the other within a tree.  Every row is cut into S slices, and a round
// is one row (or its exact re-evaluation, below) of one tree; the hand-off
// between the workgroups of a tree is described at verify_walk_kernel.  Only
// the rows on the walked path are read (or, with the speculative pass below,
// every row of a small batch at once).
//
// At T > 0 the first pass over a row works in fp32: the noise estimate
// (two v_log_f32, error below 2e-5, see gumbel_estimate) and
// est = fma(x, fp32(1 / T), g), which lies within est_err(y) of the exact
// y = x / T + g (fp64).  Each round keeps the best estimate and the second
// best value.  When they are further apart than est_slack the best one is the
// exact winner; otherwise a second round evaluates the exact fp64 noise for
// every element whose estimate comes that close to the best, and takes the
// exact maximum.
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
constexpr size_t kWalkScratchBytes = size_t(16) << 20;
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
constexpr int kSlices = 64;                  // slices per row, at most (one lane each in the merge)
constexpr int kTreesPerGroup = 2;            // trees one group of workgroups serves at most
constexpr int kNodeLds = 512;                // nodes of a tree whose links a workgroup keeps in LDS
constexpr int kWalkVec = 2;                  // 16-byte vectors per thread in flight in the walk's slices (T > 0)
constexpr int kWalkVec0 = 8;                 // the same at T = 0 (a slice is then one round of loads)
// Waits, in s_memrealtime ticks (100 MHz): a workgroup that has seen no
// progress for kHelpTicks computes a missing slice itself; one that has seen
// none for kGiveUpTicks flags its trees and leaves (never in practice).
constexpr uint64_t kHelpTicks = 5000;            // 50 us
constexpr uint64_t kGiveUpTicks = 200000000ull;  // 2 s
constexpr int kPollSleep = 1;                    // s_sleep units (64 clocks each) between polls, doubled up to 8x
constexpr double kGumbelTol = 1e-4;
constexpr float kLn2f = 0.693147180559945309f;
constexpr int kSliceVec = 2;                 // 16-byte vectors per thread per round of loads
constexpr int kMaxB1 = 16384;                // rows per tree, at most (B <= 16383)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lane_word(const Philox4& r, int l) {
  return l == 0 ? r.v[0] : (l == 1 ? r.v[1] : (l == 2 ? r.v[2] : r.v[3]));
}

// (y, index) with larger y first, then lower index.
__device__ __forceinline__ bool better(double y, int i, double by, int bi) {
  return (y > by) || (y == by && i < bi);
}

// fp32 estimate of the noise g = -ln(-ln U), U = (w + 0.5) 2^-32.
// With t = -ln U:
//  * 1 - U < 2^-8 (m = 2^32 - w <= 2^24): u = 1 - U = (m - 0.5) 2^-32 is
//    formed with relative error <= 2^-24, and t ~ u (1 + u / 2), whose
//    truncation error is below u^2 / 3 <= 2^-16 / 3 relative;
//  * otherwise U is formed with relative error <= 2^-24, which moves ln U by
//    at most 2^-24, i.e. by at most 2^-24 / |ln U| <= 2^-16 relative to t
//    (|ln U| >= 2^-8 here); v_log_f32 adds about an ulp of its result.
// A relative error e of t moves g by about e, and the final v_log_f32 and
// scaling add about 1e-6, so |estimate - g| < 2e-5.
__device__ __forceinline__ float gumbel_estimate(uint32_t w) {
  const uint32_t m = 0u - w;  // 2^32 - w where it is used (w >= 0xFF000000)
  const float u = ((float)m - 0.5f) * 0x1.0p-32f;
  const float U = ((float)w + 0.5f) * 0x1.0p-32f;
  const float t_small = u * (1.f + 0.5f * u);
  const float t_big = -__builtin_amdgcn_logf(U) * kLn2f;
  const float t = w >= 0xFF000000u ? t_small : t_big;
  return -__builtin_amdgcn_logf(t) * kLn2f;
}

// est = fma(x, fp32(1 / T), estimate) against the exact y = x / T + g: the
// noise estimate is off by < 2e-5, fp32(1 / T) by 2^-24 relative (an error of
// |x / T| 2^-24 <= (|y| + 23) 2^-24, as |g| < 23 for 32-bit U), and the fma
// rounds by 2^-24 |est|; so |est - y| <= 3e-5 + |y| 2^-22 =: est_err(y).
// Two elements whose estimates are further apart than est_err of both are in
// the same order exactly; est_slack bounds est_err(a) + est_err(b) for values
// near the given ones, with room to spare.
__device__ __forceinline__ double est_slack(double y1, double y2) {
  return 2.0 * kGumbelTol + (fabs(y1) + fabs(y2) + 2.0) * 0x1.0p-20;
}

// A value the whole wave holds alike, moved to scalar registers (so that,
// e.g., the Philox key schedule runs on the scalar unit).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint64_t uni(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double uni(double x) { return __longlong_as_double((long long)uni((uint64_t)__double_as_longlong(x))); }

// Best (value, index) and the second best value seen, per thread, in fp32
// (the estimates and the T = 0 logits).
struct Top2f {
  float y1;
  int i1;
  float y2;
};

// (selects, not branches: a branch per element splits the slice loops into
// one basic block per element; a NaN y changes nothing)
__device__ __forceinline__ void top2f_add(Top2f& t, float y, int i) {
  const bool take = (y > t.y1) | ((y == t.y1) & (i < t.i1));
  const float y2 = take ? t.y1 : (y > t.y2 ? y : t.y2);
  t.y1 = take ? y : t.y1;
  t.i1 = take ? i : t.i1;
  t.y2 = y2;
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
  int groups;  // walk kernel: groups of S workgroups, each serving its own trees
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
  int R;           // rounds a tree may take: two per depth, 2 (L + 1)
  int esz;         // bytes per target element
  uint64_t* slot;  // [N][R][S][2]: each slice's result of each round (slot_pack)
  // speculation (walk_prep_kernel / walk_spec_kernel); spec = 0: none
  int spec;
  int spec_rcap;         // rows the slice-result arrays hold
  int32_t* spec_cnt;     // [N][4]: nodes with a child, all nodes (0 for an ended tree), expected rounds x16, T > 0
  int32_t* spec_go;      // [1]: the pass's route decided by the prep pass (one tree): 0 none, 1 nodes with a
                         // child, 2 every node; -1: decided by the pass itself
  uint16_t* spec_nodes;  // [N][Bp1]: the tree's nodes with a child, then its leaves
  int32_t* choice;       // [N][Bp1]: token chosen at each evaluated node, -1 if not evaluated
  int32_t* rowdone;      // [N][Bp1]: slices finished per listed row
  int32_t* treedone;     // [N]: rows finished per tree
  double* sy;            // [spec_rcap][S]: best exact value of each slice
  int32_t* si;           // [spec_rcap][S]: its token
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

// A slice's result as two 64-bit words, each written and read as one atomic
// access and each carrying a check pattern, so a reader that finds both
// patterns has the whole result with no ordering between the two stores
// (the prep pass zeroes the slots).  Word A: the high 32 bits of the value,
// the best index (20 bits; 0xFFFFF for none) and a 12-bit pattern; word B:
// the low 32 bits and a 32-bit pattern.  The value is the best fp32 estimate
// or logit (high) with the second best one (low) after a first pass, and the
// exact fp64 winner's value (high and low halves) after an exact pass.
constexpr uint64_t kSlotTagA = 0x5A5u;
constexpr uint64_t kSlotTagB = 0x5A5A5A5Au;
constexpr int kNoIndex20 = 0xFFFFF;

__device__ __forceinline__ void slot_pack(uint32_t hi, uint32_t lo, int i1, uint64_t& A, uint64_t& B) {
  const uint32_t i20 = (i1 < 0 || i1 >= kNoIndex20) ? (uint32_t)kNoIndex20 : (uint32_t)i1;
  A = ((uint64_t)hi << 32) | ((uint64_t)i20 << 12) | kSlotTagA;
  B = ((uint64_t)lo << 32) | kSlotTagB;
}

__device__ __forceinline__ bool slot_ok(uint64_t A, uint64_t B) {
  return (A & 0xFFFu) == kSlotTagA && (B & 0xFFFFFFFFu) == kSlotTagB;
}

// A tree's walk as one workgroup of its group sees it: every workgroup of
// the group merges every round itself, so all of them step through the same
// states.
struct WalkState {
  int r;           // current round
  int kind;        // 1: the exact re-evaluation of the previous round's row
  int step;        // moves from the root so far (the output position)
  int u;           // current node
  int ended;
  int mine;        // this workgroup's own slice of round r is done
  int d;           // depth of u (keys the noise)
  int nn;          // nodes of the tree
  uint64_t miss;   // slices of round r without a result at the last poll
  double cut;      // exact round: estimates below this cannot win
  double T;        // the tree's temperature
  uint64_t sd;     // and seed
};

struct WalkShared {
  Top2 w[kWalkWaves];
  WalkState ts[kTreesPerGroup];
  int complete[kTreesPerGroup];
  int tree[kTreesPerGroup];  // the group's trees (launch-local indices)
  int scan[kWalkWaves];
  int action, help_j, help_s;
  int32_t npar[kTreesPerGroup][kNodeLds];
  int32_t ntok[kTreesPerGroup][kNodeLds];
  int32_t ndep[kTreesPerGroup][kNodeLds];
};

// Element value as float (bf16 or fp32 storage).
template <bool BF16>
__device__ __forceinline__ float elem_at(const void* row, long long i) {
  return BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(row)[i]) : static_cast<const float*>(row)[i];
}

// Calls f(i, x) for every element i of [e0, e1): scalars before and after the
// 16-byte aligned part, then the aligned vectors kSliceVec per thread at a
// time (all loads of a round issued before any is used).
// Philox block of element i (four words per counter), cached across calls.
struct NoiseCache {
  long long blk = -1;
  Philox4 r;
  __device__ __forceinline__ uint32_t word(long long i, uint64_t seed, int d) {
    const long long bk = i >> 2;
    if (bk != blk) {
      r = philox4x32_10((uint32_t)bk, (uint32_t)d, 0, 0, (uint32_t)seed, (uint32_t)(seed >> 32));
      blk = bk;
    }
    return lane_word(r, (int)(i & 3));
  }
};

// As for_slice, but each aligned vector goes to fv(i0, x) whole (x[j] is
// element i0 + j), the scalars to f(i, x).
template <bool BF16, int VECS, typename F, typename FV>
__device__ __forceinline__ void for_slice_vec(const void* row, long long e0, long long e1, F f, FV fv) {
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
  for (long long q0 = 0; q0 < nv; q0 += VECS * kWalkThreads) {
    u32x4 v[VECS];
#pragma unroll
    for (int u = 0; u < VECS; ++u) {
      long long q = q0 + u * kWalkThreads + tid;
      q = q < nv ? q : nv - 1;  // clamped; only q < nv is used
      v[u] = __builtin_nontemporal_load(vp + q);
    }
#pragma unroll
    for (int u = 0; u < VECS; ++u) {
      const long long q = q0 + u * kWalkThreads + tid;
      if (q < nv) {
        float x[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const uint32_t w = v[u][BF16 ? (j >> 1) : j];
          x[j] = BF16 ? __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w);
        }
        fv(a + q * VEC, x);
      }
    }
  }
}

template <bool BF16, int VECS = kSliceVec, typename F>
__device__ __forceinline__ void for_slice(const void* row, long long e0, long long e1, F f) {
  constexpr int VEC = BF16 ? 8 : 4;
  for_slice_vec<BF16, VECS>(row, e0, e1, f, [&](long long i0, const float (&x)[VEC]) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) f(i0 + j, x[j]);
  });
}

// The fp32 first pass at T > 0 over [e0, e1): est = fma(x, invTf, noise
// estimate) into the per-thread top two.  A vector whose first element starts
// a Philox block (every vector, when the row's aligned part does) takes its
// blocks whole, with no per-element bookkeeping.
template <bool BF16, int VECS>
__device__ __forceinline__ void slice_estimates(const void* row, long long e0, long long e1, uint64_t sd, int d,
                                                float invTf, Top2f& f) {
  constexpr int VEC = BF16 ? 8 : 4;
  NoiseCache nc;
  const uint32_t k0 = (uint32_t)sd, k1 = (uint32_t)(sd >> 32);
  auto one = [&](long long i, float x) { top2f_add(f, fmaf(x, invTf, gumbel_estimate(nc.word(i, sd, d))), (int)i); };
  for_slice_vec<BF16, VECS>(row, e0, e1, one, [&](long long i0, const float (&x)[VEC]) {
    if ((i0 & 3) == 0) {
#pragma unroll
      for (int b = 0; b < VEC / 4; ++b) {
        const Philox4 r = philox4x32_10((uint32_t)(i0 >> 2) + b, (uint32_t)d, 0, 0, k0, k1);
#pragma unroll
        for (int j = 0; j < 4; ++j) top2f_add(f, fmaf(x[4 * b + j], invTf, gumbel_estimate(r.v[j])), (int)i0 + 4 * b + j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VEC; ++j) one(i0 + j, x[j]);
    }
  });
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


// Block-wide Top2 of the per-thread values (barriers inside); every thread gets it.
__device__ __forceinline__ Top2 block_top2(Top2 t, Top2* wsh) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) top2_merge(t, top2_shfl_xor(t, o));
  if (lane_id() == 0) wsh[wave_id()] = t;
  __syncthreads();
  Top2 r = wsh[0];
  for (int w = 1; w < kWalkWaves; ++w) top2_merge(r, wsh[w]);
  __syncthreads();  // wsh may be reused
  return r;
}

__device__ int spec_route(const WalkArgs& a, int N, int* scan);

// One workgroup per tree.  Opens round 0 (the root) of a tree with a valid
// temperature and ends the others; clears the per-round counters.  With
// speculation on, also lists the tree's nodes (those with a child first, in
// node order, then the leaves), marks every node's token as not yet chosen
// and clears the speculation counters.
__global__ void __launch_bounds__(kWalkThreads) walk_prep_kernel(WalkArgs a) {
  __shared__ unsigned char has_child[kMaxB1];
  __shared__ int scan[kWalkWaves];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int Lp1 = a.L + 1, Bp1 = a.Bp1;
  for (int i = tid; i < 2 * a.R * a.S; i += kWalkThreads) a.slot[(size_t)n * 2 * a.R * a.S + i] = 0;
  const float T = a.temperature[n];
  const bool bad = !(T >= 0.f) || isinf(T);
  if (bad) {
    for (int i = tid; i < Lp1; i += kWalkThreads) {
      a.out_tokens[(size_t)n * Lp1 + i] = -1;
      a.path_nodes[(size_t)n * Lp1 + i] = -1;
    }
  }
  if (tid == 0) {
    if (bad) {
      a.tau[n] = 0;
      if (a.status) atomicOr(&a.status[n], MFD_TREE_BAD_TEMPERATURE);
      a.word[n] = kEnded;
    } else {
      a.word[n] = round_word(0, 0, 0, 0);
    }
  }
  if (!a.spec) return;
  int nn = a.n_nodes[n];
  nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
  if (bad) nn = 0;
  const size_t tb = (size_t)n * Bp1;
  for (int u = tid; u < nn; u += kWalkThreads) {
    has_child[u] = 0;
    a.choice[tb + u] = -1;
    a.rowdone[tb + u] = 0;
  }
  if (tid == 0) a.treedone[n] = 0;
  __syncthreads();
  for (int v = 1 + tid; v < nn; v += kWalkThreads) {
    const int p = a.parent[tb + v];
    if (p >= 0 && p < nn) has_child[p] = 1;
  }
  __syncthreads();
  int local = 0, dmax = 0, dsum = 0;
  for (int u = tid; u < nn; u += kWalkThreads) {
    local += has_child[u];
    const int du = a.depth[tb + u];
    dmax = du > dmax ? du : dmax;
    dsum += du;
  }
  const int nint = block_sum<kWalkThreads>(local, scan);
  const int dtot = block_sum<kWalkThreads>(dsum, scan);
  // the deepest node, by a max over the waves (scan[] is free again)
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) dmax = max(dmax, __shfl_xor(dmax, o, kWave));
  if (lane_id() == 0) scan[wave_id()] = dmax;
  __syncthreads();
  for (int w = 0; w < kWalkWaves; ++w) dmax = max(dmax, scan[w]);
  __syncthreads();
  if (tid == 0) {
    a.spec_cnt[4 * n] = nint;
    a.spec_cnt[4 * n + 1] = nn;
    // rounds the row-by-row walk is expected to take, x16: one more than
    // the mean of the nodes' mean depth and the deepest depth (the walk stops
    // at the first token the tree lacks, usually well short of its deepest
    // node in a bushy tree, near it in a chain)
    a.spec_cnt[4 * n + 2] = nn > 1 ? 16 + (int)((8ll * dtot) / (nn - 1)) + 8 * dmax : (nn > 0 ? 16 : 0);
    a.spec_cnt[4 * n + 3] = T > 0.f ? 1 : 0;
  }
  // one tree: this workgroup has every count the route needs, so it decides
  // here, the speculative pass's workgroups just read the answer, and the
  // node lists are only made when the pass runs
  if (a.N == 1) {
    __syncthreads();  // the counts above are in place
    const int route = spec_route(a, 1, scan);
    if (tid == 0) a.spec_go[0] = route + 2;
    if (route < 0) return;
  } else if (n == 0 && tid == 0) {
    a.spec_go[0] = 0;
  }
  int carry = 0;
  for (int base = 0; base < nn; base += kWalkThreads) {
    const int u = base + tid;
    const int h = u < nn ? has_child[u] : 0;
    int tot;
    const int ex = block_exclusive_scan<kWalkThreads>(h, scan, &tot);
    if (u < nn) {
      const int before = carry + ex;  // nodes with a child before u
      a.spec_nodes[tb + (h ? before : nint + (u - before))] = (uint16_t)u;
    }
    carry += tot;
  }
}

// ---------------------------------------------------------------- speculation
// The token chosen at a node depends only on the node's own row, T, the seed
// and the node's depth, not on the path that leads there.  So when the rows
// are few enough to read in one pass, every resident workgroup reduces them
// in parallel before the walk: every node's row (a small batch), or the rows
// of the nodes that have a child when those alone fit.  The tree is then
// walked from the root along the chosen tokens at once.  What remains -- the
// last node's row, when it is a leaf that was not evaluated -- is one round
// of verify_walk_kernel; when neither budget holds, that kernel does all of it.
//
// Each slice of a row gives its exact winner in one pass.  At T = 0 that is
// the largest logit (lowest id among equals).  At T > 0 every element gets the
// fp32 estimate est(v), within e(v) = est_err(y(v)) of the exact y(v).  Let w
// be the slice's exact winner and b the element of the best estimate g:
// est(w) >= y(w) - e(w) >= y(b) - e(w) >= g - e(b) - e(w).  So w is among the
// elements whose estimate is within est_slack(g, g) of g, and evaluating just
// those exactly in fp64 finds it; the row's winner is the best of its slices'
// winners.
constexpr long long kSpecAllBytes = 160ll << 20;  // every node's row, up to this many bytes per launch
constexpr long long kSpecIntBytes = 400ll << 20;  // else the rows of nodes with a child, up to this many
constexpr int kFollowLds = 2048;                  // nodes of a tree the follow step copies to LDS
constexpr int kSpecVec = 8;                       // 16-byte vectors per thread in flight in the speculative pass
// Cost estimates behind the choice between speculation and the row-by-row
// walk, measured on MI355X at V = 151936 (one tree, graph replays): a
// dependent round of the walk (8 us: 27.8 us for a 2-round walk, 108 us for
// 12 rounds), the speculative pass's fixed cost over the row-by-row walk's
// (its launch and hand-offs; 34.4 against 27.8 us on a 2-round tree whose
// interior rows take ~2 us to read), its reading rate, and the noise cost of
// one T > 0 element (Philox4x32-10 and the estimate, ~1000 G elements/s)
// spread over the whole chip.
constexpr double kRoundUs = 8.0;
constexpr double kSpecFixedUs = 25.0;
constexpr double kSpecBytesPerUs = 2.0e6;
constexpr double kNoiseUsPerElement = 1.0e-6;
constexpr int kSpecLaunchTrees = 4;  // the pass is only tried for launches of at most this many trees
constexpr int kSpecMaxTrees = 64;    // trees per launch the pass can handle (its LDS prefix array)
static_assert(kSpecLaunchTrees <= kSpecMaxTrees, "speculation prefix array too small");

// (y, i) with larger y first, then lower i, over the workgroup; every thread gets it.
struct BestYI {
  double y;
  int i;
};

__device__ __forceinline__ BestYI block_best(BestYI b, BestYI* wsh) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const double y = __shfl_xor(b.y, o, kWave);
    const int i = __shfl_xor(b.i, o, kWave);
    if (better(y, i, b.y, b.i)) {
      b.y = y;
      b.i = i;
    }
  }
  if (lane_id() == 0) wsh[wave_id()] = b;
  __syncthreads();
  BestYI r = wsh[0];
  for (int w = 1; w < kWalkWaves; ++w)
    if (better(wsh[w].y, wsh[w].i, r.y, r.i)) r = wsh[w];
  __syncthreads();
  return r;
}

// The exact winner of slice [e0, e1) of a row (see above).
template <bool BF16>
__device__ BestYI spec_slice(const void* row, long long e0, long long e1, double T, uint64_t sd, int d,
                             BestYI* wsh) {
  if (T == 0.0) {
    BestYI b = {-INFINITY, 0x7FFFFFFF};
    for_slice<BF16, kSpecVec>(row, e0, e1, [&](long long i, float x) {
      if (better((double)x, (int)i, b.y, b.i)) {
        b.y = (double)x;
        b.i = (int)i;
      }
    });
    return block_best(b, wsh);
  }
  const float invTf = (float)(1.0 / T);
  // each thread: its two best estimates (value, id, logit) and the third best value
  float e1v = -INFINITY, e2v = -INFINITY, e3v = -INFINITY;
  int i1 = 0x7FFFFFFF, i2 = 0x7FFFFFFF;
  float x1 = 0.f, x2 = 0.f;
  NoiseCache nc;
  for_slice<BF16, kSpecVec>(row, e0, e1, [&](long long i, float x) {
    const float est = fmaf(x, invTf, gumbel_estimate(nc.word(i, sd, d)));
    if (est > e1v || (est == e1v && (int)i < i1)) {
      e3v = e2v;
      e2v = e1v;
      i2 = i1;
      x2 = x1;
      e1v = est;
      i1 = (int)i;
      x1 = x;
    } else if (est > e2v || (est == e2v && (int)i < i2)) {
      e3v = e2v;
      e2v = est;
      i2 = (int)i;
      x2 = x;
    } else if (est > e3v) {
      e3v = est;
    }
  });
  BestYI g = block_best(BestYI{(double)e1v, i1}, wsh);
  const double lim = g.y - est_slack(g.y, g.y);
  BestYI b = {-INFINITY, 0x7FFFFFFF};
  auto exact = [&](long long i, float x) {
    const uint32_t w = nc.word(i, sd, d);
    const double y = (double)x / T + gumbel_from_word(w);
    if (better(y, (int)i, b.y, b.i)) {
      b.y = y;
      b.i = (int)i;
    }
  };
  if (e3v >= lim) {
    // three or more of this thread's elements are close to the slice's best
    // (rare): go over its elements again
    for_slice<BF16, kSpecVec>(row, e0, e1, [&](long long i, float x) {
      if ((double)fmaf(x, invTf, gumbel_estimate(nc.word(i, sd, d))) >= lim) exact(i, x);
    });
  } else {
    if (i1 != 0x7FFFFFFF && (double)e1v >= lim) exact(i1, x1);
    if (i2 != 0x7FFFFFFF && (double)e2v >= lim) exact(i2, x2);
  }
  return block_best(b, wsh);
}

// The speculative pass's route for the launch's N trees (their counts in
// spec_cnt): 1 every node's row, 0 the rows of the nodes with a child, -1 no
// pass.  Rows under each budget, and an estimate of each route's time.  Row
// by row, the walk takes one dependent round per move of its longest walk,
// estimated per tree by the prep pass (trees share groups of workgroups
// beyond G).  Speculation reads the rows at once, pays the noise of every
// T > 0 row, and leaves one round for the trees that end at an unevaluated
// leaf.  Either route gives the same tokens; this only picks the faster one.
// Every thread of the block calls it (barriers inside); all get the result.
__device__ int spec_route(const WalkArgs& a, int N, int* scan) {
  const int tid = threadIdx.x;
  const int S = a.S;
  const long long V = a.V;
  const size_t esz = (size_t)a.esz;
  int loc_int = 0, loc_all = 0, loc_int_hot = 0, loc_all_hot = 0, loc_d = 0;
  for (int n = tid; n < N; n += kWalkThreads) {
    const int ni = a.spec_cnt[4 * n], na = a.spec_cnt[4 * n + 1], hot = a.spec_cnt[4 * n + 3];
    loc_int += ni;
    loc_all += na;
    loc_int_hot += hot ? ni : 0;
    loc_all_hot += hot ? na : 0;
    loc_d = max(loc_d, a.spec_cnt[4 * n + 2]);
  }
  const long long tot_int = block_sum<kWalkThreads>(loc_int, scan);
  const long long tot_all = block_sum<kWalkThreads>(loc_all, scan);
  const long long hot_int = block_sum<kWalkThreads>(loc_int_hot, scan);
  const long long hot_all = block_sum<kWalkThreads>(loc_all_hot, scan);
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) loc_d = max(loc_d, __shfl_xor(loc_d, o, kWave));
  if (lane_id() == 0) scan[wave_id()] = loc_d;
  __syncthreads();
  int dmax = 0;
  for (int w = 0; w < kWalkWaves; ++w) dmax = max(dmax, scan[w]);
  __syncthreads();
  const long long row_bytes = V * (long long)esz;
  const double sharing = (double)(((long long)N * S + a.G - 1) / a.G);  // rounds open at once per workgroup
  const double t_rows = (dmax / 16.0) * kRoundUs * sharing;  // dmax: the largest expected rounds x16
  auto t_spec = [&](long long rows, long long hot) {
    return kSpecFixedUs + (double)rows * row_bytes / kSpecBytesPerUs + (double)hot * V * kNoiseUsPerElement;
  };
  const double t_all = t_spec(tot_all, hot_all);
  const double t_int = t_spec(tot_int, hot_int) + kRoundUs * sharing;
  const bool ok_all = tot_all <= a.spec_rcap && tot_all * row_bytes <= kSpecAllBytes && t_all < t_rows;
  const bool ok_int = tot_int <= a.spec_rcap && tot_int * row_bytes <= kSpecIntBytes && t_int < t_rows;
  if (ok_all && (!ok_int || t_all <= t_int)) return 1;
  if (ok_int) return 0;
  return -1;
}

template <bool BF16>
__global__ void __launch_bounds__(kWalkThreads, 4) walk_spec_kernel(WalkArgs a) {
  __shared__ int pre[kSpecMaxTrees + 1];
  __shared__ int scan[kWalkWaves];
  __shared__ BestYI wsh[kWalkWaves];
  __shared__ int sh_row, sh_tree;  // separate flags: see the barriers
  __shared__ int32_t fpar[kFollowLds], ftok[kFollowLds], fch[kFollowLds];
  const int tid = threadIdx.x;
  const int N = a.N, S = a.S, Bp1 = a.Bp1, L = a.L, Lp1 = L + 1;
  const long long V = a.V;
  const size_t esz = BF16 ? 2 : 4;
  // the route: decided by the prep pass for one tree (a previous launch;
  // spec_go = route + 2), else here
  const int go = a.spec_go[0];
  const int which = go > 0 ? go - 2 : spec_route(a, N, scan);
  if (which < 0) return;
  // prefix of the chosen row counts over the trees
  int carry = 0;
  for (int base = 0; base < N; base += kWalkThreads) {
    const int n = base + tid;
    const int c = n < N ? a.spec_cnt[4 * n + which] : 0;
    int tot;
    const int ex = block_exclusive_scan<kWalkThreads>(c, scan, &tot);
    if (n < N) pre[n] = carry + ex;
    carry += tot;
  }
  if (tid == 0) pre[N] = carry;
  __syncthreads();
  // slices per row for this pass: about one (row, slice) item per workgroup,
  // at most the walk's slice count (the result arrays' row stride stays S)
  int S2 = carry > 0 ? (int)((gridDim.x + carry - 1) / carry) : 1;
  if (S2 > S) S2 = S;
  if (S2 < 1) S2 = 1;
  const long long items = (long long)carry * S2;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int r = (int)(it / S2), s = (int)(it - (long long)r * S2);
    int lo = 0, hi = N - 1;  // the tree of row r: the last n with pre[n] <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= r) lo = mid;
      else hi = mid - 1;
    }
    const int n = lo, j = r - pre[n];
    const size_t tb = (size_t)n * Bp1;
    const int u = a.spec_nodes[tb + j];
    const double T = (double)a.temperature[n];
    const void* row = static_cast<const char*>(a.target) + ((tb + u) * (size_t)V) * esz;
    long long e0, e1;
    slice_range<BF16>(row, V, S2, s, e0, e1);
    const BestYI b = spec_slice<BF16>(row, e0, e1, T, a.seed[n], a.depth[tb + u], wsh);
    if (tid == 0) {
      st(&a.sy[(size_t)r * S + s], b.y);
      st(&a.si[(size_t)r * S + s], b.i);
      drain();  // the slice's result is in place before it counts as done
      const int old = __hip_atomic_fetch_add(&a.rowdone[tb + j], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      drain();
      sh_row = old == S2 - 1;
    }
    __syncthreads();
    if (!sh_row) continue;  // uniform: read after the barrier, rewritten only after the next iteration's
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // the row's last slice: merge the S slice winners
    if (tid < kWave) {
      BestYI m = {-INFINITY, 0x7FFFFFFF};
      for (int q = tid; q < S2; q += kWave) {
        const double y = ld(&a.sy[(size_t)r * S + q]);
        const int i = ld(&a.si[(size_t)r * S + q]);
        if (better(y, i, m.y, m.i)) {
          m.y = y;
          m.i = i;
        }
      }
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const double y = __shfl_xor(m.y, o, kWave);
        const int i = __shfl_xor(m.i, o, kWave);
        if (better(y, i, m.y, m.i)) {
          m.y = y;
          m.i = i;
        }
      }
      if (tid == 0) {
        st(&a.choice[tb + u], m.i == 0x7FFFFFFF ? 0 : m.i);
        drain();  // the choice is in place before the row counts as done
        const int old = __hip_atomic_fetch_add(&a.treedone[n], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        drain();
        sh_tree = old == a.spec_cnt[4 * n + which] - 1;
      }
    }
    __syncthreads();
    if (!sh_tree) continue;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // the tree's last row: follow the chosen tokens from the root (wave 0,
    // with the tree's links and choices copied to LDS when they fit)
    if (tid < kWave) {
      const int lane = tid;
      int nn = a.n_nodes[n];
      nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
      const bool in_lds = nn <= kFollowLds;
      if (in_lds) {
        for (int q = lane; q < nn; q += kWave) {
          fpar[q] = a.parent[tb + q];
          ftok[q] = a.node_token[tb + q];
          fch[q] = ld(&a.choice[tb + q]);
        }
      }
      wave_sync();
      int32_t* ot = a.out_tokens + (size_t)n * Lp1;
      int32_t* pn = a.path_nodes + (size_t)n * Lp1;
      int cur = 0, step = 0;
      while (true) {
        const int t = in_lds ? fch[cur] : ld(&a.choice[tb + cur]);
        if (t < 0) {
          // not evaluated (a leaf, when only nodes with a child were): the
          // walk kernel reduces this row in its first round
          if (lane == 0) st(&a.word[n], round_word(0, 0, step, cur));
          break;
        }
        int child = 0x7FFFFFFF;
        for (int q = 1 + lane; q < nn; q += kWave) {
          const int p = in_lds ? fpar[q] : a.parent[tb + q];
          const int tk = in_lds ? ftok[q] : a.node_token[tb + q];
          if (p == cur && tk == t) {
            child = q;
            break;
          }
        }
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) child = min(child, __shfl_xor(child, o, kWave));
        if (child != 0x7FFFFFFF && step < L) {
          if (lane == 0) {
            ot[step] = t;
            pn[step] = cur;
          }
          ++step;
          cur = child;
          continue;
        }
        for (int i = step + 1 + lane; i < Lp1; i += kWave) {
          ot[i] = -1;
          pn[i] = -1;
        }
        if (lane == 0) {
          ot[step] = t;
          pn[step] = cur;
          a.tau[n] = a.depth[tb + cur] + 1;
          st(&a.word[n], kEnded);
        }
        break;
      }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ uint64_t rotr64(uint64_t m, int r) { return r ? ((m >> r) | (m << (64 - r))) : m; }

// The walk proper.  A round is one row of one tree (or its exact
// re-evaluation), cut into S slices.  The launch's workgroups form groups of
// S; group q serves trees q, q + groups, ... (at most kTreesPerGroup).
// Workgroup m of a group reduces slice m of each round of its trees and
// stores the result in that round's own slot (two self-checking words, see
// slot_pack).  Every workgroup of the group polls the round's S slots and,
// once all hold a result, merges them itself in one fixed order, so each one
// finds the same winner and the same child and goes on to the next round
// with no further hand-off: per round, one store per slice and one poll per
// reader, and no read-modify-write.
//
// No workgroup relies on another being resident.  A result depends only on
// its tree, round and slice, and every round has slots of its own, so a slot
// written twice holds the same bits either time: a workgroup that has seen
// no progress for kHelpTicks computes a slice that is still missing, and one
// that fell behind merges the rounds it missed from their slots.  A
// workgroup leaves once its trees have ended (or, after kGiveUpTicks without
// progress, flags them).
template <bool BF16>
__global__ void __launch_bounds__(kWalkThreads, 4) verify_walk_kernel(WalkArgs a) {
  __shared__ WalkShared sh;
  const int tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const int N = a.N, S = a.S, L = a.L, Lp1 = L + 1, Bp1 = a.Bp1, R = a.R;
  const long long V = a.V;
  const size_t esz = BF16 ? 2 : 4;
  // consecutive workgroups serve one tree: the device deals workgroups to
  // its XCDs in turn, so each tree's slices spread over all of them (and each
  // XCD gets slices of every tree) rather than landing on one
  const int grp = (int)(blockIdx.x / S);
  const int member = (int)(blockIdx.x % S);                    // own slice

  const int nt = grp < N ? (N - 1 - grp) / a.groups + 1 : 0;  // trees of the group

  // The group's trees: position p of the launch's trees, those sampled at
  // T > 0 first and then the rest, each kind in index order, goes to group
  // p % groups.  A sampled row costs several times a greedy one (the noise of
  // every element), so where groups serve two trees this pairs sampled trees
  // with greedy ones rather than giving some groups two sampled rows per
  // round while the groups of two greedy trees wait between theirs.  Results
  // do not depend on which group serves a tree.
  {
    const auto sampled = [&](int i) {
      const float T = a.temperature[i];
      return T > 0.f && !isinf(T);
    };
    const int c = (N + kWalkThreads - 1) / kWalkThreads;
    const int i0 = min(tid * c, N), i1 = min(i0 + c, N);
    int h = 0;
    for (int i = i0; i < i1; ++i) h += sampled(i) ? 1 : 0;
    int nsampled = 0;
    const int hb = block_exclusive_scan<kWalkThreads>(h, sh.scan, &nsampled);
    for (int j = 0; j < nt; ++j) {
      const int p = grp + j * a.groups;
      const bool want = p < nsampled;
      const int k = want ? p : p - nsampled;               // rank among the trees of its kind
      const int before = want ? hb : i0 - hb;              // trees of that kind before this thread's range
      const int here = want ? h : (i1 - i0) - h;
      if (k >= before && k < before + here) {
        int seen = before;
        for (int i = i0; i < i1; ++i)
          if (sampled(i) == want) {
            if (seen == k) {
              sh.tree[j] = i;
              break;
            }
            ++seen;
          }
      }
    }
    __syncthreads();
  }

  // each tree's first round (set by the prep or the speculative pass)
  for (int j = 0; j < nt; ++j) {
    const int n = sh.tree[j];
    const size_t tb = (size_t)n * Bp1;
    int nn = a.n_nodes[n];
    nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
    if (tid == 0) {
      const uint32_t w = a.word[n];
      WalkState& t = sh.ts[j];
      t.r = 0;
      t.kind = 0;
      t.ended = w == kEnded ? 1 : 0;
      t.step = (int)((w >> 8) & 0x3Fu);
      t.u = t.ended ? 0 : (int)(w >> 14);
      t.d = a.depth[tb + t.u];
      t.nn = nn;
      t.mine = 0;
      t.miss = 0;
      t.cut = 0.0;
      t.T = (double)a.temperature[n];
      t.sd = a.seed[n];
    }
  }

  // Reduce slice s of the current round of tree j (state t) and publish it.
  // (The state's fields are read from LDS where they are used, into scalar
  // registers, so that no copy of it stays live across the row's loop.)
  auto do_slice = [&](int j, int s) __attribute__((always_inline)) {
    const WalkState& t = sh.ts[j];
    const int n = uni(sh.tree[j]);
    const size_t tb = (size_t)n * Bp1;
    const double T = uni(t.T);
    const uint64_t sd = uni(t.sd);
    const int d = uni(t.d);
    const int r = uni(t.r);
    const void* row = static_cast<const char*>(a.target) + ((tb + uni(t.u)) * (size_t)V) * esz;
    long long e0, e1;
    slice_range<BF16>(row, V, S, uni(s), e0, e1);
    Top2 acc = {-INFINITY, 0x7FFFFFFF, -INFINITY};
    NoiseCache nc;
    const bool exact_pass = T != 0.0 && uni(t.kind) != 0;
    if (!exact_pass) {
      // the logits (T = 0) or the fp32 estimates, per thread in fp32
      Top2f f = {-INFINITY, 0x7FFFFFFF, -INFINITY};
      if (T == 0.0) {
        for_slice<BF16, kWalkVec0>(row, e0, e1, [&](long long i, float x) { top2f_add(f, x, (int)i); });
      } else {
        slice_estimates<BF16, kWalkVec>(row, e0, e1, sd, d, (float)(1.0 / T), f);
      }
      acc = {(double)f.y1, f.i1, (double)f.y2};
    } else {
      // exact fp64 noise for every element whose estimate comes within the
      // slack of the previous round's best estimate
      const float invTf = (float)(1.0 / T);
      const double cut = uni(t.cut);
      for_slice<BF16, kWalkVec>(row, e0, e1, [&](long long i, float x) {
        const uint32_t w = nc.word(i, sd, d);
        if ((double)fmaf(x, invTf, gumbel_estimate(w)) >= cut)
          top2_add(acc, (double)x / T + gumbel_from_word(w), (int)i);
      });
    }
    const Top2 m = block_top2(acc, sh.w);
    if (tid == 0) {
      const size_t slot = ((size_t)n * R + r) * S + uni(s);
      uint64_t A, B;
      if (exact_pass) {
        const uint64_t y = (uint64_t)__double_as_longlong(m.y1);
        slot_pack((uint32_t)(y >> 32), (uint32_t)y, m.i1, A, B);
      } else {  // fp32 values, held exactly in the doubles
        slot_pack(__float_as_uint((float)m.y1), __float_as_uint((float)m.y2), m.i1, A, B);
      }
      st(&a.slot[2 * slot], A);
      st(&a.slot[2 * slot + 1], B);
    }
  };

  uint64_t last_progress = 0;  // thread 0's clock decides; 0: read it at the next idle pass
  int backoff = 1;
  bool links = false;
  while (true) {
    __syncthreads();  // the previous pass's shared fields have been read
    bool progress = false;
    if (!links) {
      // the first round's own slices, then the trees' links and depths (when
      // they fit): the first merge is their first reader, so their loads
      // wait behind the slices instead of delaying them
      for (int j = 0; j < nt; ++j)
        if (!uni(sh.ts[j].ended) && !uni(sh.ts[j].mine)) {
          do_slice(j, member);
          if (tid == 0) sh.ts[j].mine = 1;
          progress = true;
        }
      for (int j = 0; j < nt; ++j) {
        const int nn = uni(sh.ts[j].nn);
        const size_t tb = (size_t)uni(sh.tree[j]) * Bp1;
        if (nn <= kNodeLds)
          for (int q = tid; q < nn; q += kWalkThreads) {
            sh.npar[j][q] = a.parent[tb + q];
            sh.ntok[j][q] = a.node_token[tb + q];
            sh.ndep[j][q] = a.depth[tb + q];
          }
      }
      links = true;
      __syncthreads();
    }
    int alive = 0;
    for (int j = 0; j < nt; ++j) {
      if (uni(sh.ts[j].ended)) continue;
      ++alive;
      const int n = sh.tree[j];
      if (!uni(sh.ts[j].mine)) {
        do_slice(j, member);
        if (tid == 0) sh.ts[j].mine = 1;
        progress = true;
      }
      // poll the round's slots; once all hold a result, merge and step (wave 0)
      if (wid == 0) {
        WalkState& t = sh.ts[j];
        const size_t base = ((size_t)n * R + uni(t.r)) * S;
        uint64_t A = 0, B = 0;
        if (lane < S) {
          A = ld(&a.slot[2 * (base + lane)]);
          B = ld(&a.slot[2 * (base + lane) + 1]);
        }
        const uint64_t have = __ballot(lane >= S || slot_ok(A, B));
        const int complete = have == ~0ull;
        if (complete) {
          Top2 g = {-INFINITY, 0x7FFFFFFF, -INFINITY};
          if (lane < S) {
            const uint32_t hi = (uint32_t)(A >> 32), lo = (uint32_t)(B >> 32);
            const int i20 = (int)((A >> 12) & 0xFFFFFu);
            g.i1 = i20 == kNoIndex20 ? 0x7FFFFFFF : i20;
            if (uni(t.T) != 0.0 && uni(t.kind) != 0) {
              g.y1 = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
            } else {
              g.y1 = (double)__uint_as_float(hi);
              g.y2 = (double)__uint_as_float(lo);
            }
          }
#pragma unroll
          for (int o = kWave / 2; o > 0; o >>= 1) top2_merge(g, top2_shfl_xor(g, o));
          // every lane holds the merged result; lane 0 updates the state
          const int r = uni(t.r), step = uni(t.step), u = uni(t.u);
          const double slack = est_slack(g.y1, g.y2);
          wave_sync();  // every lane has read the state before lane 0 rewrites it
          if (uni(t.T) != 0.0 && uni(t.kind) == 0 && !(g.y1 - g.y2 > slack) && r + 1 < R) {
            // too close to call from the estimates: the same row once more, exactly
            if (lane == 0) {
              t.r = r + 1;
              t.kind = 1;
              t.cut = g.y1 - slack;
              t.mine = 0;
              t.miss = 0;
            }
          } else {
            const int tstar = g.i1 == 0x7FFFFFFF ? 0 : g.i1;
            const size_t tb = (size_t)n * Bp1;
            const int nn = uni(t.nn);
            const bool cached = nn <= kNodeLds;
            int child = 0x7FFFFFFF;
            for (int q = 1 + lane; q < nn; q += kWave) {
              const int p = cached ? sh.npar[j][q] : a.parent[tb + q];
              const int tk = cached ? sh.ntok[j][q] : a.node_token[tb + q];
              if (p == u && tk == tstar && q < child) child = q;
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) child = min(child, __shfl_xor(child, o, kWave));
            int32_t* ot = a.out_tokens + (size_t)n * Lp1;
            int32_t* pn = a.path_nodes + (size_t)n * Lp1;
            if (lane == 0) {
              ot[step] = tstar;
              pn[step] = u;
            }
            if (child != 0x7FFFFFFF && step < L && r + 1 < R) {
              const int dc = cached ? sh.ndep[j][child] : a.depth[tb + child];
              if (lane == 0) {
                t.r = r + 1;
                t.kind = 0;
                t.step = step + 1;
                t.u = child;
                t.d = dc;
                t.mine = 0;
                t.miss = 0;
              }
            } else {
              for (int i = step + 1 + lane; i < Lp1; i += kWave) {
                ot[i] = -1;
                pn[i] = -1;
              }
              const int dd = uni(t.d);
              if (lane == 0) {
                a.tau[n] = dd + 1;
                t.ended = 1;
              }
            }
          }
        } else if (lane == 0) {
          t.miss = ~have;
        }
        if (lane == 0) sh.complete[j] = complete;
      }
      __syncthreads();
      if (sh.complete[j]) progress = true;
    }
    if (alive == 0) break;
    // nothing moved: wait, help with a missing slice, or give up (thread 0
    // decides for the workgroup)
    if (tid == 0) {
      int act = 0, hj = -1, hs = 0;
      // (the clock is read on idle passes only: a read takes a while)
      const uint64_t now = progress ? 0 : __builtin_amdgcn_s_memrealtime();
      if (progress || last_progress == 0) {
        last_progress = now;
      } else if (now - last_progress > kGiveUpTicks) {
        act = 2;
      } else if (now - last_progress > kHelpTicks) {
        for (int j = 0; j < nt && hj < 0; ++j)
          if (!sh.ts[j].ended && sh.ts[j].miss != 0ull) {
            hj = j;
            // the first missing slice at or after this workgroup's own
            const uint64_t m = sh.ts[j].miss;
            hs = (__builtin_ctzll(rotr64(m, member & (kWave - 1))) + member) & (kWave - 1);
          }
        if (hj >= 0) {
          act = 1;
          last_progress = now;
        }
      }
      sh.action = act;
      sh.help_j = hj;
      sh.help_s = hs;
    }
    __syncthreads();
    const int act = sh.action;
    if (act == 2) {
      if (tid == 0)
        for (int j = 0; j < nt; ++j)
          if (!sh.ts[j].ended) {
            const int n = sh.tree[j];
            if (a.status) atomicOr(&a.status[n], MFD_TREE_CAPACITY);
            a.tau[n] = 0;
          }
      break;
    }
    if (act == 1) {
      do_slice(uni(sh.help_j), uni(sh.help_s));
      backoff = 1;
    } else if (!progress) {
      backoff = backoff < 8 ? backoff * 2 : 8;
      for (int z = 0; z < backoff; ++z) __builtin_amdgcn_s_sleep(kPollSleep);
    } else {
      backoff = 1;
    }
  }
}

template <size_t A>
constexpr size_t round_up(size_t x) {
  return (x + A - 1) / A * A;
}

struct WalkWsLayout {
  size_t word, slot, seq_total;                                           // the walk kernel
  size_t spec_cnt, spec_go, spec_nodes, choice, rowdone, treedone, sy, si, total;  // speculation
  int rcap;
};

// Slices per row of V elements of esz bytes: at least one 16-byte vector per
// thread, at most kSlices and at most `cap`.
long long walk_slices(long long V, size_t esz, long long cap) {
  const long long nvec = V / (long long)(16 / esz);
  long long S = (nvec + kWalkThreads - 1) / kWalkThreads;
  if (S > kSlices) S = kSlices;
  if (S > cap) S = cap;
  if (S < 1) S = 1;
  return S;
}

// Rounds a tree's walk may take: the root's row and one per move, each at
// most twice (the estimate, then the exact re-evaluation).
int walk_rounds(int L) { return 2 * (L + 1); }

// Rows the speculation may reduce in one launch of N trees of Bp1 nodes over
// rows of V elements of esz bytes.
long long spec_rows(int N, int Bp1, long long V, size_t esz) {
  long long r = kSpecIntBytes / (V * (long long)esz);
  const long long all = (long long)N * Bp1;
  return r < all ? r : all;
}

// Workspace: the walk kernel's arrays, then (Bp1 > 0) the speculation's,
// sized for rows of V elements of either element size.
WalkWsLayout walk_ws_layout(int N, int L, int Bp1 = 0, long long V = 0) {
  WalkWsLayout w = {};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = round_up<128>(o + bytes);
    return r;
  };
  // per tree, round and slice: a result slot of two 64-bit words
  const size_t slots = (size_t)N * walk_rounds(L) * kSlices;
  w.word = take((size_t)N * sizeof(uint32_t));
  w.slot = take(slots * 2 * sizeof(uint64_t));
  w.seq_total = o + 128;  // room to align the base
  if (Bp1 > 0 && V > 0) {
    long long rs = 0;  // rows x slices, the larger over the two element sizes
    for (size_t esz : {(size_t)2, (size_t)4}) {
      const long long v = spec_rows(N, Bp1, V, esz) * walk_slices(V, esz, kSlices);
      if (v > rs) rs = v;
    }
    w.rcap = (int)spec_rows(N, Bp1, V, 2);
    w.spec_cnt = take((size_t)N * 4 * sizeof(int32_t));
    w.spec_go = take(sizeof(int32_t));
    w.spec_nodes = take((size_t)N * Bp1 * sizeof(uint16_t));
    w.choice = take((size_t)N * Bp1 * sizeof(int32_t));
    w.rowdone = take((size_t)N * Bp1 * sizeof(int32_t));
    w.treedone = take((size_t)N * sizeof(int32_t));
    w.sy = take((size_t)rs * sizeof(double));
    w.si = take((size_t)rs * sizeof(int32_t));
  }
  w.total = o + 128;
  return w;
}

}  // namespace

size_t walk_ws_bytes(int N, int L) { return walk_ws_layout(N, L).seq_total; }

size_t walk_ws_bytes_full(int N, int L, int Bp1, long long V) {
  if (V < 1 || Bp1 < 1 || Bp1 > kMaxB1) return walk_ws_bytes(N, L);
  return walk_ws_layout(N, L, Bp1, V).total;
}

hipError_t launch_verify_walk(const void* target, bool bf16, int N, int Bp1, long long V, int L,
                              const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                              const int32_t* n_nodes, const float* temperature, const uint64_t* seed, int32_t* tau,
                              int32_t* out_tokens, int32_t* path_nodes, int32_t* status, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const void* fn = bf16 ? reinterpret_cast<const void*>(&verify_walk_kernel<true>)
                        : reinterpret_cast<const void*>(&verify_walk_kernel<false>);
  const size_t esz = bf16 ? 2 : 4;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kWalkThreads, 0);
  if (e != hipSuccess) return e;
  const long long resident = (long long)cus * (per_cu < 1 ? 1 : per_cu);
  // trees per launch: one slice per row and kTreesPerGroup trees per group
  const long long per_launch = resident * kTreesPerGroup;
  const int R = walk_rounds(L);

  // speculation when its arrays fit the workspace (the walk gives the same
  // result without it)
  const WalkWsLayout lf = walk_ws_layout(N, L, Bp1, V);
  const bool spec = Bp1 <= kMaxB1 && lf.total <= ws_bytes;
  const WalkWsLayout l = spec ? lf : walk_ws_layout(N, L);
  const long long Smax = walk_slices(V, esz, kSlices);  // the slice-result arrays' row stride bound
  const void* sfn = bf16 ? reinterpret_cast<const void*>(&walk_spec_kernel<true>)
                         : reinterpret_cast<const void*>(&walk_spec_kernel<false>);
  int spec_per_cu = 0;
  if (spec) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&spec_per_cu, sfn, kWalkThreads, 0);
    if (e != hipSuccess) return e;
  }
  const long long spec_grid = (long long)cus * (spec_per_cu < 1 ? 1 : spec_per_cu);

  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 127) & ~uintptr_t(127));
  for (long long n0 = 0; n0 < N; n0 += per_launch) {
    const int nb = (int)(N - n0 < per_launch ? N - n0 : per_launch);
    // S slices per row, as many as the resident workgroups allow for one
    // group per tree; groups of S workgroups, each serving at most
    // kTreesPerGroup trees
    long long S = resident / nb;
    if (S > Smax) S = Smax;
    if (S < 1) S = 1;
    long long groups = resident / S;
    if (groups > nb) groups = nb;
    if ((nb + groups - 1) / groups > kTreesPerGroup) return hipErrorInvalidConfiguration;  // (cannot happen)
    const long long G = groups * S;
    WalkArgs a = {};
    a.groups = (int)groups;
    a.target = static_cast<const char*>(target) + (size_t)n0 * Bp1 * V * esz;
    a.N = nb;
    a.Bp1 = Bp1;
    a.L = L;
    a.S = (int)S;
    a.G = (int)G;
    a.R = R;
    a.esz = (int)esz;
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
    // the slot arrays are cleared by each launch's prep pass and indexed
    // from the launch's first tree with row stride S <= kSlices
    a.slot = reinterpret_cast<uint64_t*>(w + l.slot);
    int rcap = 0;
    if (spec) {
      const long long rs = (long long)((l.si - l.sy) / sizeof(double));  // rows x slices the arrays hold (at least)
      long long r = spec_rows(nb, Bp1, V, esz);
      if (r * Smax > rs) r = rs / Smax;
      rcap = (int)r;
    }
    a.spec = (spec && nb <= kSpecLaunchTrees && rcap > 0) ? 1 : 0;
    if (a.spec) {
      a.spec_rcap = rcap;
      a.spec_cnt = reinterpret_cast<int32_t*>(w + l.spec_cnt) + (size_t)n0 * 4;
      a.spec_go = reinterpret_cast<int32_t*>(w + l.spec_go);
      a.spec_nodes = reinterpret_cast<uint16_t*>(w + l.spec_nodes) + (size_t)n0 * Bp1;
      a.choice = reinterpret_cast<int32_t*>(w + l.choice) + (size_t)n0 * Bp1;
      a.rowdone = reinterpret_cast<int32_t*>(w + l.rowdone) + (size_t)n0 * Bp1;
      a.treedone = reinterpret_cast<int32_t*>(w + l.treedone) + n0;
      a.sy = reinterpret_cast<double*>(w + l.sy);
      a.si = reinterpret_cast<int32_t*>(w + l.si);
    }
    hipLaunchKernelGGL(walk_prep_kernel, dim3(nb), dim3(kWalkThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.spec) {
      if (bf16) hipLaunchKernelGGL(walk_spec_kernel<true>, dim3((unsigned)spec_grid), dim3(kWalkThreads), 0, stream, a);
      else hipLaunchKernelGGL(walk_spec_kernel<false>, dim3((unsigned)spec_grid), dim3(kWalkThreads), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (bf16) hipLaunchKernelGGL(verify_walk_kernel<true>, dim3((unsigned)G), dim3(kWalkThreads), 0, stream, a);
    else hipLaunchKernelGGL(verify_walk_kernel<false>, dim3((unsigned)G), dim3(kWalkThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mfd
