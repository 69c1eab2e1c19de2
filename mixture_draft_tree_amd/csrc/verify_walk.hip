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
// Work layout: each tree gets C workgroups (C from the device's occupancy, up
// to 32) in one cooperative launch, so a visited row of V tokens is split C
// ways across the chip.  Per round every workgroup reduces its slice, publishes
// the result (double-buffered by round parity) and waits on the tree's arrival
// counter; then all C workgroups read the C results at once (one lane each),
// agree on the same token and child, and move on together.  Waits are
// bounded; a wait that runs out flags the tree and ends its walk, so every
// wave exits.  Only the rows on the walked path are read.
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

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kWalkThreads = 256;
constexpr int kWalkWaves = kWalkThreads / kWave;
constexpr int kMaxC = 32;
constexpr long long kSpinLimit = 1LL << 21;  // bounded wait (~0.5 us sleeps), far beyond any real step
constexpr int kPollSleep = 8;                // s_sleep units (64 clocks each) between polls
constexpr int kCounterStride = 32;           // ints: one 128-byte line per tree's arrival counter
constexpr double kGumbelTol = 1e-4;
constexpr float kLn2f = 0.693147180559945309f;
constexpr int kSliceVec = 8;
constexpr int kMaxNodesLds = 4096;  // tree nodes staged in LDS for the child lookup

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

struct WalkArgs {
  const void* target;
  int Bp1;
  long long V;
  int L;
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
  int C;
  double* part_y1;  // [trees][2][C]
  double* part_y2;  // [trees][2][C]
  int32_t* part_i;  // [trees][2][C]
  int32_t* arrive;  // [trees][kCounterStride], element 0 used
};

struct WalkShared {
  Top2 w[kWalkWaves];
  Top2 g;  // the tree's result of the round
  int child;
  int timeout;
};

// Element value as float (bf16 or fp32 storage).
template <bool BF16>
__device__ __forceinline__ float elem_at(const void* row, long long i) {
  return BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(row)[i]) : static_cast<const float*>(row)[i];
}

// Calls f(i, x) for every element i of [e0, e1): scalars before and after the
// 16-byte aligned part, then the aligned vectors kSliceVec per thread at a
// time (all loads of a round issued before any is used; one round covers a
// slice of up to kSliceVec * 256 vectors).
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

// Block-wide Top2 of the per-thread values (barrier inside); every thread gets it.
__device__ __forceinline__ Top2 block_top2(Top2 t, WalkShared& sh) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) top2_merge(t, top2_shfl_xor(t, o));
  if (lane_id() == 0) sh.w[wave_id()] = t;
  __syncthreads();
  Top2 r = sh.w[0];
  for (int w = 1; w < kWalkWaves; ++w) top2_merge(r, sh.w[w]);
  return r;
}

template <bool BF16>
__global__ void __launch_bounds__(kWalkThreads, 4) verify_walk_kernel(WalkArgs a) {
  __shared__ WalkShared sh;
  // dynamic LDS: the tree's parents, then its tokens (min(B + 1, kMaxNodesLds) each)
  extern __shared__ int32_t node_lds[];
  const int C = a.C;
  const int n = blockIdx.x / C;
  const int c = blockIdx.x - n * C;
  const int tid = threadIdx.x;
  const int L = a.L, Lp1 = L + 1, Bp1 = a.Bp1;
  const long long V = a.V;
  const float Tf = a.temperature[n];
  const size_t tb = (size_t)n * Bp1;
  int32_t* ot = a.out_tokens + (size_t)n * Lp1;
  int32_t* pn = a.path_nodes + (size_t)n * Lp1;
  if (!(Tf >= 0.f) || isinf(Tf)) {
    if (c == 0) {
      for (int i = tid; i < Lp1; i += kWalkThreads) {
        ot[i] = -1;
        pn[i] = -1;
      }
      if (tid == 0) {
        a.tau[n] = 0;
        if (a.status) atomicOr(&a.status[n], MFD_TREE_BAD_TEMPERATURE);
      }
    }
    return;
  }
  const double T = (double)Tf;
  const double invT = T > 0.0 ? 1.0 / T : 0.0;
  const uint64_t sd = a.seed[n];
  int nn = a.n_nodes[n];
  nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
  const char* tbase = static_cast<const char*>(a.target);
  const size_t esz = BF16 ? 2 : 4;
  const long long e0 = (V * c) / C, e1 = (V * (c + 1)) / C;  // this workgroup's slice
  double* py1 = a.part_y1 + (size_t)n * 2 * C;
  double* py2 = a.part_y2 + (size_t)n * 2 * C;
  int32_t* pi = a.part_i + (size_t)n * 2 * C;
  int32_t* ctr = a.arrive + (size_t)n * kCounterStride;  // this tree's arrival counter
  // the tree's parents and tokens, for the child lookup of every step
  const int ncap = Bp1 < kMaxNodesLds ? Bp1 : kMaxNodesLds;
  int32_t* lpar = node_lds;
  int32_t* ltok = node_lds + ncap;
  const bool nodes_lds = nn <= ncap;
  if (nodes_lds) {
    for (int q = tid; q < nn; q += kWalkThreads) {
      lpar[q] = a.parent[tb + q];
      ltok[q] = a.node_token[tb + q];
    }
  }
  int round = 0;

  // One exchange round: publish this workgroup's Top2, wait for the tree's
  // other workgroups (bounded), read all C results (lane q reads workgroup
  // q's) and merge them in the same order everywhere.  Result in sh.g.
  auto exchange = [&](const Top2& mine) {
    const int slot = (round & 1) * C;
    if (wave_id() == 0) {
      const int lane = lane_id();
      int to = 0;
      if (lane == 0) {
        __hip_atomic_store(&py1[slot + c], mine.y1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&py2[slot + c], mine.y2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&pi[slot + c], mine.i1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const int want = C * (round + 1);
        long long spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < want) {
          if (++spins > kSpinLimit) {
            to = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(kPollSleep);
        }
      }
      to = __shfl(to, 0, kWave);
      // every lane acquires the counter itself (it already reached `want`), so
      // the results published before the other workgroups' arrivals are visible
      (void)__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      Top2 t = {-INFINITY, 0x7FFFFFFF, -INFINITY};
      if (lane < C) {
        t.y1 = __hip_atomic_load(&py1[slot + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t.y2 = __hip_atomic_load(&py2[slot + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t.i1 = __hip_atomic_load(&pi[slot + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) top2_merge(t, top2_shfl_xor(t, o));
      if (lane == 0) {
        sh.g = t;
        sh.timeout = to;
        sh.child = 0x7FFFFFFF;
      }
    }
    ++round;
    __syncthreads();
  };

  int u = 0, step = 0;
  bool timed_out = false;
  while (true) {
    const int d = a.depth[tb + u];
    const void* row = tbase + ((tb + u) * (size_t)V) * esz;
    Top2 t = {-INFINITY, 0x7FFFFFFF, -INFINITY};
    NoiseCache nc;
    if (T == 0.0) {
      for_slice<BF16>(row, e0, e1, [&](long long i, float x) { top2_add(t, (double)x, (int)i); });
    } else {
      for_slice<BF16>(row, e0, e1, [&](long long i, float x) {
        const float g = gumbel_estimate(nc.word(i, sd, d));
        top2_add(t, (double)x * invT + (double)g, (int)i);
      });
    }
    const Top2 mine = block_top2(t, sh);
    exchange(mine);
    if (sh.timeout) {
      timed_out = true;
      break;
    }
    int tstar = sh.g.i1;
    // the estimates also carry the rounding of x / T (a few ulp of |y|)
    const double slack = 2.0 * kGumbelTol + (fabs(sh.g.y1) + fabs(sh.g.y2)) * 0x1.0p-48;
    if (T != 0.0 && !(sh.g.y1 - sh.g.y2 > slack)) {
      // too close to call from the estimates: exact fp64 noise for every
      // element whose estimate comes within the slack of the best
      const double cut = sh.g.y1 - slack;
      Top2 ex = {-INFINITY, 0x7FFFFFFF, -INFINITY};
      NoiseCache nc2;
      for_slice<BF16>(row, e0, e1, [&](long long i, float x) {
        const uint64_t w = nc2.word(i, sd, d);
        if ((double)x * invT + (double)gumbel_estimate(w) >= cut)
          top2_add(ex, (double)x / T + gumbel_from_word(w), (int)i);
      });
      __syncthreads();  // sh.w is reused
      const Top2 mex = block_top2(ex, sh);
      exchange(mex);
      if (sh.timeout) {
        timed_out = true;
        break;
      }
      tstar = sh.g.i1;
    }
    if (tstar == 0x7FFFFFFF) tstar = 0;
    if (nodes_lds) {
      for (int q = 1 + tid; q < nn; q += kWalkThreads)
        if (lpar[q] == u && ltok[q] == tstar) atomicMin(&sh.child, q);
    } else {
      for (int q = 1 + tid; q < nn; q += kWalkThreads)
        if (a.parent[tb + q] == u && a.node_token[tb + q] == tstar) atomicMin(&sh.child, q);
    }
    __syncthreads();
    const int child = sh.child;
    if (c == 0 && tid == 0) {
      ot[step] = tstar;
      pn[step] = u;
    }
    if (child == 0x7FFFFFFF || step >= L) {
      if (c == 0 && tid == 0) a.tau[n] = d + 1;
      break;
    }
    u = child;
    ++step;
    __syncthreads();
  }
  if (timed_out) {
    if (tid == 0 && a.status) atomicOr(&a.status[n], MFD_TREE_CAPACITY);
    if (c == 0 && tid == 0) a.tau[n] = 0;
  }
  if (c == 0) {
    for (int i = step + 1 + tid; i < Lp1; i += kWalkThreads) {
      ot[i] = -1;
      pn[i] = -1;
    }
  }
}

__global__ void zero_i32(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

size_t walk_ws_bytes(int N) {
  // per tree: the round results (two values and an index), double-buffered,
  // for up to kMaxC workgroups, and an arrival counter on a line of its own
  return (size_t)N * (2 * kMaxC * (2 * sizeof(double) + sizeof(int32_t)) + kCounterStride * sizeof(int32_t)) + 256;
}

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
  const size_t lds = (size_t)2 * (Bp1 < kMaxNodesLds ? Bp1 : kMaxNodesLds) * sizeof(int32_t);
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kWalkThreads, lds);
  if (e != hipSuccess) return e;
  long long resident = (long long)cus * per_cu;
  if (resident < 1) resident = 1;
  int C = (int)(resident / N);
  if (C > kMaxC) C = kMaxC;
  if (C < 1) C = 1;
  // with more trees than resident workgroups, walk them in several launches
  const int per_launch = (int)(resident / C < 1 ? 1 : resident / C);

  char* w = static_cast<char*>(ws);
  double* part_y1 = reinterpret_cast<double*>(w);
  double* part_y2 = part_y1 + (size_t)N * 2 * kMaxC;
  int32_t* part_i = reinterpret_cast<int32_t*>(part_y2 + (size_t)N * 2 * kMaxC);
  // 128-byte aligned counters, one line per tree
  const uintptr_t cbase = (reinterpret_cast<uintptr_t>(part_i + (size_t)N * 2 * kMaxC) + 127) & ~uintptr_t(127);
  int32_t* arrive = reinterpret_cast<int32_t*>(cbase);
  hipLaunchKernelGGL(zero_i32, dim3((N * kCounterStride + 255) / 256), dim3(256), 0, stream, arrive,
                     N * kCounterStride);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int n0 = 0; n0 < N; n0 += per_launch) {
    const int nb = (N - n0 < per_launch) ? N - n0 : per_launch;
    WalkArgs a;
    a.target = static_cast<const char*>(target) + (size_t)n0 * Bp1 * V * (bf16 ? 2 : 4);
    a.Bp1 = Bp1;
    a.V = V;
    a.L = L;
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
    a.C = C;
    a.part_y1 = part_y1 + (size_t)n0 * 2 * C;
    a.part_y2 = part_y2 + (size_t)n0 * 2 * C;
    a.part_i = part_i + (size_t)n0 * 2 * C;
    a.arrive = arrive + (size_t)n0 * kCounterStride;
    void* args[] = {&a};
    e = hipLaunchCooperativeKernel(fn, dim3(nb * C), dim3(kWalkThreads), args, lds, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mfd
