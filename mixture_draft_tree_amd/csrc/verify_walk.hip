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
// ways across the chip.  Per depth step every workgroup reduces its slice to
// a (value, index) pair, publishes it (double-buffered by step parity) and
// waits on the tree's arrival counter; then all C workgroups read the C
// pairs, agree on the same token and child, and move on together.  Waits are
// bounded; a wait that runs out flags the tree and ends its walk, so every
// wave exits.  Only the rows on the walked path are read.
#include <math.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kWalkThreads = 256;
constexpr int kWalkWaves = kWalkThreads / kWave;
constexpr int kMaxC = 32;
constexpr long long kSpinLimit = 1LL << 22;  // bounded wait (short sleeps), far beyond any real step

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t lane_word(const Philox4& r, int l) {
  return l == 0 ? r.v[0] : (l == 1 ? r.v[1] : (l == 2 ? r.v[2] : r.v[3]));
}

// (y, index) with larger y first, then lower index.
__device__ __forceinline__ bool better(double y, int i, double by, int bi) {
  return (y > by) || (y == by && i < bi);
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
  double* part_y;   // [trees][2][C]
  int32_t* part_i;  // [trees][2][C]
  int32_t* arrive;  // [trees]
};

struct WalkShared {
  double y[kWalkWaves];
  int i[kWalkWaves];
  int child;
  int tstar;
  int timeout;
};

template <bool BF16, bool SAMPLE>
__device__ __forceinline__ void consider(long long i, float x, const Philox4& r, double T, double& by, int& bi) {
  double y = (double)x;
  if (SAMPLE) y = y / T + gumbel_from_word(lane_word(r, (int)(i & 3)));
  if (better(y, (int)i, by, bi)) {
    by = y;
    bi = (int)i;
  }
}

// This thread's best (y, index) over its share of elements [e0, e1) of a row.
template <bool BF16, bool SAMPLE>
__device__ void slice_best(const void* row, long long e0, long long e1, double T, uint64_t seed, int d, double& by,
                           int& bi) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int esz = BF16 ? 2 : 4;
  const int tid = threadIdx.x;
  // 16-byte aligned vectors fully inside [e0, e1); scalars before and after
  const uintptr_t base = reinterpret_cast<uintptr_t>(row);
  long long a = e0;
  while (a < e1 && ((base + (uintptr_t)a * esz) & 15u)) ++a;
  const long long nv = (e1 - a) / VEC;
  const long long b = a + nv * VEC;
  for (int part = 0; part < 2; ++part) {
    const long long s0 = part == 0 ? e0 : b, s1 = part == 0 ? a : e1;
    for (long long i = s0 + tid; i < s1; i += kWalkThreads) {
      const float x = BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(row)[i]) : static_cast<const float*>(row)[i];
      Philox4 r = {};
      if (SAMPLE) r = philox4x64_10((uint64_t)i >> 2, (uint64_t)d, 0, 0, seed, 0);
      consider<BF16, SAMPLE>(i, x, r, T, by, bi);
    }
  }
  const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + a * esz);
  for (long long q = tid; q < nv; q += kWalkThreads) {
    const u32x4 v = __builtin_nontemporal_load(vp + q);
    const long long i0 = a + q * VEC;
    Philox4 r = {};
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const long long i = i0 + j;
      if (SAMPLE && (j == 0 || (i & 3) == 0)) r = philox4x64_10((uint64_t)i >> 2, (uint64_t)d, 0, 0, seed, 0);
      const uint32_t w = v[BF16 ? (j >> 1) : j];
      const float x = BF16 ? __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w);
      consider<BF16, SAMPLE>(i, x, r, T, by, bi);
    }
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kWalkThreads) verify_walk_kernel(WalkArgs a) {
  __shared__ WalkShared sh;
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
  const uint64_t sd = a.seed[n];
  int nn = a.n_nodes[n];
  nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
  const char* tbase = static_cast<const char*>(a.target);
  const size_t esz = BF16 ? 2 : 4;
  const long long e0 = (V * c) / C, e1 = (V * (c + 1)) / C;  // this workgroup's slice
  double* py = a.part_y + (size_t)n * 2 * C;
  int32_t* pi = a.part_i + (size_t)n * 2 * C;

  int u = 0, step = 0;
  while (true) {
    const int d = a.depth[tb + u];
    const void* row = tbase + ((tb + u) * (size_t)V) * esz;
    double by = -INFINITY;
    int bi = 0x7FFFFFFF;
    if (T == 0.0) slice_best<BF16, false>(row, e0, e1, T, sd, d, by, bi);
    else slice_best<BF16, true>(row, e0, e1, T, sd, d, by, bi);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const double oy = __shfl_xor(by, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(oy, oi, by, bi)) {
        by = oy;
        bi = oi;
      }
    }
    if (lane_id() == 0) {
      sh.y[wave_id()] = by;
      sh.i[wave_id()] = bi;
    }
    __syncthreads();
    const int slot = (step & 1) * C;
    if (tid == 0) {
      double y = sh.y[0];
      int i = sh.i[0];
      for (int w = 1; w < kWalkWaves; ++w)
        if (better(sh.y[w], sh.i[w], y, i)) {
          y = sh.y[w];
          i = sh.i[w];
        }
      __hip_atomic_store(&py[slot + c], y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&pi[slot + c], i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // publish, then wait for the tree's other workgroups (bounded)
      __hip_atomic_fetch_add(&a.arrive[n], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const int want = C * (step + 1);
      long long spins = 0;
      int to = 0;
      while (__hip_atomic_load(&a.arrive[n], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < want) {
        if (++spins > kSpinLimit) {
          to = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      // every workgroup reduces the same C pairs in the same order
      double wy = -INFINITY;
      int wi = 0x7FFFFFFF;
      for (int q = 0; q < C; ++q) {
        const double qy = __hip_atomic_load(&py[slot + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int qi = __hip_atomic_load(&pi[slot + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (better(qy, qi, wy, wi)) {
          wy = qy;
          wi = qi;
        }
      }
      sh.tstar = (wi == 0x7FFFFFFF) ? 0 : wi;
      sh.timeout = to;
      sh.child = 0x7FFFFFFF;
    }
    __syncthreads();
    if (sh.timeout) {
      if (tid == 0 && a.status) atomicOr(&a.status[n], MFD_TREE_CAPACITY);
      if (c == 0 && tid == 0) a.tau[n] = 0;
      break;
    }
    const int t = sh.tstar;
    for (int q = 1 + tid; q < nn; q += kWalkThreads)
      if (a.parent[tb + q] == u && a.node_token[tb + q] == t) atomicMin(&sh.child, q);
    __syncthreads();
    const int child = sh.child;
    if (c == 0 && tid == 0) {
      ot[step] = t;
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
  // partial (y, index) pairs, double-buffered, for up to kMaxC workgroups per
  // tree, and one arrival counter per tree
  return (size_t)N * (2 * kMaxC * (sizeof(double) + sizeof(int32_t)) + sizeof(int32_t)) + 256;
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
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kWalkThreads, 0);
  if (e != hipSuccess) return e;
  long long resident = (long long)cus * per_cu;
  if (resident < 1) resident = 1;
  int C = (int)(resident / N);
  if (C > kMaxC) C = kMaxC;
  if (C < 1) C = 1;
  // with more trees than resident workgroups, walk them in several launches
  const int per_launch = (int)(resident / C < 1 ? 1 : resident / C);

  char* w = static_cast<char*>(ws);
  double* part_y = reinterpret_cast<double*>(w);
  int32_t* part_i = reinterpret_cast<int32_t*>(part_y + (size_t)N * 2 * kMaxC);
  int32_t* arrive = part_i + (size_t)N * 2 * kMaxC;
  hipLaunchKernelGGL(zero_i32, dim3((N + 255) / 256), dim3(256), 0, stream, arrive, N);
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
    a.part_y = part_y + (size_t)n0 * 2 * C;
    a.part_i = part_i + (size_t)n0 * 2 * C;
    a.arrive = arrive + n0;
    void* args[] = {&a};
    e = hipLaunchCooperativeKernel(fn, dim3(nb * C), dim3(kWalkThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mfd
