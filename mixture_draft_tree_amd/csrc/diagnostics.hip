// Tree diagnostics: the target mass a tree covers, and its chimeras.
//
// Under tree verification the expected number of accepted drafted tokens is
// the probability mass the tree covers under the target (project page,
// "Abstract"): the sum over drafted nodes of the target's probability of
// producing the node's whole token path, each token drawn from the target's
// distribution at its parent.  A product-ranked tree also spends budget on
// chimeras, prefixes spliced from two futures that the target never produces
// (project page, "TL;DR" and "Abstract").
//
// Covered mass is two passes.  The row pass reads the target row of every
// node that has a child -- the only rows whose distribution enters a path
// probability -- and reduces it to its log-normaliser at temperature T, or to
// its argmax at T = 0 (the target's choice is then certain).  The tree pass
// multiplies, for every drafted node, the probabilities of the tokens on its
// path, walking up the parent links (no ordering of the node arrays is
// assumed), and sums them.  Both trust nothing in the node arrays: a parent
// outside the tree or a walk longer than the tree makes that node count as
// NaN mass (and a chimera walk stop), never an out-of-range access.
#include <math.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kDiagThreads = 256;
constexpr int kDiagWaves = kDiagThreads / kWave;
constexpr float kLog2eF = 1.44269504088896340736f;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ float target_at(const void* row, long long i) {
  return BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(row)[i]) : static_cast<const float*>(row)[i];
}

// Calls f(i, x) for every element of a row of V values: scalars up to the
// first 16-byte boundary and after the last, 16-byte vectors in between.
template <bool BF16, typename F>
__device__ __forceinline__ void for_row(const void* row, long long V, F f) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  const int tid = threadIdx.x;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(row) & 15u;
  long long a = mis ? (long long)((16u - mis) / ESZ) : 0;
  if (a > V) a = V;
  const long long nv = (V - a) / VEC;
  const long long b = a + nv * VEC;
  for (long long i = tid; i < a; i += kDiagThreads) f(i, target_at<BF16>(row, i));
  for (long long i = b + tid; i < V; i += kDiagThreads) f(i, target_at<BF16>(row, i));
  const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + a * ESZ);
  for (long long q = tid; q < nv; q += kDiagThreads) {
    const u32x4 v = __builtin_nontemporal_load(vp + q);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const uint32_t w = v[BF16 ? (j >> 1) : j];
      f(a + q * VEC + j, BF16 ? __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w));
    }
  }
}

__device__ __forceinline__ bool bad_temperature(float T) { return !(T >= 0.f) || isinf(T); }

// Row pass, one workgroup per (node, tree): nodes without a child exit.
template <bool BF16>
__global__ void __launch_bounds__(kDiagThreads) row_norm_kernel(const void* target, int Bp1, long long V,
                                                                const int32_t* parent, const int32_t* n_nodes,
                                                                const float* temperature, double* lse_t,
                                                                int32_t* amax) {
  __shared__ int has_child;
  __shared__ float smax[kDiagWaves];
  __shared__ int sidx[kDiagWaves];
  __shared__ double ssum[kDiagWaves];
  const int u = blockIdx.x, n = blockIdx.y, tid = threadIdx.x;
  const size_t tb = (size_t)n * Bp1;
  int nn = n_nodes[n];
  nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
  if (u >= nn) return;
  const float Tf = temperature[n];
  if (bad_temperature(Tf)) return;
  if (tid == 0) has_child = 0;
  __syncthreads();
  for (int q = 1 + tid; q < nn; q += kDiagThreads)
    if (parent[tb + q] == u) has_child = 1;
  __syncthreads();
  if (!has_child) return;
  const void* row = static_cast<const char*>(target) + (tb + u) * (size_t)V * (BF16 ? 2 : 4);

  // row maximum and its lowest index (NaN is skipped by the comparisons)
  float m = -INFINITY;
  int mi = 0x7FFFFFFF;
  for_row<BF16>(row, V, [&](long long i, float x) {
    if (x > m || (x == m && (int)i < mi)) {
      m = x;
      mi = (int)i;
    }
  });
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, kWave);
    const int oi = __shfl_xor(mi, o, kWave);
    if (om > m || (om == m && oi < mi)) {
      m = om;
      mi = oi;
    }
  }
  if (lane_id() == 0) {
    smax[wave_id()] = m;
    sidx[wave_id()] = mi;
  }
  __syncthreads();
  m = smax[0];
  mi = sidx[0];
  for (int w = 1; w < kDiagWaves; ++w)
    if (smax[w] > m || (smax[w] == m && sidx[w] < mi)) {
      m = smax[w];
      mi = sidx[w];
    }
  if (Tf == 0.f) {
    if (tid == 0) amax[tb + u] = mi;
    return;
  }
  // sum of exp((x - m) / T): fp32 exponentials, fp64 sums
  const float sc = kLog2eF / Tf;
  double s = 0.0;
  if (m != -INFINITY)
    for_row<BF16>(row, V, [&](long long i, float x) { s += (double)__builtin_amdgcn_exp2f((x - m) * sc); });
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (lane_id() == 0) ssum[wave_id()] = s;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kDiagWaves; ++w) t += ssum[w];
    lse_t[tb + u] = (m == -INFINITY) ? -INFINITY : (double)m / (double)Tf + log(t);
  }
}

// Tree pass, one workgroup per tree.
template <bool BF16>
__global__ void __launch_bounds__(kDiagThreads) tree_mass_kernel(const void* target, int Bp1, long long V,
                                                                 const int32_t* node_token, const int32_t* parent,
                                                                 const int32_t* n_nodes, const float* temperature,
                                                                 const double* lse_t, const int32_t* amax,
                                                                 double* mass, int32_t* status) {
  __shared__ double ssum[kDiagWaves];
  const int n = blockIdx.x, tid = threadIdx.x;
  const size_t tb = (size_t)n * Bp1;
  int nn = n_nodes[n];
  nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
  const float Tf = temperature[n];
  if (bad_temperature(Tf)) {
    if (tid == 0) {
      mass[n] = NAN;
      if (status) atomicOr(&status[n], MFD_TREE_BAD_TEMPERATURE);
    }
    return;
  }
  const double T = (double)Tf;
  const size_t esz = BF16 ? 2 : 4;
  double local = 0.0;
  for (int v = 1 + tid; v < nn; v += kDiagThreads) {
    double logp = 0.0;
    bool certain = true, valid = true;
    int x = v;
    for (int steps = 0; x != 0; ++steps) {
      const int p = parent[tb + x];
      const int tok = node_token[tb + x];
      if (steps >= nn || p < 0 || p >= nn || tok < 0 || (long long)tok >= V) {
        valid = false;
        break;
      }
      if (Tf == 0.f) {
        certain = certain && tok == amax[tb + p];
      } else {
        const void* row = static_cast<const char*>(target) + (tb + p) * (size_t)V * esz;
        logp += (double)target_at<BF16>(row, tok) / T - lse_t[tb + p];
      }
      x = p;
    }
    local += !valid ? NAN : (Tf == 0.f ? (certain ? 1.0 : 0.0) : exp(logp));
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) local += __shfl_xor(local, o, kWave);
  if (lane_id() == 0) ssum[wave_id()] = local;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kDiagWaves; ++w) t += ssum[w];
    mass[n] = t;
  }
}

// Chimeras, one workgroup per tree: drafted nodes whose token at every depth is
// future A's or future B's there, yet whose path is a prefix of neither.
__global__ void __launch_bounds__(kDiagThreads) chimera_kernel(const int32_t* node_token, const int32_t* parent,
                                                               const int32_t* depth, const int32_t* n_nodes,
                                                               int Bp1, int L, const int32_t* fa,
                                                               const int32_t* fb, int32_t* count) {
  __shared__ int total;
  const int n = blockIdx.x, tid = threadIdx.x;
  const size_t tb = (size_t)n * Bp1;
  int nn = n_nodes[n];
  nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
  if (tid == 0) total = 0;
  __syncthreads();
  int mine = 0;
  for (int v = 1 + tid; v < nn; v += kDiagThreads) {
    bool spliced = true, pa = true, pb = true, valid = true;
    int x = v;
    for (int steps = 0; x != 0; ++steps) {
      const int dx = depth[tb + x];
      const int p = parent[tb + x];
      if (steps >= nn || dx < 1 || dx > L || p < 0 || p >= nn) {
        valid = false;
        break;
      }
      const int tok = node_token[tb + x];
      const int a = fa[(size_t)n * L + dx - 1], b = fb[(size_t)n * L + dx - 1];
      spliced = spliced && (tok == a || tok == b);
      pa = pa && tok == a;
      pb = pb && tok == b;
      x = p;
    }
    mine += (valid && spliced && !pa && !pb) ? 1 : 0;
  }
  if (mine) atomicAdd(&total, mine);
  __syncthreads();
  if (tid == 0) count[n] = total;
}

}  // namespace

size_t covered_mass_ws_bytes(int N, int Bp1) {
  return (size_t)N * Bp1 * (sizeof(double) + sizeof(int32_t)) + 256;
}

hipError_t launch_covered_mass(const void* target, bool bf16, int N, int Bp1, long long V,
                               const int32_t* node_token, const int32_t* parent, const int32_t* n_nodes,
                               const float* temperature, double* mass, int32_t* status, void* ws,
                               hipStream_t stream) {
  if (N == 0) return hipSuccess;
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 7) & ~uintptr_t(7));
  double* lse_t = reinterpret_cast<double*>(w);
  int32_t* amax = reinterpret_cast<int32_t*>(lse_t + (size_t)N * Bp1);
  const dim3 rows((unsigned)Bp1, (unsigned)N);
  if (bf16) {
    hipLaunchKernelGGL(row_norm_kernel<true>, rows, dim3(kDiagThreads), 0, stream, target, Bp1, V, parent, n_nodes,
                       temperature, lse_t, amax);
    hipLaunchKernelGGL(tree_mass_kernel<true>, dim3(N), dim3(kDiagThreads), 0, stream, target, Bp1, V, node_token,
                       parent, n_nodes, temperature, lse_t, amax, mass, status);
  } else {
    hipLaunchKernelGGL(row_norm_kernel<false>, rows, dim3(kDiagThreads), 0, stream, target, Bp1, V, parent,
                       n_nodes, temperature, lse_t, amax);
    hipLaunchKernelGGL(tree_mass_kernel<false>, dim3(N), dim3(kDiagThreads), 0, stream, target, Bp1, V,
                       node_token, parent, n_nodes, temperature, lse_t, amax, mass, status);
  }
  return hipGetLastError();
}

hipError_t launch_chimera_count(const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                                const int32_t* n_nodes, int N, int Bp1, int L, const int32_t* future_a,
                                const int32_t* future_b, int32_t* count, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(chimera_kernel, dim3(N), dim3(kDiagThreads), 0, stream, node_token, parent, depth, n_nodes,
                     Bp1, L, future_a, future_b, count);
  return hipGetLastError();
}

}  // namespace mfd
