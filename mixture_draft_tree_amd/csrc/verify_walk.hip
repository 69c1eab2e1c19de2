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
// One 1024-thread workgroup per tree; each visited row is streamed once with
// 16-byte loads, reduced with wave shuffles and one LDS step.  Only the rows
// on the walked path are read.
#include <math.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / kWave;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct WalkShared {
  uint64_t best_key[kWalkWaves];
  double best_y[kWalkWaves];
  int best_i[kWalkWaves];
  int child;
  int tstar;
};

__device__ __forceinline__ uint64_t lane_word(const Philox4& r, int l) {
  return l == 0 ? r.v[0] : (l == 1 ? r.v[1] : (l == 2 ? r.v[2] : r.v[3]));
}

// (y, index) with larger y first, then lower index.
__device__ __forceinline__ bool better(double y, int i, double by, int bi) {
  return (y > by) || (y == by && i < bi);
}

template <bool BF16>
__device__ __forceinline__ float elem_val(const void* row, long long i) {
  if (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(row)[i]);
  return static_cast<const float*>(row)[i];
}
template <bool BF16>
__device__ __forceinline__ uint32_t elem_key(const void* row, long long i) {
  if (BF16) return bf16_key(static_cast<const uint16_t*>(row)[i]);
  return f32_key(__float_as_uint(static_cast<const float*>(row)[i]));
}

// Argmax of one row at T = 0: the largest (key, ~index).
template <bool BF16>
__device__ int row_argmax(const void* row, long long V, WalkShared& sh) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int tid = threadIdx.x;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  const int esz = BF16 ? 2 : 4;
  long long head = (long long)(((16u - (addr & 15u)) & 15u) / esz);
  if (head > V) head = V;
  const long long nvec = (V - head) / VEC;
  const long long tail0 = head + nvec * VEC;
  uint64_t best = 0;
  for (long long i = tid; i < head; i += kWalkThreads)
    best = max(best, ((uint64_t)elem_key<BF16>(row, i) << 32) | (0xFFFFFFFFu - (uint32_t)i));
  for (long long i = tail0 + tid; i < V; i += kWalkThreads)
    best = max(best, ((uint64_t)elem_key<BF16>(row, i) << 32) | (0xFFFFFFFFu - (uint32_t)i));
  const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + head * esz);
  for (long long q = tid; q < nvec; q += kWalkThreads) {
    const u32x4 v = __builtin_nontemporal_load(vp + q);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const uint32_t w = v[BF16 ? (j >> 1) : j];
      const uint32_t bits = BF16 ? ((j & 1) ? (w >> 16) : (w & 0xFFFFu)) : w;
      const uint32_t key = BF16 ? bf16_key(bits) : f32_key(bits);
      const uint32_t idx = (uint32_t)(head + q * VEC + j);
      best = max(best, ((uint64_t)key << 32) | (0xFFFFFFFFu - idx));
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) best = max(best, (uint64_t)__shfl_xor((unsigned long long)best, o, kWave));
  if (lane_id() == 0) sh.best_key[wave_id()] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t b = sh.best_key[0];
    for (int w = 1; w < kWalkWaves; ++w) b = max(b, sh.best_key[w]);
    sh.tstar = (int)(0xFFFFFFFFu - (uint32_t)b);
  }
  __syncthreads();
  return sh.tstar;
}

// Gumbel-max sample of one row at T > 0.
template <bool BF16>
__device__ int row_sample(const void* row, long long V, double T, uint64_t seed, int d, WalkShared& sh) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int tid = threadIdx.x;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  const int esz = BF16 ? 2 : 4;
  long long head = (long long)(((16u - (addr & 15u)) & 15u) / esz);
  if (head > V) head = V;
  const long long nvec = (V - head) / VEC;
  const long long tail0 = head + nvec * VEC;
  double by = -INFINITY;
  int bi = 0x7FFFFFFF;
  auto scalar = [&](long long i) {
    const Philox4 r = philox4x64_10((uint64_t)i >> 2, (uint64_t)d, 0, 0, seed, 0);
    const double y = (double)elem_val<BF16>(row, i) / T + gumbel_from_word(lane_word(r, (int)(i & 3)));
    if (better(y, (int)i, by, bi)) {
      by = y;
      bi = (int)i;
    }
  };
  for (long long i = tid; i < head; i += kWalkThreads) scalar(i);
  for (long long i = tail0 + tid; i < V; i += kWalkThreads) scalar(i);
  const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + head * esz);
  for (long long q = tid; q < nvec; q += kWalkThreads) {
    const u32x4 v = __builtin_nontemporal_load(vp + q);
    const long long i0 = head + q * VEC;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const long long i = i0 + j;
      // one Philox block per aligned group of four tokens
      Philox4 r;
      if (j == 0 || ((i & 3) == 0)) r = philox4x64_10((uint64_t)i >> 2, (uint64_t)d, 0, 0, seed, 0);
      const uint32_t w = v[BF16 ? (j >> 1) : j];
      const float x = BF16 ? __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w);
      const double y = (double)x / T + gumbel_from_word(lane_word(r, (int)(i & 3)));
      if (better(y, (int)i, by, bi)) {
        by = y;
        bi = (int)i;
      }
    }
  }
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
    sh.best_y[wave_id()] = by;
    sh.best_i[wave_id()] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    double y = sh.best_y[0];
    int i = sh.best_i[0];
    for (int w = 1; w < kWalkWaves; ++w)
      if (better(sh.best_y[w], sh.best_i[w], y, i)) {
        y = sh.best_y[w];
        i = sh.best_i[w];
      }
    sh.tstar = (i == 0x7FFFFFFF) ? 0 : i;
  }
  __syncthreads();
  return sh.tstar;
}

template <bool BF16>
__global__ void __launch_bounds__(kWalkThreads)
    verify_walk_kernel(const void* __restrict__ target, int Bp1, long long V, int L,
                       const int32_t* __restrict__ node_token, const int32_t* __restrict__ parent,
                       const int32_t* __restrict__ depth, const int32_t* __restrict__ n_nodes,
                       const float* __restrict__ temperature, const uint64_t* __restrict__ seed,
                       int32_t* __restrict__ tau_out, int32_t* __restrict__ out_tokens,
                       int32_t* __restrict__ path_nodes, int32_t* __restrict__ status) {
  __shared__ WalkShared sh;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int Lp1 = L + 1;
  const float Tf = temperature[n];
  const size_t tb = (size_t)n * Bp1;
  int32_t* ot = out_tokens + (size_t)n * Lp1;
  int32_t* pn = path_nodes + (size_t)n * Lp1;
  if (!(Tf >= 0.f) || isinf(Tf)) {
    for (int i = tid; i < Lp1; i += kWalkThreads) {
      ot[i] = -1;
      pn[i] = -1;
    }
    if (tid == 0) {
      tau_out[n] = 0;
      if (status) atomicOr(&status[n], MFD_TREE_BAD_TEMPERATURE);
    }
    return;
  }
  const double T = (double)Tf;
  const uint64_t sd = seed[n];
  int nn = n_nodes[n];
  nn = nn < 1 ? 1 : (nn > Bp1 ? Bp1 : nn);
  const char* base = static_cast<const char*>(target);
  const size_t esz = BF16 ? 2 : 4;
  int u = 0, step = 0;
  while (true) {
    const int d = depth[tb + u];
    const void* row = base + ((tb + u) * (size_t)V) * esz;
    const int t = (T == 0.0) ? row_argmax<BF16>(row, V, sh) : row_sample<BF16>(row, V, T, sd, d, sh);
    if (tid == 0) sh.child = 0x7FFFFFFF;
    __syncthreads();
    for (int c = 1 + tid; c < nn; c += kWalkThreads)
      if (parent[tb + c] == u && node_token[tb + c] == t) atomicMin(&sh.child, c);
    __syncthreads();
    const int child = sh.child;
    if (tid == 0) {
      ot[step] = t;
      pn[step] = u;
    }
    __syncthreads();
    if (child == 0x7FFFFFFF || step >= L) {
      if (tid == 0) tau_out[n] = d + 1;
      break;
    }
    u = child;
    ++step;
  }
  for (int i = step + 1 + tid; i < Lp1; i += kWalkThreads) {
    ot[i] = -1;
    pn[i] = -1;
  }
}

}  // namespace

hipError_t launch_verify_walk(const void* target, bool bf16, int N, int Bp1, long long V, int L,
                              const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                              const int32_t* n_nodes, const float* temperature, const uint64_t* seed, int32_t* tau,
                              int32_t* out_tokens, int32_t* path_nodes, int32_t* status, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(verify_walk_kernel<true>, dim3(N), dim3(kWalkThreads), 0, stream, target, Bp1, V, L,
                       node_token, parent, depth, n_nodes, temperature, seed, tau, out_tokens, path_nodes, status);
  else
    hipLaunchKernelGGL(verify_walk_kernel<false>, dim3(N), dim3(kWalkThreads), 0, stream, target, Bp1, V, L,
                       node_token, parent, depth, n_nodes, temperature, seed, tau, out_tokens, path_nodes, status);
  return hipGetLastError();
}

}  // namespace mfd
