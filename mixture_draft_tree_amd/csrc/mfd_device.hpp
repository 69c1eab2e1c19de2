// Device helpers shared by the gfx950 kernels of libmfdtree.
//
// Everything here is wave64-native: scans and ballots work on 64 lanes, and
// block-level helpers take the block size as a template argument so loops
// and LDS sizes are compile-time.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfd {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }
__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// Orders LDS traffic between lanes of one wavefront (no block barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- ordered keys
// Unsigned keys that order like the floating-point values (larger value ->
// larger key).  -0.0 is folded onto +0.0 so equal values give equal keys.

__device__ __forceinline__ uint32_t bf16_key(uint32_t b) {
  b &= 0xFFFFu;
  if (b == 0x8000u) b = 0;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
__device__ __forceinline__ uint32_t bf16_from_key(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
}
__device__ __forceinline__ uint32_t f32_key(uint32_t u) {
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t f32_from_key(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
}
__device__ __forceinline__ uint64_t f64_key(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  if (u == 0x8000000000000000ull) u = 0;
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double f64_from_key(uint64_t k) {
  uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)u);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float((b & 0xFFFFu) << 16); }

// ---------------------------------------------------------------- lane exchange
// Cross-lane moves that stay in the vector ALU instead of going through the
// LDS crossbar (ds_bpermute): DPP quad permutes and row rotations within rows
// of 16 lanes, and the gfx950 permlane swaps across rows and wave halves.
// The whole wave must be active.

// DPP controls (gfx9 encoding)
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111;  // row_shr:n = 0x110 + n: lane i takes lane i - n of its row
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowRor4 = 0x124;   // row_ror:n = 0x120 + n: lane i takes lane (i - n) mod 16 of its row
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowRor12 = 0x12C;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  // lanes whose source lies outside the row read 0 (the "old" operand)
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// v of lane (lane ^ s), s in {1, 2, 4, 8, 16, 32}.
__device__ __forceinline__ uint32_t xor_lanes(uint32_t v, int s) {
  const int lane = lane_id();
  switch (s) {
    case 1:
      return dpp_u32<kDppQuadXor1>(v);
    case 2:
      return dpp_u32<kDppQuadXor2>(v);
    case 4: {
      const uint32_t below = dpp_u32<kDppRowRor4>(v), above = dpp_u32<kDppRowRor12>(v);
      return (lane & 4) ? below : above;
    }
    case 8:
      return dpp_u32<kDppRowRor8>(v);
    case 16: {
      // the swap hands each odd row the even row below it, and each even row the odd row above
      const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane & 16) ? p[0] : p[1];
    }
    default: {
      const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane & 32) ? p[0] : p[1];
    }
  }
}
__device__ __forceinline__ int xor_lanes(int v, int s) { return (int)xor_lanes((uint32_t)v, s); }
__device__ __forceinline__ float xor_lanes(float v, int s) {
  return __uint_as_float(xor_lanes(__float_as_uint(v), s));
}
__device__ __forceinline__ uint64_t xor_lanes(uint64_t v, int s) {
  const uint32_t lo = xor_lanes((uint32_t)v, s), hi = xor_lanes((uint32_t)(v >> 32), s);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ double xor_lanes(double v, int s) {
  return __longlong_as_double((long long)xor_lanes((uint64_t)__double_as_longlong(v), s));
}

// ---------------------------------------------------------------- scans

// Inclusive sum over lanes 0..lane: within each row of 16 lanes by four DPP
// shifted adds (Hillis-Steele), then the totals of the rows below.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  uint32_t u = (uint32_t)x;
  u += dpp_u32<kDppRowShr1>(u);
  u += dpp_u32<kDppRowShr2>(u);
  u += dpp_u32<kDppRowShr4>(u);
  u += dpp_u32<kDppRowShr8>(u);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)u, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)u, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)u, 47);
  const int row = lane_id() >> 4;
  u += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
  return (int)u;
}

// op over all 64 lanes (xor strides 32, 16, ..., 1).  The loop runs over the
// stride's log2, a linear induction variable, so it unrolls fully and every
// xor_lanes gets a constant stride.
template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T x, Op op) {
#pragma unroll
  for (int lg = 5; lg >= 0; --lg) x = op(x, xor_lanes(x, 1 << lg));
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
  return wave_allreduce(x, [](int a, int b) { return a + b; });
}

// Exclusive scan over the block; `total` receives the block sum.  `smem` needs
// NT/64 ints.  Contains barriers: every thread of the block must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* smem, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id(), wid = wave_id();
  int x = wave_inclusive_scan(v);
  if (lane == kWave - 1) smem[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = (lane < NW) ? smem[lane] : 0;
    w = wave_inclusive_scan(w);
    if (lane < NW) smem[lane] = w;
  }
  __syncthreads();
  int prefix = (wid > 0 ? smem[wid - 1] : 0) + x - v;
  *total = smem[NW - 1];
  __syncthreads();
  return prefix;
}

template <int NT>
__device__ __forceinline__ int block_sum(int v, int* smem) {
  int total;
  block_exclusive_scan<NT>(v, smem, &total);
  return total;
}

// ---------------------------------------------------------------- bitonic sort
// Sorts a[0..n) ascending in LDS; n must be a power of two.  Barriers inside.
template <int NT>
__device__ __forceinline__ void block_bitonic_sort(uint64_t* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += NT) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const uint64_t x = a[i], y = a[j];
        if ((x > y) == up) {
          a[i] = y;
          a[j] = x;
        }
      }
      __syncthreads();
    }
  }
}

// v of lane (lane ^ m) through the LDS crossbar (ds_bpermute), for a mask m
// known only at run time: the exchanges of several registers stay in flight
// together, where xor_lanes would branch on m for each of them.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m, kWave);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo;
}

// Sorts the 2*NT values held two per thread (thread t holds elements 2t and
// 2t+1 in a0, a1) ascending, with the same bitonic network as
// block_bitonic_sort.  Strides inside a wave go through xor_lanes (constant
// after unrolling); only the strides that cross waves go through `xchg`
// (2*NT uint64 of LDS), two barriers each.  Every thread of the block must
// call it.
template <int NT>
__device__ __forceinline__ void block_sort_pairs(uint64_t& a0, uint64_t& a1, uint64_t* xchg) {
  constexpr int P = 2 * NT;
  constexpr int LP = __builtin_ctz(P);
  const int i0 = 2 * (int)threadIdx.x;
#pragma unroll
  for (int lsize = 1; lsize <= LP; ++lsize) {
    const int size = 1 << lsize;
#pragma unroll
    for (int ls = lsize - 1; ls >= 0; --ls) {
      const int s = 1 << ls;
      const bool up = (i0 & size) == 0;
      if (s == 1) {
        const uint64_t lo = a0 < a1 ? a0 : a1, hi = a0 < a1 ? a1 : a0;
        a0 = up ? lo : hi;
        a1 = up ? hi : lo;
        continue;
      }
      uint64_t b0, b1;
      if (s < 2 * kWave) {
        b0 = xor_lanes(a0, s >> 1);
        b1 = xor_lanes(a1, s >> 1);
      } else {
        xchg[i0] = a0;
        xchg[i0 + 1] = a1;
        __syncthreads();
        b0 = xchg[i0 ^ s];
        b1 = xchg[(i0 + 1) ^ s];
        __syncthreads();
      }
      // for s >= 2 both elements share the lower/upper role and the direction
      const bool keep_min = ((i0 & s) == 0) == up;
      a0 = keep_min ? (a0 < b0 ? a0 : b0) : (a0 < b0 ? b0 : a0);
      a1 = keep_min ? (a1 < b1 ? a1 : b1) : (a1 < b1 ? b1 : a1);
    }
  }
}

// Sorts the NT values held one per thread (thread t holds element t) ascending
// with the bitonic network; strides inside a wave use xor_lanes, strides
// across waves go through `xchg` (NT uint64 of LDS, two barriers each).  Every
// thread of the block must call it.
template <int NT>
__device__ __forceinline__ void block_sort_single(uint64_t& a, uint64_t* xchg) {
  const int t = (int)threadIdx.x;
  constexpr int LN = __builtin_ctz(NT);
#pragma unroll
  for (int lsize = 1; lsize <= LN; ++lsize) {
    const int size = 1 << lsize;
#pragma unroll
    for (int ls = lsize - 1; ls >= 0; --ls) {
      const int s = 1 << ls;
      uint64_t b;
      if (s < kWave) {
        b = xor_lanes(a, s);
      } else {
        xchg[t] = a;
        __syncthreads();
        b = xchg[t ^ s];
        __syncthreads();
      }
      const bool keep_min = ((t & s) == 0) == ((t & size) == 0);
      a = keep_min ? (a < b ? a : b) : (a < b ? b : a);
    }
  }
}

// block_bitonic_sort's network with each wave's segment of P keys held in
// registers: thread (wave w, lane l) holds elements w*64E + e*64 + l,
// e < E.  Strides below 64 are lane exchanges (shfl_xor_u64: the stride is a
// run-time value here), strides from 64 to 64E - 1 swap
// registers within a thread, and only strides of a whole segment or more
// go through LDS, one barrier each (plus one on either side of such a run).
// P is a power of two: 64 <= P <= NT for E = 1, P = E * NT for E > 1.
// Waves past P/(64E) hold nothing and only join the barriers.
template <int NT, int E>
__device__ __forceinline__ void block_sort_regs(uint64_t* a, int P) {
  constexpr int S = kWave * E;
  const int W = P / S;
  const int w = wave_id(), lane = lane_id();
  const bool act = w < W;
  const int base = w * S;
  uint64_t r[E];
  if (act) {
#pragma unroll
    for (int e = 0; e < E; ++e) r[e] = a[base + e * kWave + lane];
  }
  for (int k = 2; k <= P; k <<= 1) {
    int j = k >> 1;
    if (j >= S) {
      if (act) {
#pragma unroll
        for (int e = 0; e < E; ++e) a[base + e * kWave + lane] = r[e];
      }
      __syncthreads();
      for (; j >= S; j >>= 1) {
        for (int t = (int)threadIdx.x; t < (P >> 1); t += NT) {
          const int i = 2 * t - (t & (j - 1));
          const int i2 = i + j;
          const bool up = (i & k) == 0;
          const uint64_t x = a[i], y = a[i2];
          if ((x > y) == up) {
            a[i] = y;
            a[i2] = x;
          }
        }
        __syncthreads();
      }
      if (act) {
#pragma unroll
        for (int e = 0; e < E; ++e) r[e] = a[base + e * kWave + lane];
      }
    }
    if (!act) continue;
    for (; j >= kWave; j >>= 1) {
      const int m = j / kWave;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (e & m) continue;
        const int e2 = e | m;
        const bool up = ((base + e * kWave + lane) & k) == 0;
        const uint64_t x = r[e], y = r[e2];
        const bool sw = (x > y) == up;
        r[e] = sw ? y : x;
        r[e2] = sw ? x : y;
      }
    }
    for (; j > 0; j >>= 1) {
      const bool lower = (lane & j) == 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint64_t o = shfl_xor_u64(r[e], j);
        const bool up = ((base + e * kWave + lane) & k) == 0;
        const bool keep_min = lower == up;
        r[e] = keep_min ? (r[e] < o ? r[e] : o) : (r[e] < o ? o : r[e]);
      }
    }
  }
  if (act) {
#pragma unroll
    for (int e = 0; e < E; ++e) a[base + e * kWave + lane] = r[e];
  }
  __syncthreads();
}

// block_sort_regs for one size P = 2^LP <= NT (one key per lane) with every
// loop unrolled: all strides are constants, so the exchanges inside a wave
// are xor_lanes moves and the network has no loop or branch on the stride
// (about 40% faster than the rolled network for 64 to 256 keys, 20% for
// 1024).  Strides of 64 or more go through LDS, two barriers each.
template <int NT, int LP>
__device__ __forceinline__ void block_sort_static(uint64_t* a) {
  constexpr int P = 1 << LP;
  static_assert(P >= kWave && P <= NT, "one key per lane of P / 64 waves");
  const int lane = lane_id();
  const int i = (int)threadIdx.x;  // this lane's key
  const bool act = i < P;
  uint64_t r = act ? a[i] : 0ull;
#pragma unroll
  for (int lk = 1; lk <= LP; ++lk) {
    const int k = 1 << lk;
#pragma unroll
    for (int lj = lk - 1; lj >= 0; --lj) {
      const int j = 1 << lj;
      const bool up = (i & k) == 0;
      if (j >= kWave) {
        if (act) a[i] = r;
        __syncthreads();
        const uint64_t o = act ? a[i ^ j] : 0ull;
        __syncthreads();
        const bool keep_min = ((i & j) == 0) == up;
        if (act) r = keep_min ? (r < o ? r : o) : (r < o ? o : r);
      } else if (act) {
        const uint64_t o = xor_lanes(r, j);
        const bool keep_min = ((lane & j) == 0) == up;
        r = keep_min ? (r < o ? r : o) : (r < o ? o : r);
      }
    }
  }
  if (act) a[i] = r;
  __syncthreads();
}

// Sorts a[0, P) ascending, P a power of two (a[] written and visible to the
// block on entry, sorted and visible on return).  Sizes from 64 to
// min(NT, 1024) take the unrolled network of their size, sizes up to 4*NT
// the register-resident one, others the LDS one.  Every thread calls it.
template <int NT>
__device__ __forceinline__ void block_sort_keys(uint64_t* a, int P) {
  if (P >= kWave && P <= NT && P <= 1024) {
    switch (P) {
      case 64: block_sort_static<NT, 6>(a); return;
      case 128: block_sort_static<NT, 7>(a); return;
      case 256: block_sort_static<NT, 8>(a); return;
      case 512: if constexpr (NT >= 512) block_sort_static<NT, 9>(a); return;
      default: if constexpr (NT >= 1024) block_sort_static<NT, 10>(a); return;
    }
  }
  if (P < kWave || P > 4 * NT) {
    block_bitonic_sort<NT>(a, P);
  } else if (P <= NT) {
    block_sort_regs<NT, 1>(a, P);
  } else if (P <= 2 * NT) {
    block_sort_regs<NT, 2>(a, P);
  } else {
    block_sort_regs<NT, 4>(a, P);
  }
}

// Sorts the 64 values held one per lane of a wave descending (lane 0 gets the
// largest).  Wave-level, no barrier.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t a) {
  const int t = lane_id();
#pragma unroll
  for (int lsize = 1; lsize <= 6; ++lsize) {
    const int size = 1 << lsize;
#pragma unroll
    for (int ls = lsize - 1; ls >= 0; --ls) {
      const int s = 1 << ls;
      const uint64_t b = xor_lanes(a, s);
      const bool keep_max = ((t & s) == 0) == ((t & size) == 0);
      a = keep_max ? (a < b ? b : a) : (a < b ? a : b);
    }
  }
  return a;
}

__host__ __device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// ---------------------------------------------------------------- radix select
// Wave 0 of the block: given a 256-bin histogram, find the digit holding the
// `remaining`-th largest element and how many lie strictly above that digit.
__device__ __forceinline__ void wave_pick_digit(const uint32_t* hist, int remaining, int* out_digit,
                                                int* out_above) {
  const int lane = lane_id();
  int c[4];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = (int)hist[255 - 4 * lane - j];
    sum += c[j];
  }
  const int incl = wave_inclusive_scan(sum);
  const int excl = incl - sum;
  if (excl < remaining && remaining <= incl) {
    int cum = excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (cum + c[j] >= remaining) {
        *out_digit = 255 - 4 * lane - j;
        *out_above = cum;
        break;
      }
      cum += c[j];
    }
  }
}

// The rank-th largest (rank >= 1) 64-bit key among the items i in [0, n) for
// which get(i, &key) returns true.  The caller guarantees at least `rank`
// such items.  `hist` needs 256 uint32, `sh` 2 ints.  Barriers inside.
template <int NT, int BITS, typename Get>
__device__ __forceinline__ uint64_t block_kth_largest(int n, int rank, Get get, uint32_t* hist, int* sh) {
  uint64_t prefix = 0;
  int remaining = rank;
  for (int shift = BITS - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    const uint64_t hi_mask = (shift + 8 >= 64) ? 0ull : (~0ull << (shift + 8));
    for (int i = threadIdx.x; i < n; i += NT) {
      uint64_t key;
      if (get(i, &key) && ((key & hi_mask) == (prefix & hi_mask)))
        atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      int digit = 0, above = 0;
      wave_pick_digit(hist, remaining, &digit, &above);
      // exactly one lane found it; spread with a max-reduce
      const auto mx = [](int x, int y) { return x > y ? x : y; };
      const int d = wave_allreduce(digit, mx), a = wave_allreduce(above, mx);
      if (threadIdx.x == 0) {
        sh[0] = d;
        sh[1] = a;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sh[0] << shift;
    remaining -= sh[1];
    __syncthreads();
  }
  return prefix;
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC'11: per round, two 32x32->64 products of counter words 0 and 2 with the
// round constants; the key is bumped by Weyl constants between rounds.  Each
// product is one v_mad_u64_u32; with a wave-uniform key the key schedule
// stays on the scalar unit.
struct Philox4 {
  uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += W0;
    k1 += W1;
  }
  Philox4 out;
  out.v[0] = c0;
  out.v[1] = c1;
  out.v[2] = c2;
  out.v[3] = c3;
  return out;
}

// Standard Gumbel noise from one 32-bit word: U = (w + 1/2) 2^-32, in fp64.
__device__ __forceinline__ double gumbel_from_word(uint32_t w) {
  const double u = ((double)w + 0.5) * 0x1.0p-32;
  return -log(-log(u));
}

}  // namespace mfd
