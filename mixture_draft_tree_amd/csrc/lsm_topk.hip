// Fused per-row log-softmax and top-k over drafter logits [N, K, L, V].
//
// Each of the K block copies gives one distribution per drafted position
// (project page, Figure 2); the tree search needs, per (tree, mode, position)
// row, the log-normaliser and the candidates in rank order (project page,
// "How it works" step 3: best-first searches take each position's tokens from
// most to least probable).  This kernel reads each logit once from HBM.
//
// Design (gfx950, wave64):
//  * One workgroup of 256 threads (4 waves) per row; rows are independent, so
//    the grid is N*K*L workgroups with no cross-workgroup traffic.
//  * 16-byte non-temporal vector loads (8 bf16 or 4 fp32), consecutive lanes on
//    consecutive 16-byte chunks, four per lane per chunk, double-buffered in
//    registers so the next chunk is in flight while one is consumed.
//  * Online log-sum-exp per lane in base 2 (one FMA and one v_exp_f32 per
//    element, fp32 terms summed per vector into an fp64 running sum); lanes,
//    waves and the block are combined in fp64.
//  * Top-k in the same pass.  The first chunk (8192 bf16 elements) is a sample:
//    the block radix-selects the key that should leave about 3k elements of
//    the row above it.  During the stream a lane whose vector maximum reaches
//    that key copies the whole 16-byte vector into its wave's LDS area (slot
//    from ballot + popcount).  At the end the block radix-selects the exact
//    k-th key over the staged elements, gathers those at or above it, and
//    bitonic-sorts them by (key descending, token ascending).
//  * Whenever the guess does not hold (fewer than k elements reach it, a
//    wave's area fills up, or too many ties sit at the k-th key), the row
//    takes an exact multi-pass radix top-k that re-reads the row.  The guess
//    changes speed only, never results.
#include <math.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;
constexpr long long kStep = (long long)kThreads * kUnroll;
constexpr int kOversample = 3;
constexpr float kLog2e = 1.44269504088896340736f;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  using T = uint16_t;
  static constexpr int VEC = 8;
  static constexpr int KEYBITS = 16;
  __device__ static uint32_t key_of_bits(uint32_t b) { return bf16_key(b); }
  __device__ static float val_of_key(uint32_t k) { return bf16_bits_to_f32(bf16_from_key(k)); }
  __device__ static uint32_t bits_at(const T* p, long long i) { return p[i]; }
  __device__ static float val_of_bits(uint32_t b) { return bf16_bits_to_f32(b); }
};
template <>
struct Elem<false> {
  using T = float;
  static constexpr int VEC = 4;
  static constexpr int KEYBITS = 32;
  __device__ static uint32_t key_of_bits(uint32_t b) { return f32_key(b); }
  __device__ static float val_of_key(uint32_t k) { return __uint_as_float(f32_from_key(k)); }
  __device__ static uint32_t bits_at(const T* p, long long i) { return __float_as_uint(p[i]); }
  __device__ static float val_of_bits(uint32_t b) { return __uint_as_float(b); }
};

// Element j of a 16-byte vector (j may be a run-time value), as raw bits / as a float.
template <bool BF16>
__device__ __forceinline__ uint32_t vec_bits(const u32x4& v, int j) {
  const int wi = BF16 ? (j >> 1) : j;
  const uint32_t w = wi == 0 ? v.x : (wi == 1 ? v.y : (wi == 2 ? v.z : v.w));
  if (BF16) return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
  return w;
}
template <bool BF16>
__device__ __forceinline__ float vec_val(const u32x4& v, int j) {
  const uint32_t w = v[BF16 ? (j >> 1) : j];
  if (BF16) return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  return __uint_as_float(w);
}

struct Shared {
  uint32_t thr;     // the row's sampled threshold key
  int overflow;     // the staged guess cannot be used: take the exact fallback
  int cnt[kWaves];  // staged vectors per wave
  int nsurv;
  int sh[4];
  int scan[kWaves];
  float red_m[kWaves];
  double red_s[kWaves];
  double lse;
  uint32_t skey[64];  // head/tail scalars: keys
  uint32_t sidx[64];  //                    and indices
  int nscal;
};

// Smallest non-NaN key (that of -inf) for the element type.
template <bool BF16>
__device__ __forceinline__ uint32_t min_real_key() {
  return BF16 ? 0x007Fu : 0x007FFFFFu;
}

template <bool BF16>
__device__ __forceinline__ float thr_float(uint32_t thr) {
  return thr <= min_real_key<BF16>() ? -INFINITY : Elem<BF16>::val_of_key(thr);
}

// Per-wave staging of candidate vectors.
struct Stager {
  u32x4* svec;     // staged vectors
  uint32_t* sidx;  // index of each staged vector's first element
  int cap;
  int scnt;        // wave-uniform
  float thr_f;     // value of the threshold key (-inf below the smallest real key)
  bool full;       // wave-uniform: a candidate did not fit

  // Wave-level: lanes with `p` stage their vector.
  __device__ __forceinline__ void stage(bool p, const u32x4& v, uint32_t i0) {
    const uint64_t m = __ballot(p);
    if (m == 0ull) return;
    const int n = __popcll(m);
    if (scnt + n > cap) {
      full = true;
      return;
    }
    if (p) {
      const int slot = scnt + __popcll(m & lanemask_lt());
      svec[slot] = v;
      sidx[slot] = i0;
    }
    scnt += n;
  }
};

// Per-lane running log-sum-exp in base 2: s = sum 2^(x*log2e - ml) with
// ml = m*log2e rounded to fp32 (m the lane's running max).  The rounding of ml
// is undone exactly at the end, in fp64; each rise of the maximum costs one
// fp32 rounding of the rescale factor (a few per lane per row).
struct LaneLse {
  float m = -INFINITY;
  float ml = -INFINITY;
  double s = 0.0;

  __device__ __forceinline__ void rescale(float vm) {
    if (vm > m) {
      const float mln = vm * kLog2e;
      s *= (double)__builtin_amdgcn_exp2f(ml - mln);
      m = vm;
      ml = mln;
    }
  }
  __device__ __forceinline__ float bias() const { return (m == -INFINITY) ? 0.f : ml; }
  // sum exp(x - m) in natural units
  __device__ __forceinline__ double natural_sum() const {
    if (m == -INFINITY || m == INFINITY) return s;
    return s * exp2((double)ml - (double)m * (double)kLog2e);
  }
};

template <bool BF16, bool FULL, bool STAGE>
__device__ __forceinline__ void consume_vector(const u32x4& v, uint32_t i0, bool valid, LaneLse& st, Stager& sg) {
  constexpr int VEC = Elem<BF16>::VEC;
  float f[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) f[j] = (FULL || valid) ? vec_val<BF16>(v, j) : -INFINITY;
  float vm = f[0];
#pragma unroll
  for (int j = 1; j < VEC; ++j) vm = fmaxf(vm, f[j]);
  st.rescale(vm);
  const float b = st.bias();
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc += __builtin_amdgcn_exp2f(fmaf(f[j], kLog2e, -b));
  st.s += (double)acc;
  if (STAGE) sg.stage((FULL || valid) && !(vm < sg.thr_f), v, i0);
}

__device__ __forceinline__ void load_chunk(u32x4* buf, const u32x4* vrow, long long c, long long nvec, int tid) {
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    long long q = c * kStep + (long long)u * kThreads + tid;
    q = q < nvec ? q : nvec - 1;  // clamped: every load is valid
    buf[u] = __builtin_nontemporal_load(vrow + q);
  }
}

template <bool BF16, bool STAGE>
__device__ __forceinline__ void consume_chunk(const u32x4* buf, long long c, long long nvec, long long head, int tid,
                                              LaneLse& st, Stager& sg) {
  constexpr int VEC = Elem<BF16>::VEC;
  const long long base = c * kStep;
  if (base + kStep <= nvec) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = base + (long long)u * kThreads + tid;
      consume_vector<BF16, true, STAGE>(buf[u], (uint32_t)(head + q * VEC), true, st, sg);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = base + (long long)u * kThreads + tid;
      consume_vector<BF16, false, STAGE>(buf[u], (uint32_t)(head + q * VEC), q < nvec, st, sg);
    }
  }
}

// Calls f(key, index) for every staged element (and head/tail scalar) whose
// key reaches `thr`.  Block-strided; no barrier.
template <bool BF16, typename F>
__device__ __forceinline__ void for_each_staged(const u32x4* svec_all, const uint32_t* sidx_all, int cap,
                                                const Shared& S, uint32_t thr, F f) {
  constexpr int VEC = Elem<BF16>::VEC;
  for (int i = threadIdx.x; i < kWaves * cap; i += kThreads) {
    const int w = i / cap, j = i - w * cap;
    if (j >= S.cnt[w]) continue;
    const u32x4 v = svec_all[i];
    const uint32_t i0 = sidx_all[i];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const uint32_t key = Elem<BF16>::key_of_bits(vec_bits<BF16>(v, e));
      if (key >= thr) f(key, i0 + e);
    }
  }
  for (int i = threadIdx.x; i < S.nscal; i += kThreads)
    if (S.skey[i] >= thr) f(S.skey[i], S.sidx[i]);
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads, 4) lsm_topk_kernel(const typename Elem<BF16>::T* __restrict__ logits,
                                                               long long V, int k, int cap_w, int sort_cap,
                                                               int rows_per_tree, double* __restrict__ lse_out,
                                                               int32_t* __restrict__ topk_id,
                                                               float* __restrict__ topk_raw,
                                                               float* __restrict__ topk_logp,
                                                               int32_t* __restrict__ status) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int VEC = E::VEC;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  u32x4* svec_all = reinterpret_cast<u32x4*>(smem_raw);
  uint64_t* sortbuf = reinterpret_cast<uint64_t*>(svec_all + (size_t)kWaves * cap_w);
  uint32_t* hist = reinterpret_cast<uint32_t*>(sortbuf + sort_cap);
  uint32_t* sidx_all = hist + 256;
  __shared__ Shared S;

  const int tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const long long row = blockIdx.x;
  const T* rowp = logits + row * V;

  if (tid == 0) {
    S.thr = 0;
    S.overflow = 0;
    S.nsurv = 0;
  }

  Stager sg;
  sg.svec = svec_all + (size_t)wid * cap_w;
  sg.sidx = sidx_all + (size_t)wid * cap_w;
  sg.cap = cap_w;
  sg.scnt = 0;
  sg.thr_f = -INFINITY;
  sg.full = false;

  LaneLse st;

  // Split the row into a scalar head (to 16-byte alignment), aligned vectors
  // and a scalar tail.
  const uintptr_t addr = reinterpret_cast<uintptr_t>(rowp);
  long long head = (long long)(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const long long nvec = (V - head) / VEC;
  const long long tail0 = head + nvec * VEC;
  const int nscalar = (int)(head + (V - tail0));

  // scalars (head / tail, at most 2 * (VEC - 1) < 64): wave 0, one per lane
  if (wid == 0) {
    const bool has = lane < nscalar;
    const long long i = has ? (lane < head ? (long long)lane : tail0 + (lane - head)) : 0;
    const uint32_t bits = has ? E::bits_at(rowp, i) : 0u;
    const float x = has ? E::val_of_bits(bits) : -INFINITY;
    st.rescale(x);
    st.s += (double)__builtin_amdgcn_exp2f(fmaf(x, kLog2e, -st.bias()));
    if (has) {
      S.skey[lane] = E::key_of_bits(bits);
      S.sidx[lane] = (uint32_t)i;
    }
    if (lane == 0) S.nscal = nscalar;
  }
  __syncthreads();

  // Vectors, double-buffered chunks.  Chunk 0 doubles as the sample.
  const u32x4* vrow = reinterpret_cast<const u32x4*>(rowp + head);
  if (nvec > 0) {
    const long long nchunks = (nvec + kStep - 1) / kStep;
    u32x4 bufA[kUnroll], bufB[kUnroll];
    load_chunk(bufA, vrow, 0, nvec, tid);
    load_chunk(bufB, vrow, 1, nvec, tid);
    consume_chunk<BF16, false>(bufA, 0, nvec, head, tid, st, sg);
    // sampled threshold: the r-th largest key of chunk 0, r chosen so that
    // about kOversample * k elements of the row are expected above it
    const long long n0 = (kStep <= nvec ? kStep : nvec) * VEC;
    long long r = (kOversample * (long long)k * n0 + V - 1) / V;
    r = r < 1 ? 1 : (r > n0 ? n0 : r);
    uint32_t prefix = 0;
    int remaining = (int)r;
    for (int shift = E::KEYBITS - 8; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      const uint32_t hi_mask = (shift + 8 >= 32) ? 0u : (~0u << (shift + 8));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const long long q = (long long)u * kThreads + tid;
        if (q < nvec) {
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            const uint32_t key = E::key_of_bits(vec_bits<BF16>(bufA[u], j));
            if ((key & hi_mask) == (prefix & hi_mask)) atomicAdd(&hist[(key >> shift) & 255u], 1u);
          }
        }
      }
      __syncthreads();
      if (wid == 0) {
        int digit = 0, above = 0;
        wave_pick_digit(hist, remaining, &digit, &above);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
          digit = max(digit, __shfl_xor(digit, o, kWave));
          above = max(above, __shfl_xor(above, o, kWave));
        }
        if (tid == 0) {
          S.sh[0] = digit;
          S.sh[1] = above;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)S.sh[0] << shift;
      remaining -= S.sh[1];
      __syncthreads();
    }
    if (tid == 0) S.thr = prefix;
    sg.thr_f = thr_float<BF16>(prefix);
    // stage chunk 0's survivors
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = (long long)u * kThreads + tid;
      float vm = -INFINITY;
#pragma unroll
      for (int j = 0; j < VEC; ++j) vm = fmaxf(vm, vec_val<BF16>(bufA[u], j));
      sg.stage(q < nvec && !(vm < sg.thr_f), bufA[u], (uint32_t)(head + q * VEC));
    }
    for (long long c = 1; c < nchunks; c += 2) {
      load_chunk(bufA, vrow, c + 1, nvec, tid);
      consume_chunk<BF16, true>(bufB, c, nvec, head, tid, st, sg);
      if (c + 1 >= nchunks) break;
      load_chunk(bufB, vrow, c + 2, nvec, tid);
      consume_chunk<BF16, true>(bufA, c + 1, nvec, head, tid, st, sg);
    }
  }
  const float m = st.m;
  const double s = st.natural_sum();

  // ------------------------------------------------------------ log-normaliser
  // m is never NaN (it only moves on `>`); a NaN logit turns s into NaN.
  {
    float mw = m;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) mw = fmaxf(mw, __shfl_xor(mw, o, kWave));
    double sw = s * ((m == -INFINITY) ? 0.0 : exp((double)m - (double)mw));
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) sw += __shfl_xor(sw, o, kWave);
    if (lane == 0) {
      S.red_m[wid] = mw;
      S.red_s[wid] = sw;
      S.cnt[wid] = sg.scnt;
      if (sg.full) S.overflow = 1;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float mb = S.red_m[0];
    for (int w = 1; w < kWaves; ++w) mb = fmaxf(mb, S.red_m[w]);
    double sb = 0.0;
    for (int w = 0; w < kWaves; ++w)
      sb += S.red_s[w] * ((S.red_m[w] == -INFINITY) ? 0.0 : exp((double)S.red_m[w] - (double)mb));
    double l;
    if (mb == -INFINITY) l = (sb == 0.0) ? -INFINITY : NAN;
    else l = (double)mb + log(sb);
    S.lse = l;
    lse_out[row] = l;
    if (status && (isnan(l) || l == INFINITY)) atomicOr(&status[row / rows_per_tree], 1);
  }
  __syncthreads();
  const double lse = S.lse;

  // ------------------------------------------------------------ exact top-k
  if (!S.overflow) {
    // the k-th largest key among the staged elements reaching the threshold
    const uint32_t thr = S.thr;
    uint32_t prefix = 0;
    int remaining = k;
    for (int shift = E::KEYBITS - 8; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      const uint32_t hi_mask = (shift + 8 >= 32) ? 0u : (~0u << (shift + 8));
      for_each_staged<BF16>(svec_all, sidx_all, cap_w, S, thr, [&](uint32_t key, uint32_t) {
        if ((key & hi_mask) == (prefix & hi_mask)) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      });
      __syncthreads();
      if (wid == 0) {
        int tot = 0;
        for (int b = lane; b < 256; b += kWave) tot += (int)hist[b];
        tot = wave_sum(tot);
        int digit = 0, above = 0;
        wave_pick_digit(hist, remaining, &digit, &above);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
          digit = max(digit, __shfl_xor(digit, o, kWave));
          above = max(above, __shfl_xor(above, o, kWave));
        }
        if (tid == 0) {
          S.sh[0] = digit;
          S.sh[1] = above;
          if (shift == E::KEYBITS - 8 && tot < k) S.overflow = 1;  // fewer than k reached the guess
        }
      }
      __syncthreads();
      if (S.overflow) break;
      prefix |= (uint32_t)S.sh[0] << shift;
      remaining -= S.sh[1];
      __syncthreads();
    }
    if (!S.overflow) {
      // gather everything at or above the k-th key (k plus the ties)
      for_each_staged<BF16>(svec_all, sidx_all, cap_w, S, prefix, [&](uint32_t key, uint32_t idx) {
        const int slot = atomicAdd(&S.nsurv, 1);
        if (slot < sort_cap) sortbuf[slot] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - idx);
      });
      __syncthreads();
      if (tid == 0 && S.nsurv > sort_cap) {
        S.overflow = 1;  // too many ties at the k-th key for the sort buffer
        S.nsurv = 0;
      }
      __syncthreads();
    }
  }
  if (S.overflow) {
    // Exact fallback: radix-select the k-th largest key over the row, then
    // take every element above it and the lowest-index ties at it.
    auto getk = [&](int i, uint64_t* out) -> bool {
      *out = E::key_of_bits(E::bits_at(rowp, i));
      return true;
    };
    const uint32_t kk = (uint32_t)block_kth_largest<kThreads, E::KEYBITS>((int)V, k, getk, hist, S.sh);
    if (tid == 0) S.nsurv = 0;
    __syncthreads();
    for (long long i = tid; i < V; i += kThreads) {
      const uint32_t key = E::key_of_bits(E::bits_at(rowp, i));
      if (key > kk) {
        const int slot = atomicAdd(&S.nsurv, 1);
        if (slot < sort_cap) sortbuf[slot] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
      }
    }
    __syncthreads();
    const int taken = S.nsurv;  // elements strictly above the k-th key: fewer than k
    const int need = k - taken;
    int ties_before = 0;
    for (long long b0 = 0; b0 < V && ties_before < need; b0 += kThreads) {
      const long long i = b0 + tid;
      const bool tie = i < V && E::key_of_bits(E::bits_at(rowp, i)) == kk;
      int tot;
      const int r = ties_before + block_exclusive_scan<kThreads>(tie ? 1 : 0, S.scan, &tot);
      if (tie && r < need && taken + r < sort_cap)
        sortbuf[taken + r] = ((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
      ties_before += tot;
    }
    if (tid == 0) S.nsurv = k;
    __syncthreads();
  }
  // sort the survivors (descending composite = key descending, token ascending)
  const int ns = S.nsurv;
  const int P = next_pow2(ns < k ? k : ns);
  for (int i = ns + tid; i < P; i += kThreads) sortbuf[i] = 0ull;
  __syncthreads();
  block_bitonic_sort<kThreads>(sortbuf, P);
  for (int j = tid; j < k; j += kThreads) {
    const uint64_t c = sortbuf[P - 1 - j];
    const uint32_t key = (uint32_t)(c >> 32);
    const uint32_t idx = 0xFFFFFFFFu - (uint32_t)c;
    const float x = E::val_of_key(key);
    const long long o = row * k + j;
    topk_id[o] = (int32_t)idx;
    topk_raw[o] = x;
    if (topk_logp) topk_logp[o] = (float)((double)x - lse);
  }
}

// Staging area per wave: 1.5x the expected survivor vectors of one wave, plus
// one full round of slack.
int wave_cap(int k) {
  int c = (kOversample * k * 3) / (2 * kWaves) + kWave;
  return (c + 63) / 64 * 64;
}

// Sort buffer: k survivors plus room for ties at the k-th key.
int sort_cap_for(int k) { return 2 * next_pow2(k); }

size_t lsm_lds_bytes(int k) {
  return (size_t)kWaves * wave_cap(k) * 16 + (size_t)sort_cap_for(k) * 8 + 256 * 4 +
         (size_t)kWaves * wave_cap(k) * 4 + 64;
}

}  // namespace

hipError_t launch_logsoftmax_topk(const void* logits, bool bf16, int rows, int rows_per_tree, long long V, int k,
                                  double* lse, int32_t* topk_id, float* topk_raw, float* topk_logp,
                                  int32_t* status, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int cap = wave_cap(k);
  const int scap = sort_cap_for(k);
  const size_t lds = lsm_lds_bytes(k);
  if (bf16) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lsm_topk_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lsm_topk_kernel<true>, dim3(rows), dim3(kThreads), lds, stream,
                       static_cast<const uint16_t*>(logits), V, k, cap, scap, rows_per_tree, lse, topk_id, topk_raw,
                       topk_logp, status);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lsm_topk_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lsm_topk_kernel<false>, dim3(rows), dim3(kThreads), lds, stream,
                       static_cast<const float*>(logits), V, k, cap, scap, rows_per_tree, lse, topk_id, topk_raw,
                       topk_logp, status);
  }
  return hipGetLastError();
}

}  // namespace mfd
