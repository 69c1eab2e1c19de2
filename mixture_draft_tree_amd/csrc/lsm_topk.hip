// Fused per-row log-softmax and top-k over drafter logits [N, K, L, V].
//
// Each of the K block copies gives one distribution per drafted position
// (project page, Figure 2); the tree search needs, per (tree, mode, position)
// row, the log-normaliser and the candidates in rank order (project page,
// "How it works" step 3: best-first searches take each position's tokens from
// most to least probable).  This kernel reads each logit exactly once from
// HBM.
//
// Design (gfx950, wave64):
//  * One workgroup of 256 threads (4 waves) per row; rows are independent, so
//    the grid is N*K*L workgroups and no cross-workgroup traffic exists.
//  * 16-byte vector loads (8 bf16 or 4 fp32), four in flight per lane, with
//    consecutive lanes on consecutive 16-byte chunks.
//  * Online max / sum-of-exp per lane (fp32 exps summed per vector, the
//    running sum kept in fp64), reduced at the end in fp64.
//  * Top-k in the same pass: every wave keeps a private candidate buffer in
//    LDS holding elements whose ordered key reaches a threshold.  The
//    threshold only rises: when a buffer fills, the wave radix-selects the
//    k-th largest key of its own buffer (a lower bound on the row's k-th
//    largest, since the buffer holds distinct row elements), drops what is
//    below, and publishes the value to the other waves through an LDS
//    atomicMax.  Appends use ballot + popcount, so the streaming loop has no
//    block barrier.  The common case per vector is one float compare of the
//    vector max against the threshold.
//  * At the end the block radix-selects the exact k-th largest composite
//    (key, ~index) over all wave buffers, keeps exactly k, sorts them
//    (bitonic, LDS) and writes ids, values and log-probs.
//  * If a buffer cannot make room (more than ~256 exact ties at the
//    threshold), the row falls back to an exact multi-pass radix top-k that
//    re-reads the row.
#include <math.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;

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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Element j of a 16-byte vector, as raw bits.
template <bool BF16>
__device__ __forceinline__ uint32_t vec_bits(const u32x4& v, int j) {
  const uint32_t w = v[BF16 ? (j >> 1) : j];
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
  uint32_t thr;        // shared threshold key (max over waves)
  int overflow;        // a wave lost candidates
  int cnt[kWaves];     // final per-wave candidate counts
  int nsurv;
  int sh[4];
  int scan[kWaves];
  float red_m[kWaves];
  double red_s[kWaves];
  double lse;
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

template <bool BF16>
struct WaveTopk {
  uint64_t* cand;   // this wave's buffer
  uint32_t* hist;   // this wave's 256-bin histogram
  int cap;
  int k;
  int cnt;          // wave-uniform
  uint32_t thr;     // wave-uniform
  bool overflow;    // wave-uniform

  // Raise the threshold to the k-th largest key in this wave's buffer and drop
  // everything below it.  Wave-synchronous; no block barrier.
  __device__ void compact(uint32_t* shared_thr) {
    if (cnt < k) return;
    const int lane = lane_id();
    uint32_t prefix = 0;
    int remaining = k;
    for (int shift = Elem<BF16>::KEYBITS - 8; shift >= 0; shift -= 8) {
      for (int b = lane; b < 256; b += kWave) hist[b] = 0;
      wave_sync();
      const uint32_t hi_mask = (shift + 8 >= 32) ? 0u : (~0u << (shift + 8));
      for (int i = lane; i < cnt; i += kWave) {
        const uint32_t key = (uint32_t)(cand[i] >> 32);
        if ((key & hi_mask) == (prefix & hi_mask)) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      wave_sync();
      int digit = 0, above = 0;
      wave_pick_digit(hist, remaining, &digit, &above);
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        digit = max(digit, __shfl_xor(digit, o, kWave));
        above = max(above, __shfl_xor(above, o, kWave));
      }
      prefix |= (uint32_t)digit << shift;
      remaining -= above;
      wave_sync();
    }
    // keep key >= prefix, in place (writes never pass the chunk being read)
    int w = 0;
    for (int base = 0; base < cnt; base += kWave) {
      const int i = base + lane;
      const uint64_t c = (i < cnt) ? cand[i] : 0ull;
      const bool keep = (i < cnt) && ((uint32_t)(c >> 32) >= prefix);
      const uint64_t m = __ballot(keep);
      wave_sync();
      if (keep) cand[w + __popcll(m & lanemask_lt())] = c;
      w += __popcll(m);
      wave_sync();
    }
    cnt = w;
    if (prefix > thr) thr = prefix;
    if (lane == 0) atomicMax(shared_thr, prefix);
  }

  // Offer one element per lane (`take` false for lanes without one).
  __device__ __forceinline__ void offer(bool has, uint32_t key, uint32_t idx, uint32_t* shared_thr) {
    bool p = has && key >= thr;
    uint64_t m = __ballot(p);
    if (m == 0) return;
    if (overflow) return;
    if (cnt + kWave > cap) {
      compact(shared_thr);
      p = has && key >= thr;
      m = __ballot(p);
      if (m == 0) return;
      if (cnt + kWave > cap) {
        overflow = true;
        return;
      }
    }
    if (p) cand[cnt + __popcll(m & lanemask_lt())] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - idx);
    cnt += __popcll(m);
  }
};

template <bool BF16>
__global__ void __launch_bounds__(kThreads) lsm_topk_kernel(const typename Elem<BF16>::T* __restrict__ logits,
                                                            long long V, int k, int cap_w, int rows_per_tree,
                                                            double* __restrict__ lse_out,
                                                            int32_t* __restrict__ topk_id,
                                                            float* __restrict__ topk_raw,
                                                            float* __restrict__ topk_logp,
                                                            int32_t* __restrict__ status) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int VEC = E::VEC;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint64_t* cand_all = reinterpret_cast<uint64_t*>(smem_raw);
  uint32_t* hist_all = reinterpret_cast<uint32_t*>(cand_all + (size_t)kWaves * cap_w);
  const int kp = next_pow2(k);
  uint64_t* sortbuf = reinterpret_cast<uint64_t*>(hist_all + kWaves * 256);
  Shared& S = *reinterpret_cast<Shared*>(sortbuf + kp);

  const int tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const long long row = blockIdx.x;
  const T* rowp = logits + row * V;

  if (tid == 0) {
    S.thr = 0;
    S.overflow = 0;
    S.nsurv = 0;
  }
  __syncthreads();

  WaveTopk<BF16> wt;
  wt.cand = cand_all + (size_t)wid * cap_w;
  wt.hist = hist_all + wid * 256;
  wt.cap = cap_w;
  wt.k = k;
  wt.cnt = 0;
  wt.thr = 0;
  wt.overflow = false;

  float m = -INFINITY;  // per-lane running max
  double s = 0.0;       // per-lane sum of exp(x - m)

  // Split the row into a scalar head (to 16-byte alignment), aligned vectors
  // and a scalar tail.
  const uintptr_t addr = reinterpret_cast<uintptr_t>(rowp);
  long long head = (long long)(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const long long nvec = (V - head) / VEC;
  const long long tail0 = head + nvec * VEC;
  const int nscalar = (int)(head + (V - tail0));

  // scalars: wave 0, one per lane (at most 2 * (VEC - 1) < 64)
  if (wid == 0) {
    const bool has = lane < nscalar;
    const long long i = has ? (lane < head ? (long long)lane : tail0 + (lane - head)) : 0;
    uint32_t bits = has ? E::bits_at(rowp, i) : 0u;
    const float x = has ? E::val_of_bits(bits) : -INFINITY;
    if (x > m) {
      s *= (double)__expf(m - x);
      m = x;
    }
    s += (double)__expf(x - (m == -INFINITY ? 0.f : m));
    wt.offer(has, E::key_of_bits(bits), (uint32_t)i, &S.thr);
  }

  const u32x4* vrow = reinterpret_cast<const u32x4*>(rowp + head);
  const long long step = (long long)kThreads * kUnroll;
  for (long long base = 0; base < nvec; base += step) {
    u32x4 buf[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = base + (long long)u * kThreads + tid;
      if (q < nvec) buf[u] = __builtin_nontemporal_load(vrow + q);
      else buf[u] = u32x4{0u, 0u, 0u, 0u};
    }
    {
      const uint32_t st = *(volatile uint32_t*)&S.thr;
      if (st > wt.thr) wt.thr = st;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = base + (long long)u * kThreads + tid;
      const bool valid = q < nvec;
      float f[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) f[j] = valid ? vec_val<BF16>(buf[u], j) : -INFINITY;
      float vm = f[0];
#pragma unroll
      for (int j = 1; j < VEC; ++j) vm = fmaxf(vm, f[j]);
      if (vm > m) {
        s *= (double)__expf(m - vm);
        m = vm;
      }
      {
        const float mm = (m == -INFINITY) ? 0.f : m;  // every f is -inf then
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc += __expf(f[j] - mm);
        s += (double)acc;
      }
      // top-k filter: one compare per vector in the common case
      const bool maybe = valid && !(vm < thr_float<BF16>(wt.thr));
      if (__ballot(maybe) != 0ull) {
        const long long i0 = head + q * VEC;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const uint32_t key = E::key_of_bits(vec_bits<BF16>(buf[u], j));
          wt.offer(valid, key, (uint32_t)(i0 + j), &S.thr);
        }
      }
    }
  }

  // ------------------------------------------------------------ log-normaliser
  // m is never NaN (it only moves on `>`); a NaN or +inf logit turns s into NaN.
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
      S.cnt[wid] = wt.cnt;
      if (wt.overflow) S.overflow = 1;
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
  constexpr int CBITS = E::KEYBITS + 32;
  if (!S.overflow) {
    auto get = [&](int i, uint64_t* out) -> bool {
      const int w = i / cap_w, j = i - w * cap_w;
      if (j >= S.cnt[w]) return false;
      *out = cand_all[i];
      return true;
    };
    const uint64_t ck = block_kth_largest<kThreads, CBITS>(kWaves * cap_w, k, get, hist_all, S.sh);
    for (int i = tid; i < kWaves * cap_w; i += kThreads) {
      const int w = i / cap_w, j = i - w * cap_w;
      if (j < S.cnt[w] && cand_all[i] >= ck) {
        const int slot = atomicAdd(&S.nsurv, 1);
        if (slot < kp) sortbuf[slot] = cand_all[i];
      }
    }
  } else {
    // Exact fallback: radix-select the k-th largest key over the row, then
    // take every element above it and the lowest-index ties at it.
    auto getk = [&](int i, uint64_t* out) -> bool {
      *out = E::key_of_bits(E::bits_at(rowp, i));
      return true;
    };
    const uint32_t kk = (uint32_t)block_kth_largest<kThreads, E::KEYBITS>((int)V, k, getk, hist_all, S.sh);
    for (long long i = tid; i < V; i += kThreads) {
      const uint32_t key = E::key_of_bits(E::bits_at(rowp, i));
      if (key > kk) {
        const int slot = atomicAdd(&S.nsurv, 1);
        if (slot < kp) sortbuf[slot] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
      }
    }
    __syncthreads();
    int taken = S.nsurv;  // elements strictly above the k-th key
    const int need = k - taken;
    int ties_before = 0;
    for (long long b0 = 0; b0 < V && ties_before < need; b0 += kThreads) {
      const long long i = b0 + tid;
      const bool tie = i < V && E::key_of_bits(E::bits_at(rowp, i)) == kk;
      int tot;
      const int r = ties_before + block_exclusive_scan<kThreads>(tie ? 1 : 0, S.scan, &tot);
      if (tie && r < need && taken + r < kp)
        sortbuf[taken + r] = ((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
      ties_before += tot;
    }
  }
  __syncthreads();
  for (int i = k + tid; i < kp; i += kThreads) sortbuf[i] = 0ull;
  __syncthreads();
  block_bitonic_sort<kThreads>(sortbuf, kp);
  for (int j = tid; j < k; j += kThreads) {
    const uint64_t c = sortbuf[kp - 1 - j];
    const uint32_t key = (uint32_t)(c >> 32);
    const uint32_t idx = 0xFFFFFFFFu - (uint32_t)c;
    const float x = E::val_of_key(key);
    const long long o = row * k + j;
    topk_id[o] = (int32_t)idx;
    topk_raw[o] = x;
    if (topk_logp) topk_logp[o] = (float)((double)x - lse);
  }
}

int wave_cap(int k, bool bf16) {
  const int vec = bf16 ? 8 : 4;
  int c = k + kWave * vec + 256;
  return (c + 63) / 64 * 64;
}

size_t lsm_lds_bytes(int k, bool bf16) {
  const int cap = wave_cap(k, bf16);
  return (size_t)kWaves * cap * 8 + (size_t)kWaves * 256 * 4 + (size_t)next_pow2(k) * 8 + sizeof(Shared) + 64;
}

}  // namespace

hipError_t launch_logsoftmax_topk(const void* logits, bool bf16, int rows, int rows_per_tree, long long V, int k,
                                  double* lse, int32_t* topk_id, float* topk_raw, float* topk_logp,
                                  int32_t* status, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int cap = wave_cap(k, bf16);
  const size_t lds = lsm_lds_bytes(k, bf16);
  if (bf16) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lsm_topk_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lsm_topk_kernel<true>, dim3(rows), dim3(kThreads), lds, stream,
                       static_cast<const uint16_t*>(logits), V, k, cap, rows_per_tree, lse, topk_id, topk_raw,
                       topk_logp, status);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lsm_topk_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lsm_topk_kernel<false>, dim3(rows), dim3(kThreads), lds, stream,
                       static_cast<const float*>(logits), V, k, cap, rows_per_tree, lse, topk_id, topk_raw,
                       topk_logp, status);
  }
  return hipGetLastError();
}

}  // namespace mfd
