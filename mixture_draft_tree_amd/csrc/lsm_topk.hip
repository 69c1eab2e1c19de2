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
//  * 16-byte non-temporal vector loads (8 bf16 or 4 fp32), consecutive lanes
//    on consecutive 16-byte chunks, four per lane per chunk, double-buffered
//    in registers so the next chunk is in flight while one is consumed.
//  * Online log-sum-exp per lane in base 2 (one FMA and one v_exp_f32 per
//    element, fp32 terms summed per vector into an fp64 running sum); lanes,
//    waves and the block are combined in fp64.
//  * Top-k in the same pass.  A lane whose vector maximum reaches the wave's
//    threshold stages the whole 16-byte vector into a small per-wave LDS ring
//    (slot from ballot + popcount: a few instructions per round, however many
//    lanes hold candidates).  When the ring fills, the wave processes the
//    staged vectors 64 at a time (one per lane) and appends the elements whose
//    ordered key reaches the threshold to a per-wave candidate buffer.  When
//    that buffer fills, the wave radix-selects the k-th largest key of its own
//    buffer -- a lower bound on the row's k-th largest, since the buffer holds
//    distinct row elements -- drops what lies below and publishes the value to
//    the other waves (LDS atomicMax).  The threshold only rises; the
//    streaming loop has no block barrier.
//  * At the end the block radix-selects the exact k-th largest composite
//    (key, ~index) over all wave buffers, keeps exactly k, sorts them
//    (bitonic, LDS) and writes ids, values and log-probs.
//  * A buffer that cannot make room (more than ~256 exact ties at the
//    threshold) sends the row to an exact multi-pass radix top-k that
//    re-reads the row.
#include <math.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;
constexpr long long kStep = (long long)kThreads * kUnroll;
constexpr int kStage = 192;      // staged vectors per wave
constexpr int kFlushAt = 64;     // flush after a chunk once this many are staged
constexpr int kOversample = 3;   // the sampled threshold aims at ~3k survivors per row
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

// Element j of a 16-byte vector, as raw bits / as a float.
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
  uint32_t thr;     // shared threshold key (max over waves)
  int overflow;     // a wave lost candidates
  int cnt[kWaves];  // final per-wave candidate counts
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
  uint64_t* cand;   // candidate buffer (composite keys)
  uint32_t* hist;   // 256-bin histogram
  u32x4* svec;      // staged vectors
  uint32_t* sidx;   // element index of each staged vector's first element
  int cap;
  int k;
  int cnt;          // wave-uniform
  int scnt;         // wave-uniform
  uint32_t thr;     // wave-uniform threshold key
  float thr_f;      // its value (-inf below the smallest real key)
  bool overflow;    // wave-uniform

  __device__ __forceinline__ void raise(uint32_t t) {
    if (t > thr) {
      thr = t;
      thr_f = thr_float<BF16>(t);
    }
  }

  // Raise the threshold to the k-th largest key in the candidate buffer and
  // drop everything below it.  Wave-synchronous.
  __device__ __forceinline__ void compact(uint32_t* shared_thr) {
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
    raise(prefix);
    if (lane == 0) atomicMax(shared_thr, prefix);
  }

  // Wave-level append: every lane offers at most one element.
  __device__ __forceinline__ void append(bool has, uint32_t key, uint32_t idx, uint32_t* shared_thr) {
    bool p = has && key >= thr;
    uint64_t m = __ballot(p);
    if (m == 0ull || overflow) return;
    if (cnt + kWave > cap) {
      compact(shared_thr);
      p = has && key >= thr;
      m = __ballot(p);
      if (m == 0ull) return;
      if (cnt + kWave > cap) {
        overflow = true;
        return;
      }
    }
    if (p) cand[cnt + __popcll(m & lanemask_lt())] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - idx);
    cnt += __popcll(m);
  }

  // Process the staged vectors, 64 at a time (one per lane).
  __device__ __forceinline__ void flush(uint32_t* shared_thr) {
    constexpr int VEC = Elem<BF16>::VEC;
    const int lane = lane_id();
    wave_sync();
    for (int b = 0; b < scnt; b += kWave) {
      const int i = b + lane;
      const bool has = i < scnt;
      const u32x4 v = has ? svec[i] : u32x4{0u, 0u, 0u, 0u};
      const uint32_t i0 = has ? sidx[i] : 0u;
#pragma unroll 1
      for (int j = 0; j < VEC; ++j) {
        const int wi = BF16 ? (j >> 1) : j;
        const uint32_t w = wi == 0 ? v.x : (wi == 1 ? v.y : (wi == 2 ? v.z : v.w));
        const uint32_t bits = BF16 ? ((j & 1) ? (w >> 16) : (w & 0xFFFFu)) : w;
        append(has, Elem<BF16>::key_of_bits(bits), i0 + j, shared_thr);
      }
    }
    wave_sync();
    scnt = 0;
  }

  // Wave-level: lanes with `p` stage their vector.  The caller flushes after
  // each chunk once kFlushAt are staged; a ring that still fills marks the
  // row for the exact fallback.
  __device__ __forceinline__ void stage(bool p, const u32x4& v, uint32_t i0) {
    const uint64_t m = __ballot(p);
    if (m == 0ull) return;
    const int n = __popcll(m);
    if (scnt + n > kStage) {
      overflow = true;
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
      s *= (double)__builtin_amdgcn_exp2f(ml - mln);  // one fp32 rounding per new maximum
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

template <bool BF16, bool FULL, bool STAGE = true>
__device__ __forceinline__ void consume_vector(const u32x4& v, uint32_t i0, bool valid, LaneLse& st, WaveTopk<BF16>& wt) {
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
  if (STAGE) wt.stage((FULL || valid) && !(vm < wt.thr_f), v, i0);
}

__device__ __forceinline__ void load_chunk(u32x4* buf, const u32x4* vrow, long long c, long long nvec, int tid) {
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    long long q = c * kStep + (long long)u * kThreads + tid;
    q = q < nvec ? q : nvec - 1;  // clamped: every load is valid
    buf[u] = __builtin_nontemporal_load(vrow + q);
  }
}

template <bool BF16>
__device__ __forceinline__ void consume_chunk(const u32x4* buf, long long c, long long nvec, long long head, int tid,
                                              LaneLse& st, WaveTopk<BF16>& wt, uint32_t* shared_thr) {
  constexpr int VEC = Elem<BF16>::VEC;
  wt.raise(*shared_thr);
  const long long base = c * kStep;
  if (base + kStep <= nvec) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = base + (long long)u * kThreads + tid;
      consume_vector<BF16, true>(buf[u], (uint32_t)(head + q * VEC), true, st, wt);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = base + (long long)u * kThreads + tid;
      consume_vector<BF16, false>(buf[u], (uint32_t)(head + q * VEC), q < nvec, st, wt);
    }
  }
  if (wt.scnt >= kFlushAt) wt.flush(shared_thr);
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads, 4) lsm_topk_kernel(const typename Elem<BF16>::T* __restrict__ logits,
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
  u32x4* svec_all = reinterpret_cast<u32x4*>(smem_raw);
  uint64_t* cand_all = reinterpret_cast<uint64_t*>(svec_all + kWaves * kStage);
  uint32_t* hist_all = reinterpret_cast<uint32_t*>(cand_all + (size_t)kWaves * cap_w);
  uint32_t* sidx_all = hist_all + kWaves * 256;
  const int kp = next_pow2(k);
  uint64_t* sortbuf = reinterpret_cast<uint64_t*>(sidx_all + kWaves * kStage);
  __shared__ Shared S;

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
  wt.svec = svec_all + wid * kStage;
  wt.sidx = sidx_all + wid * kStage;
  wt.cap = cap_w;
  wt.k = k;
  wt.cnt = 0;
  wt.scnt = 0;
  wt.thr = 0;
  wt.thr_f = -INFINITY;
  wt.overflow = false;

  LaneLse st;

  // Split the row into a scalar head (to 16-byte alignment), aligned vectors
  // and a scalar tail.
  const uintptr_t addr = reinterpret_cast<uintptr_t>(rowp);
  long long head = (long long)(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const long long nvec = (V - head) / VEC;
  const long long tail0 = head + nvec * VEC;
  const int nscalar = (int)(head + (V - tail0));

  // Vectors, double-buffered chunks.  Chunk 0 doubles as a sample: the block
  // picks a threshold key such that about kOversample * k elements of the row
  // are expected above it; if fewer than k turn out to be, the row takes the
  // exact fallback below, so the guess affects speed only.
  const u32x4* vrow = reinterpret_cast<const u32x4*>(rowp + head);
  if (nvec > 0) {
    const long long nchunks = (nvec + kStep - 1) / kStep;
    u32x4 bufA[kUnroll], bufB[kUnroll];
    load_chunk(bufA, vrow, 0, nvec, tid);
    load_chunk(bufB, vrow, 1, nvec, tid);
    const bool full0 = kStep <= nvec;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = (long long)u * kThreads + tid;
      if (full0) consume_vector<BF16, true, false>(bufA[u], (uint32_t)(head + q * VEC), true, st, wt);
      else consume_vector<BF16, false, false>(bufA[u], (uint32_t)(head + q * VEC), q < nvec, st, wt);
    }
    // sampled threshold: the r-th largest key of chunk 0
    const long long n0 = (full0 ? kStep : nvec) * VEC;
    long long r = (kOversample * (long long)k * n0 + V - 1) / V;
    r = r < 1 ? 1 : (r > n0 ? n0 : r);
    uint32_t prefix = 0;
    int remaining = (int)r;
    for (int shift = E::KEYBITS - 8; shift >= 0; shift -= 8) {
      hist_all[tid] = 0;
      __syncthreads();
      const uint32_t hi_mask = (shift + 8 >= 32) ? 0u : (~0u << (shift + 8));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const long long q = (long long)u * kThreads + tid;
        if (q < nvec) {
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            const uint32_t key = E::key_of_bits(vec_bits<BF16>(bufA[u], j));
            if ((key & hi_mask) == (prefix & hi_mask)) atomicAdd(&hist_all[(key >> shift) & 255u], 1u);
          }
        }
      }
      __syncthreads();
      if (wid == 0) {
        int digit = 0, above = 0;
        wave_pick_digit(hist_all, remaining, &digit, &above);
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
    wt.raise(prefix);
    if (tid == 0) S.thr = prefix;
    // stage chunk 0's survivors
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = (long long)u * kThreads + tid;
      const bool valid = q < nvec;
      float vm = -INFINITY;
#pragma unroll
      for (int j = 0; j < VEC; ++j) vm = fmaxf(vm, vec_val<BF16>(bufA[u], j));
      wt.stage(valid && !(vm < wt.thr_f), bufA[u], (uint32_t)(head + q * VEC));
    }
    if (wt.scnt >= kFlushAt) wt.flush(&S.thr);
    for (long long c = 1; c < nchunks; c += 2) {
      load_chunk(bufA, vrow, c + 1, nvec, tid);
      consume_chunk<BF16>(bufB, c, nvec, head, tid, st, wt, &S.thr);
      if (c + 1 >= nchunks) break;
      load_chunk(bufB, vrow, c + 2, nvec, tid);
      consume_chunk<BF16>(bufA, c + 1, nvec, head, tid, st, wt, &S.thr);
    }
  }

  // scalars (head / tail, at most 2 * (VEC - 1) < 64): wave 0, one per lane
  if (wid == 0) {
    wt.raise(S.thr);
    const bool has = lane < nscalar;
    const long long i = has ? (lane < head ? (long long)lane : tail0 + (lane - head)) : 0;
    const uint32_t bits = has ? E::bits_at(rowp, i) : 0u;
    const float x = has ? E::val_of_bits(bits) : -INFINITY;
    st.rescale(x);
    st.s += (double)__builtin_amdgcn_exp2f(fmaf(x, kLog2e, -st.bias()));
    wt.append(has, E::key_of_bits(bits), (uint32_t)i, &S.thr);
  }
  if (wt.scnt > 0) wt.flush(&S.thr);
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
  int total = 0;
  for (int w = 0; w < kWaves; ++w) total += S.cnt[w];
  if (!S.overflow && total >= k) {
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
    const int taken = S.nsurv;  // elements strictly above the k-th key
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

// Candidate buffer per wave: k survivors, up to ~256 ties at the threshold,
// and room for one append round (64).
int wave_cap(int k) {
  int c = k + 256 + kWave;
  return (c + 63) / 64 * 64;
}

size_t lsm_lds_bytes(int k) {
  const int cap = wave_cap(k);
  return (size_t)kWaves * kStage * 16 + (size_t)kWaves * cap * 8 + (size_t)kWaves * 256 * 4 +
         (size_t)kWaves * kStage * 4 + (size_t)next_pow2(k) * 8 + 64;
}

}  // namespace

hipError_t launch_logsoftmax_topk(const void* logits, bool bf16, int rows, int rows_per_tree, long long V, int k,
                                  double* lse, int32_t* topk_id, float* topk_raw, float* topk_logp,
                                  int32_t* status, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int cap = wave_cap(k);
  const size_t lds = lsm_lds_bytes(k);
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
