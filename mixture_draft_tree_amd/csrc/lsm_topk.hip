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
//  * The first two chunks (16384 bf16 elements, already in registers when the
//    stream starts) are a sample.  Their maximum M0 fixes the exponent bias of
//    the whole row: every element adds 2^(x*log2e - M0*log2e) (one FMA and one
//    v_exp_f32), summed pairwise in fp32 per chunk and in fp64 across chunks;
//    no running maximum, no rescaling.  If that sum overflows or underflows
//    (the row maximum lies far from M0), it is redone with the true maximum.
//  * The r-th largest of the 256 lanes' sample maxima (a bitwise search on
//    ballot counts) is a threshold that leaves, with high probability, between
//    k and a few k elements of the row at or above it.  During the stream a
//    lane whose vector's term sum reaches that of the threshold copies the
//    whole 16-byte vector into its wave's LDS area (slot from ballot +
//    popcount), or into a shared pool once that area is full.
//  * At the end the staged elements that reach the threshold are compacted
//    into a candidate list, the block radix-selects the exact k-th key over
//    it, gathers the candidates at or above it (k plus ties) and sorts them by
//    (key descending, token ascending), mostly in registers.
//  * Whenever the guess does not hold the row still gets the exact answer:
//    too many candidates -> select straight from the staged vectors; fewer
//    than k, or the staging space overflowed -> a radix top-k over the row,
//    streamed again with the same vector loads.  The guess changes speed only,
//    never results.
#include <math.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;
constexpr long long kStep = (long long)kThreads * kUnroll;
// Chunks at the head of the row that form the sample (2 or 3; all three chunk
// buffers are in flight before the sample is taken).
constexpr int kSampleChunks = 2;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLn2 = 0.693147180559945309417232121458;
// LDS one workgroup may use (of 160 KB per CU), static part included.
constexpr size_t kMaxLds = 156 * 1024;

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
  __device__ static uint32_t key_of_float(float x) { return bf16_key(__float_as_uint(x) >> 16); }
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
  __device__ static uint32_t key_of_float(float x) { return f32_key(__float_as_uint(x)); }
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

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ float term(float x, float bias) {
  return __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -bias));
}

// Rank of the sample threshold among the lanes' sample maxima.  The number of
// row elements at or above the r-th largest of n0 sampled ones is about
// (V / n0) * Gamma(r); r is the smallest value whose mean minus 3 standard
// deviations still reaches k.  (The r-th largest lane maximum lies at or below
// the r-th largest sampled element, so the true margin is wider.)  A row that
// still ends up with fewer than k takes the exact fallback, which costs a few
// more passes over that row only; a wider margin would stage more elements on
// every row.  Host and device use the same formula.
__host__ __device__ __forceinline__ int sample_rank(long long V, long long n0, int k) {
  const double a = (double)k * (double)n0 / (double)V;
  const double sr = 0.5 * (3.0 + sqrt(9.0 + 4.0 * a));
  long long r = (long long)ceil(sr * sr);
  if (r < 1) r = 1;
  if (r > kThreads) r = kThreads;
  return (int)r;
}

struct Shared {
  int overflow;         // the staged guess cannot be used: take the exact fallback
  int cnt[kWaves];      // staged vectors per wave
  int pool;             // pool slots handed out (may exceed the pool on overflow)
  uint32_t fail_at;     // index of the first element whose vector found no room
  int nsurv;
  int ncand;
  int sh[4];
  int scan[kWaves];
  float red_max[kWaves];
  double red_s[kWaves];
  uint32_t skey[64];    // head/tail scalars: keys
  uint32_t sidx[64];    //                    and indices
  int nscal;
  uint32_t hist[256];   // radix histogram; the lanes' sample keys before that
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

// Staging of candidate vectors: a wave's own area first, then the shared pool.
struct Stager {
  u32x4* svec;     // own area: staged vectors
  uint32_t* sidx;  //           index of each staged vector's first element
  u32x4* pvec;     // shared pool
  uint32_t* pidx;
  int* pool_used;
  uint32_t* fail_at;
  int pool_cap;
  int cap;
  int scnt;        // wave-uniform
  bool full;       // wave-uniform: a candidate did not fit

  // Wave-level: lanes with `p` stage their vector, whose first element has
  // index ibase + ioff.
  __device__ __forceinline__ void stage(bool p, const u32x4& v, uint32_t ibase, uint32_t ioff) {
    if (full) return;  // the row is staged again anyway
    const uint64_t m = __ballot(p);
    if (m == 0ull) return;
    const int n = __popcll(m);
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const uint32_t i0 = ibase + ioff;
    if (scnt + n <= cap) {
      if (p) {
        svec[scnt + rank] = v;
        sidx[scnt + rank] = i0;
      }
      scnt = __builtin_amdgcn_readfirstlane(scnt + n);
      return;
    }
    int base = 0;
    if (lane_id() == 0) base = atomicAdd(pool_used, n);
    base = __builtin_amdgcn_readfirstlane(base);
    if (base + n > pool_cap) {
      if (lane_id() == 0) atomicMin(fail_at, ibase);
      full = true;
      return;
    }
    if (p) {
      pvec[base + rank] = v;
      pidx[base + rank] = i0;
    }
  }
};

// One vector: returns the sum of its terms (pairwise, fp32) and stages the
// vector if one of its two half sums (the last two partial sums of the
// pairwise tree) reaches tau.  With tau = 0.999 * term(threshold) this keeps
// every vector holding an element at or above the threshold: such an
// element's term is at least term(threshold) up to an ulp or two of exp2, and
// the other terms of its half are not negative.  Testing the halves rather
// than the whole sum stages far fewer vectors whose elements all lie below
// the threshold (several medium terms that add up), for one v_max.  (NaN
// terms stage nothing from their half.)
template <bool BF16, bool FULL>
__device__ __forceinline__ float consume_vector(const u32x4& v, uint32_t ibase, uint32_t ioff, bool valid, float bias,
                                                float tau, Stager& sg) {
  constexpr int VEC = Elem<BF16>::VEC;
  float e[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) e[j] = (FULL || valid) ? term(vec_val<BF16>(v, j), bias) : 0.f;
#pragma unroll
  for (int w = VEC / 2; w > 1; w >>= 1) {
#pragma unroll
    for (int j = 0; j < w; ++j) e[j] += e[j + w];
  }
  sg.stage((FULL || valid) && fmaxf(e[0], e[1]) >= tau, v, ibase, ioff);
  return e[0] + e[1];
}

// Loads chunk c (four 16-byte vectors per lane).  Byte offsets are 32-bit
// and clamped to the row's last vector, so every load is in bounds and there
// is no branch between the loads of the two buffers.
__device__ __forceinline__ void load_chunk(u32x4* buf, const u32x4* vrow, long long c, uint32_t last_byte, int tid) {
  const uint32_t cbyte = (uint32_t)(c * kStep) * (uint32_t)sizeof(u32x4);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t off = min(cbyte + (uint32_t)((u * kThreads + tid) * (int)sizeof(u32x4)), last_byte);
    buf[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(vrow) + off));
  }
}

template <bool BF16>
__device__ __forceinline__ float consume_chunk(const u32x4* buf, long long c, long long nvec, long long head, int tid,
                                               float bias, float tau, Stager& sg) {
  constexpr int VEC = Elem<BF16>::VEC;
  const long long base = c * kStep;
  const uint32_t ibase = (uint32_t)(head + base * VEC);
  float t[kUnroll];
  if (base + kStep <= nvec) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      t[u] = consume_vector<BF16, true>(buf[u], ibase, (uint32_t)((u * kThreads + tid) * VEC), true, bias, tau, sg);
  } else {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = base + (long long)u * kThreads + tid;
      t[u] = consume_vector<BF16, false>(buf[u], ibase, (uint32_t)((u * kThreads + tid) * VEC), q < nvec, bias, tau,
                                         sg);
    }
  }
  return (t[0] + t[1]) + (t[2] + t[3]);
}

// Streams the row's aligned vectors once more (same loads as the main pass)
// and calls f(v, q, valid) for each lane's vector q.  Every lane of the block
// makes the same calls, so f may use wave-level operations.
template <typename F>
__device__ __forceinline__ void stream_vectors(const u32x4* vrow, long long nvec, int tid, F f) {
  if (nvec <= 0) return;
  const long long nchunks = (nvec + kStep - 1) / kStep;
  const uint32_t last_byte = (uint32_t)(nvec - 1) * (uint32_t)sizeof(u32x4);
  u32x4 a[kUnroll], b[kUnroll];
  load_chunk(a, vrow, 0, last_byte, tid);
  for (long long c = 0; c < nchunks; c += 2) {
    load_chunk(b, vrow, c + 1, last_byte, tid);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = c * kStep + (long long)u * kThreads + tid;
      f(a[u], q, q < nvec);
    }
    if (c + 1 >= nchunks) break;
    load_chunk(a, vrow, c + 2, last_byte, tid);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = (c + 1) * kStep + (long long)u * kThreads + tid;
      f(b[u], q, q < nvec);
    }
  }
}

// Appends the composites of the lanes with `p` to buf[*counter ...] (entries
// past `cap` are counted but not written).  Wave-level, whole wave active; one
// LDS atomic per wave.
__device__ __forceinline__ void wave_append(bool p, uint64_t c, uint64_t* buf, int cap, int* counter) {
  const uint64_t m = __ballot(p);
  int base = 0;
  if (lane_id() == 0 && m) base = atomicAdd(counter, __popcll(m));
  base = __builtin_amdgcn_readfirstlane(base);
  const int pos = base + __popcll(m & lanemask_lt());
  if (p && pos < cap) buf[pos] = c;
}

// Wave 0 helper of the radix selections: digit of the `remaining`-th largest
// key in S.hist and the count above it, into S.sh[0..1].
__device__ __forceinline__ void pick_digit_into(Shared& S, int remaining) {
  int digit = 0, above = 0;
  wave_pick_digit(S.hist, remaining, &digit, &above);
  const auto mx = [](int x, int y) { return x > y ? x : y; };
  digit = wave_allreduce(digit, mx);
  above = wave_allreduce(above, mx);
  if (lane_id() == 0) {
    S.sh[0] = digit;
    S.sh[1] = above;
  }
}

// Exact k-th largest key of the whole row (vectors streamed again, scalars
// from S).  Barriers inside; every thread returns the same key.
template <bool BF16>
__device__ __forceinline__ uint32_t row_kth_largest(const u32x4* vrow, long long nvec, int k, Shared& S) {
  using E = Elem<BF16>;
  constexpr int VEC = E::VEC;
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  int remaining = k;
  for (int shift = E::KEYBITS - 8; shift >= 0; shift -= 8) {
    S.hist[tid] = 0;
    __syncthreads();
    const uint32_t hi_mask = (shift + 8 >= 32) ? 0u : (~0u << (shift + 8));
    const uint32_t want = prefix & hi_mask;
    stream_vectors(vrow, nvec, tid, [&](const u32x4& v, long long, bool valid) {
      if (!valid) return;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const uint32_t key = E::key_of_bits(vec_bits<BF16>(v, e));
        if ((key & hi_mask) == want) atomicAdd(&S.hist[(key >> shift) & 255u], 1u);
      }
    });
    if (tid < S.nscal) {
      const uint32_t key = S.skey[tid];
      if ((key & hi_mask) == want) atomicAdd(&S.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave_id() == 0) pick_digit_into(S, remaining);
    __syncthreads();
    prefix |= (uint32_t)S.sh[0] << shift;
    remaining -= S.sh[1];
    __syncthreads();
  }
  return prefix;
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads, 5) lsm_topk_kernel(const typename Elem<BF16>::T* __restrict__ logits,
                                                               long long V, int k, int cap_w, int pool_cap,
                                                               int sort_cap, int cand_cap, int rows_per_tree,
                                                               int L, const int32_t* __restrict__ modes,
                                                               double* __restrict__ lse_out,
                                                               const int32_t* __restrict__ vocab_map,
                                                               int32_t* __restrict__ topk_id,
                                                               float* __restrict__ topk_raw,
                                                               float* __restrict__ topk_logp,
                                                               int32_t* __restrict__ status) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int VEC = E::VEC;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // LDS: staged vectors (4 wave areas, then the pool) | their indices |
  // candidate list.  Once the staged vectors have been compacted the start of
  // their area holds the sort buffer.
  const int nslot = kWaves * cap_w + pool_cap;
  u32x4* svec_all = reinterpret_cast<u32x4*>(smem_raw);
  uint32_t* sidx_all = reinterpret_cast<uint32_t*>(svec_all + nslot);
  uint64_t* cand = reinterpret_cast<uint64_t*>(sidx_all + nslot);
  uint64_t* sortbuf = reinterpret_cast<uint64_t*>(smem_raw);
  __shared__ Shared S;

  const int tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const long long row = blockIdx.x;
  const T* rowp = logits + row * V;
  if (modes) {
    // rows of a mode at or past the tree's mode count are neither read nor
    // written (the whole workgroup leaves before its first barrier)
    const int n = (int)(row / rows_per_tree);
    const int m = (int)(row - (long long)n * rows_per_tree) / L;
    const int kn = modes[n];
    if (m >= (kn < 1 ? 1 : kn)) return;
  }

  if (tid == 0) {
    S.overflow = 0;
    S.pool = 0;
    S.fail_at = 0xFFFFFFFFu;
    S.nsurv = 0;
    S.ncand = 0;
  }

  Stager sg;
  sg.svec = svec_all + (size_t)wid * cap_w;
  sg.sidx = sidx_all + (size_t)wid * cap_w;
  sg.pvec = svec_all + (size_t)kWaves * cap_w;
  sg.pidx = sidx_all + (size_t)kWaves * cap_w;
  sg.pool_used = &S.pool;
  sg.fail_at = &S.fail_at;
  sg.pool_cap = pool_cap;
  sg.cap = cap_w;
  sg.scnt = 0;
  sg.full = false;

  // Split the row into a scalar head (to 16-byte alignment), aligned vectors
  // and a scalar tail.
  const uintptr_t addr = reinterpret_cast<uintptr_t>(rowp);
  long long head = (long long)(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const long long nvec = (V - head) / VEC;
  const long long tail0 = head + nvec * VEC;
  const int nscalar = (int)(head + (V - tail0));
  const u32x4* vrow = reinterpret_cast<const u32x4*>(rowp + head);
  const long long nchunks = (nvec + kStep - 1) / kStep;
  const uint32_t last_byte = nvec > 0 ? (uint32_t)(nvec - 1) * (uint32_t)sizeof(u32x4) : 0u;

  // Scalars (head / tail, at most 2 * (VEC - 1) < 64): wave 0, one per lane.
  // Loaded before the chunks and used after them, so that waiting for them
  // does not wait for the chunks too.
  const bool shas = wid == 0 && lane < nscalar;
  const long long si = shas ? (lane < head ? (long long)lane : tail0 + (lane - head)) : 0;
  const uint32_t sbits = E::bits_at(rowp, si);  // every lane loads (element 0 if none), no branch

  // Three chunk buffers: two chunks stay in flight while one is consumed.
  u32x4 bufA[kUnroll], bufB[kUnroll], bufC[kUnroll];
  if (nvec > 0) {
    load_chunk(bufA, vrow, 0, last_byte, tid);
    load_chunk(bufB, vrow, 1, last_byte, tid);
    load_chunk(bufC, vrow, 2, last_byte, tid);
  }

  const float xs = shas ? E::val_of_bits(sbits) : -INFINITY;
  if (shas) {
    S.skey[lane] = E::key_of_bits(sbits);
    S.sidx[lane] = (uint32_t)si;
  }
  if (tid == 0) S.nscal = nscalar;

  // ------------------------------------------------------------ the sample
  // The sample is chunks 0 and 1 (both already in registers) and the scalars.
  // Lane maxima over it; NaN is skipped by fmaxf.
  // (Selects, not branches, so the wait covers chunks 0 and 1 only.)
  float lmax = xs;
  if (nvec > 0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long q = (long long)u * kThreads + tid;
      float ma = vec_val<BF16>(bufA[u], 0), mb = vec_val<BF16>(bufB[u], 0), mc = vec_val<BF16>(bufC[u], 0);
#pragma unroll
      for (int j = 1; j < VEC; ++j) {
        ma = fmaxf(ma, vec_val<BF16>(bufA[u], j));
        mb = fmaxf(mb, vec_val<BF16>(bufB[u], j));
        if (kSampleChunks > 2) mc = fmaxf(mc, vec_val<BF16>(bufC[u], j));
      }
      lmax = fmaxf(lmax, q < nvec ? ma : -INFINITY);
      lmax = fmaxf(lmax, q + kStep < nvec ? mb : -INFINITY);
      if (kSampleChunks > 2) lmax = fmaxf(lmax, q + 2 * kStep < nvec ? mc : -INFINITY);
    }
  }
  S.hist[tid] = E::key_of_float(lmax);
  __syncthreads();
  const uint32_t k0 = S.hist[lane], k1 = S.hist[lane + kWave], k2 = S.hist[lane + 2 * kWave],
                 k3 = S.hist[lane + 3 * kWave];
  // Threshold: the r-th largest lane maximum, so at least r sampled elements
  // reach it.  Every wave runs the same bitwise search over all 256 keys (four
  // ballots per bit), so all agree without another barrier.
  const long long n0 = (kSampleChunks * kStep <= nvec ? kSampleChunks * kStep : nvec) * VEC + nscalar;
  const int r = sample_rank(V, n0, k);
  uint32_t thr = 0;
#pragma unroll 1
  for (int bit = E::KEYBITS - 1; bit >= 0; --bit) {
    const uint32_t tt = thr | (1u << bit);
    const int c = __popcll(__ballot(k0 >= tt)) + __popcll(__ballot(k1 >= tt)) + __popcll(__ballot(k2 >= tt)) +
                  __popcll(__ballot(k3 >= tt));
    if (c >= r) thr = tt;
  }
  // Bias: the sample maximum M0 in log2 units (0 if M0 is not finite).
  uint32_t mkey = max(max(k0, k1), max(k2, k3));
  mkey = wave_allreduce(mkey, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
  const float m0 = thr_float<BF16>(mkey);
  const float bias = isfinite(m0) ? m0 * kLog2e : 0.f;
  // Staging cut on a vector's term sum (see consume_vector); 0 stages every vector.
  const float thr_f = thr_float<BF16>(thr);
  const float tau = thr_f == -INFINITY ? 0.f : 0.999f * term(thr_f, bias);

  // ------------------------------------------------------------ the stream
  double s = (double)term(xs, bias);
  if (nvec > 0) {
    s += (double)consume_chunk<BF16>(bufA, 0, nvec, head, tid, bias, tau, sg);
    // invariant at the loop head: B holds chunk c, C chunk c + 1
    long long c = 1;
    for (; c + 2 < nchunks; c += 3) {
      load_chunk(bufA, vrow, c + 2, last_byte, tid);
      s += (double)consume_chunk<BF16>(bufB, c, nvec, head, tid, bias, tau, sg);
      load_chunk(bufB, vrow, c + 3, last_byte, tid);
      s += (double)consume_chunk<BF16>(bufC, c + 1, nvec, head, tid, bias, tau, sg);
      load_chunk(bufC, vrow, c + 4, last_byte, tid);
      s += (double)consume_chunk<BF16>(bufA, c + 2, nvec, head, tid, bias, tau, sg);
    }
    if (c < nchunks) s += (double)consume_chunk<BF16>(bufB, c, nvec, head, tid, bias, tau, sg);
    if (c + 1 < nchunks) s += (double)consume_chunk<BF16>(bufC, c + 1, nvec, head, tid, bias, tau, sg);
  }

  // ------------------------------------------------------------ log-normaliser
  s = wave_allreduce(s, [](double x, double y) { return x + y; });
  if (lane == 0) {
    S.red_s[wid] = s;
    S.cnt[wid] = sg.scnt;
    if (sg.full) S.overflow = 1;
  }
  __syncthreads();
  double sum = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += S.red_s[w];
  double lse;
  if (isnan(sum)) {
    lse = NAN;
  } else if (isfinite(sum) && sum >= 0x1p-60) {
    // no term overflowed, and every term that matters is a normal float
    lse = (double)bias * kLn2 + log(sum);
  } else {
    // The sample maximum was too far from the row maximum (or the row holds
    // +inf or only -inf): find the row maximum, then sum again with it as the
    // bias.
    float mx = xs;
    stream_vectors(vrow, nvec, tid, [&](const u32x4& v, long long, bool valid) {
      if (!valid) return;
#pragma unroll
      for (int j = 0; j < VEC; ++j) mx = fmaxf(mx, vec_val<BF16>(v, j));
    });
    mx = wave_allreduce(mx, [](float x, float y) { return fmaxf(x, y); });
    __syncthreads();
    if (lane == 0) S.red_max[wid] = mx;
    __syncthreads();
    float rmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) rmax = fmaxf(rmax, S.red_max[w]);
    if (rmax == INFINITY) {
      lse = INFINITY;
    } else if (rmax == -INFINITY) {
      lse = -INFINITY;  // every element is -inf
    } else {
      const float b2 = rmax * kLog2e;
      double s2 = (double)term(xs, b2);
      stream_vectors(vrow, nvec, tid, [&](const u32x4& v, long long, bool valid) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc += valid ? term(vec_val<BF16>(v, j), b2) : 0.f;
        s2 += (double)acc;
      });
      s2 = wave_allreduce(s2, [](double x, double y) { return x + y; });
      if (lane == 0) S.red_s[wid] = s2;
      __syncthreads();
      double sum2 = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum2 += S.red_s[w];
      lse = (double)b2 * kLn2 + log(sum2);
    }
  }
  if (tid == 0 && status && (isnan(lse) || lse == INFINITY)) atomicOr(&status[row / rows_per_tree], 1);

  // ------------------------------------------------------------ exact top-k
  uint64_t* sb = sortbuf;  // where the survivors end up
  uint32_t sel = thr;      // every row element at or above `sel` is staged
  // Staged vectors: wave areas 0..3, then the pool, indexed g in [0, tot).
  int o1, o2, o3, o4, tot;
  auto staged_layout = [&]() {
    const int c4 = S.pool < pool_cap ? S.pool : pool_cap;
    o1 = S.cnt[0];
    o2 = o1 + S.cnt[1];
    o3 = o2 + S.cnt[2];
    o4 = o3 + S.cnt[3];
    tot = o4 + c4;
  };
  auto slot_of = [&](int g) -> int {
    const int w = (g >= o1) + (g >= o2) + (g >= o3) + (g >= o4);
    const int off = w == 0 ? 0 : (w == 1 ? o1 : (w == 2 ? o2 : (w == 3 ? o3 : o4)));
    return w * cap_w + (g - off);
  };
  // Element i of the staged data (scalars after the vectors), if it reaches `sel`.
  auto staged_key = [&](int i, uint64_t* out) -> bool {
    const int nst = tot * VEC;
    uint32_t key;
    if (i < nst) key = E::key_of_bits(vec_bits<BF16>(svec_all[slot_of(i / VEC)], i % VEC));
    else key = S.skey[i - nst];
    *out = key;
    return key >= sel;
  };
  staged_layout();
  if (S.overflow) {
    // The staging space overflowed: far more elements reached the threshold
    // than the sample predicted.  The staged ones cover about the first
    // fail_at elements of the row; take the rank among them that scales to
    // 2.5k over the whole row, and stage the row once more with that key as
    // the threshold.  (If the row's tail differs, the next attempt overflows
    // or finds fewer than k, and the row takes the exact fallback.)
    const int n = tot * VEC + S.nscal;
    const long long covered = S.fail_at < (uint32_t)V ? (long long)S.fail_at : V;
    int r2 = (int)((5LL * k * covered + 2 * V - 1) / (2 * V));
    r2 = r2 < 1 ? 1 : r2;
    int mine = 0;
    for (int i = tid; i < n; i += kThreads) {
      uint64_t key;
      mine += staged_key(i, &key) ? 1 : 0;
    }
    const int have = block_sum<kThreads>(mine, S.scan);
    if (have >= r2) {
      const uint32_t t2 = (uint32_t)block_kth_largest<kThreads, E::KEYBITS>(n, r2, staged_key, S.hist, S.sh);
      if (tid == 0) {
        S.pool = 0;
        S.overflow = 0;
      }
      sg.scnt = 0;
      sg.full = false;
      __syncthreads();
      stream_vectors(vrow, nvec, tid, [&](const u32x4& v, long long q, bool valid) {
        uint32_t mk = 0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) mk = max(mk, E::key_of_bits(vec_bits<BF16>(v, e)));
        sg.stage(valid && mk >= t2, v, (uint32_t)(head + q * VEC), 0u);
      });
      if (lane == 0) {
        S.cnt[wid] = sg.scnt;
        if (sg.full) S.overflow = 1;
      }
      __syncthreads();
      sel = t2;
      staged_layout();
    }
  }
  if (!S.overflow) {
    // (1) compact the staged elements that reach the threshold into cand[]
    for (int g0 = 0; g0 < tot; g0 += kThreads) {
      const int g = g0 + tid;
      uint32_t hit = 0;
      u32x4 v = {0u, 0u, 0u, 0u};
      uint32_t i0 = 0;
      if (g < tot) {
        const int sl = slot_of(g);
        v = svec_all[sl];
        i0 = sidx_all[sl];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          hit |= (E::key_of_bits(vec_bits<BF16>(v, e)) >= sel ? 1u : 0u) << e;
      }
      const int c = __popc(hit);
      const int incl = wave_inclusive_scan(c);
      int base = 0;
      if (lane == kWave - 1) base = atomicAdd(&S.ncand, incl);
      base = __shfl(base, kWave - 1, kWave);
      int pos = base + incl - c;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if ((hit >> e) & 1u) {
          if (pos < cand_cap) cand[pos] = composite(E::key_of_bits(vec_bits<BF16>(v, e)), i0 + e);
          ++pos;
        }
      }
    }
    if (wid == 0) {
      const bool p = lane < S.nscal && S.skey[lane] >= sel;
      wave_append(p, p ? composite(S.skey[lane], S.sidx[lane]) : 0ull, cand, cand_cap, &S.ncand);
    }
    __syncthreads();
    const int ncand = S.ncand;
    if (ncand >= k && ncand <= cand_cap) {
      // (2) the exact k-th largest key among the candidates
      auto getc = [&](int i, uint64_t* out) -> bool {
        *out = cand[i] >> 32;
        return true;
      };
      const uint32_t kth = (uint32_t)block_kth_largest<kThreads, E::KEYBITS>(ncand, k, getc, S.hist, S.sh);
      // (3) gather the candidates above the k-th key (fewer than k), then
      // those at it
      for (int i0 = 0; i0 < ncand; i0 += kThreads) {
        const int i = i0 + tid;
        const uint64_t cv = i < ncand ? cand[i] : 0ull;
        wave_append(i < ncand && (uint32_t)(cv >> 32) > kth, cv, sortbuf, sort_cap, &S.nsurv);
      }
      __syncthreads();
      const int nabove = S.nsurv;
      for (int i0 = 0; i0 < ncand; i0 += kThreads) {
        const int i = i0 + tid;
        const uint64_t cv = i < ncand ? cand[i] : 0ull;
        wave_append(i < ncand && (uint32_t)(cv >> 32) == kth, cv, sortbuf, sort_cap, &S.nsurv);
      }
      __syncthreads();
      // (4) keep only the k - nabove lowest-index ties when there are a few
      // more (one wave sorts them; at equal keys the composite orders by index)
      const int nties = S.nsurv - nabove, need = k - nabove;
      if (nties > need && nties <= kWave) {
        if (wid == 0) {
          uint64_t tv = lane < nties ? sortbuf[nabove + lane] : 0ull;
          tv = wave_sort_desc(tv);
          if (lane < need) sortbuf[nabove + lane] = tv;
          if (lane == 0) S.nsurv = k;
        }
        __syncthreads();
      }
    } else if (ncand > cand_cap) {
      // Too many candidates for the list: select straight from the staged
      // vectors.
      const int nst = tot * VEC;
      const int n = nst + S.nscal;
      const uint32_t kth = (uint32_t)block_kth_largest<kThreads, E::KEYBITS>(n, k, staged_key, S.hist, S.sh);
      sb = cand;  // the staged vectors are still being read: gather into the list instead
      for (int i0 = 0; i0 < n; i0 += kThreads) {
        const int i = i0 + tid;
        uint64_t key = 0;
        const bool p = i < n && staged_key(i, &key) && (uint32_t)key >= kth;
        uint32_t idx = 0;
        if (p) idx = i < nst ? sidx_all[slot_of(i / VEC)] + (uint32_t)(i % VEC) : S.sidx[i - nst];
        wave_append(p, composite((uint32_t)key, idx), cand, sort_cap, &S.nsurv);
      }
    } else if (tid == 0) {
      S.overflow = 1;  // fewer than k reached the guess
    }
    __syncthreads();
    if (tid == 0 && S.nsurv > sort_cap) {
      S.overflow = 1;  // too many ties at the k-th key for the sort buffer
      S.nsurv = 0;
    }
    __syncthreads();
  }
  if (S.overflow) {
    // Exact fallback over the row: radix-select the k-th largest key, then
    // gather every element at or above it.
    sb = sortbuf;
    const uint32_t kk = row_kth_largest<BF16>(vrow, nvec, k, S);
    stream_vectors(vrow, nvec, tid, [&](const u32x4& v, long long q, bool valid) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const uint32_t key = E::key_of_bits(vec_bits<BF16>(v, e));
        wave_append(valid && key >= kk, composite(key, (uint32_t)(head + q * VEC + e)), sortbuf, sort_cap,
                    &S.nsurv);
      }
    });
    if (wid == 0) {
      const bool p = lane < S.nscal && S.skey[lane] >= kk;
      wave_append(p, p ? composite(S.skey[lane], S.sidx[lane]) : 0ull, sortbuf, sort_cap, &S.nsurv);
    }
    __syncthreads();
    const int nall = S.nsurv;
    __syncthreads();
    if (nall > sort_cap) {
      // So many ties at the k-th key that they do not fit: keep the elements
      // above it and the lowest-index ties.
      if (tid == 0) S.nsurv = 0;
      __syncthreads();
      for (long long b0 = 0; b0 < V; b0 += kThreads) {
        const long long i = b0 + tid;
        const uint32_t key = i < V ? E::key_of_bits(E::bits_at(rowp, i)) : 0u;
        wave_append(i < V && key > kk, composite(key, (uint32_t)i), sortbuf, sort_cap, &S.nsurv);
      }
      __syncthreads();
      const int taken = S.nsurv;  // fewer than k
      const int need = k - taken;
      int ties_before = 0;
      for (long long b0 = 0; b0 < V && ties_before < need; b0 += kThreads) {
        const long long i = b0 + tid;
        const bool tie = i < V && E::key_of_bits(E::bits_at(rowp, i)) == kk;
        int tot;
        const int rr = ties_before + block_exclusive_scan<kThreads>(tie ? 1 : 0, S.scan, &tot);
        if (tie && rr < need && taken + rr < sort_cap) sortbuf[taken + rr] = composite(kk, (uint32_t)i);
        ties_before += tot;
      }
      if (tid == 0) S.nsurv = k;
    }
    __syncthreads();
  }

  // The log-normaliser is stored once the row maximum (the largest survivor)
  // is known: exp2-domain rounding can leave it a little under the maximum,
  // and it is raised to it there (a NaN stays NaN), so that no
  // log-probability comes out positive.
  auto settle_lse = [&](bool mine, float top) {
    if (mine) S.red_max[0] = top;
    __syncthreads();
    const double t = (double)S.red_max[0];
    if (lse < t) lse = t;
    if (tid == 0) lse_out[row] = lse;
  };

  // sort the survivors (descending composite = key descending, token ascending)
  const int ns = S.nsurv;
  const int P = next_pow2(ns < k ? k : ns);
  if (P <= kThreads) {
    uint64_t a0 = tid < ns ? sb[tid] : 0ull;
    __syncthreads();
    block_sort_single<kThreads>(a0, sb);
    settle_lse(tid == kThreads - 1, E::val_of_key((uint32_t)(a0 >> 32)));
    const int j = kThreads - 1 - tid;
    if (j < k) {
      const uint32_t key = (uint32_t)(a0 >> 32);
      const uint32_t idx = 0xFFFFFFFFu - (uint32_t)a0;
      const float x = E::val_of_key(key);
      const long long o = row * k + j;
      topk_id[o] = vocab_map ? vocab_map[idx] : (int32_t)idx;
      topk_raw[o] = x;
      if (topk_logp) topk_logp[o] = (float)((double)x - lse);
    }
    return;
  }
  if (P <= 2 * kThreads) {
    uint64_t a0 = 2 * tid < ns ? sb[2 * tid] : 0ull;
    uint64_t a1 = 2 * tid + 1 < ns ? sb[2 * tid + 1] : 0ull;
    __syncthreads();
    block_sort_pairs<kThreads>(a0, a1, sb);
    settle_lse(tid == kThreads - 1, E::val_of_key((uint32_t)(a1 >> 32)));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = 2 * kThreads - 1 - (2 * tid + e);
      if (j < k) {
        const uint64_t c = e ? a1 : a0;
        const uint32_t key = (uint32_t)(c >> 32);
        const uint32_t idx = 0xFFFFFFFFu - (uint32_t)c;
        const float x = E::val_of_key(key);
        const long long o = row * k + j;
        topk_id[o] = vocab_map ? vocab_map[idx] : (int32_t)idx;
        topk_raw[o] = x;
        if (topk_logp) topk_logp[o] = (float)((double)x - lse);
      }
    }
    return;
  }
  for (int i = ns + tid; i < P; i += kThreads) sb[i] = 0ull;
  __syncthreads();
  block_bitonic_sort<kThreads>(sb, P);
  settle_lse(tid == 0, E::val_of_key((uint32_t)(sb[P - 1] >> 32)));
  for (int j = tid; j < k; j += kThreads) {
    const uint64_t c = sb[P - 1 - j];
    const uint32_t key = (uint32_t)(c >> 32);
    const uint32_t idx = 0xFFFFFFFFu - (uint32_t)c;
    const float x = E::val_of_key(key);
    const long long o = row * k + j;
    topk_id[o] = vocab_map ? vocab_map[idx] : (int32_t)idx;
    topk_raw[o] = x;
    if (topk_logp) topk_logp[o] = (float)((double)x - lse);
  }
}

// Capacities of one row's LDS areas.
struct LsmCaps {
  int cap_w;     // staged vectors per wave area
  int pool;      // staged vectors in the shared pool
  int sort_cap;  // survivors (k plus ties)
  int cand_cap;  // candidates (staged elements reaching the threshold)
  size_t lds;    // dynamic LDS bytes
};

LsmCaps lsm_caps(long long V, int k, bool bf16) {
  const int vec = bf16 ? 8 : 4;
  LsmCaps c;
  c.sort_cap = 2 * next_pow2(k) > 2 * kThreads ? 2 * next_pow2(k) : 2 * kThreads;
  c.cand_cap = 4 * next_pow2(k) > c.sort_cap ? 4 * next_pow2(k) : c.sort_cap;
  // expected staged vectors: about one per element at or above the threshold,
  // plus a quarter for vectors staged on a half sum of medium terms (rows of
  // low spread); a row that fits in the sample is staged whole
  const long long n0 = (kSampleChunks * kStep * vec < V ? kSampleChunks * kStep * vec : V);
  const double expect = (double)V / (double)(n0 > 0 ? n0 : 1) * sample_rank(V, n0 > 0 ? n0 : 1, k) * 1.25 + 32.0;
  long long e = (long long)expect;
  if (V <= kSampleChunks * kStep * vec && V / vec + 2 > e) e = V / vec + 2;
  long long cap_w = (e * 11 / 10 / kWaves + 15) / 16 * 16;  // a quarter each, 10% over
  long long total = (e * 8 / 5 + 63) / 64 * 64;               // 1.6x in all
  // the sort buffer lives in the staged-vector area once staging is over
  const long long need = ((long long)c.sort_cap * 8 + 15) / 16;
  if (total < need) total = need;
  if (total < kWaves * cap_w + 64) total = kWaves * cap_w + 64;
  // keep the workgroup within the LDS budget (more rows then take the exact
  // fallback, results are unchanged)
  const size_t fixed = sizeof(Shared) + (size_t)c.cand_cap * 8;
  const long long max_slots = (long long)((kMaxLds - fixed) / 20);
  if (total > max_slots) {
    total = max_slots < need ? need : max_slots;
    cap_w = (total / 2 / kWaves) / 16 * 16;
  }
  c.cap_w = (int)cap_w;
  c.pool = (int)(total - kWaves * cap_w);
  c.lds = (size_t)total * 20 + (size_t)c.cand_cap * 8;
  return c;
}

}  // namespace

hipError_t launch_logsoftmax_topk(const void* logits, bool bf16, int rows, int rows_per_tree, int L, long long V,
                                  int k, const int32_t* vocab_map, const int32_t* modes, double* lse,
                                  int32_t* topk_id, float* topk_raw, float* topk_logp, int32_t* status,
                                  hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const LsmCaps c = lsm_caps(V, k, bf16);
  if (bf16) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lsm_topk_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)c.lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lsm_topk_kernel<true>, dim3(rows), dim3(kThreads), c.lds, stream,
                       static_cast<const uint16_t*>(logits), V, k, c.cap_w, c.pool, c.sort_cap, c.cand_cap,
                       rows_per_tree, L, modes, lse, vocab_map, topk_id, topk_raw, topk_logp, status);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lsm_topk_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)c.lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lsm_topk_kernel<false>, dim3(rows), dim3(kThreads), c.lds, stream,
                       static_cast<const float*>(logits), V, k, c.cap_w, c.pool, c.sort_cap, c.cand_cap,
                       rows_per_tree, L, modes, lse, vocab_map, topk_id, topk_raw, topk_logp, status);
  }
  return hipGetLastError();
}

}  // namespace mfd
