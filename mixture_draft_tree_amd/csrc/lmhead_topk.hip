// Fused LM head + per-row log-softmax and top-k (mfd_lmhead_logsoftmax_topk).
//
// The drafter shares its target's LM head (model card "MFD drafter for
// Qwen3.5-4B", "Model" and "Parameters"), and the pages' Python interface
// turns on a fused logits path (same card, "Usage": fused_logits=True).  Here
// the drafter's final hidden states H [M, D] (M = N*K*L rows) meet the head
// W [V, D] on the matrix cores, and each row's log-normaliser and k best
// tokens come out without the [M, V] logits ever being stored.
//
// Four launches on the caller's stream:
//   1. lmh_tile_kernel<true>   (sample)  S spread V-tiles of the product; per
//      row the maximum of every disjoint group of 4 columns goes to `samp`.
//   2. lmh_threshold_kernel    per row: thr = the k-th largest of those group
//      maxima.  They are k distinct elements of the row, so the row's k-th
//      largest logit is >= thr: every top-k element passes x >= thr.  Rows with
//      fewer than k groups take thr = "everything".
//   3. lmh_tile_kernel<false>  (main)  every tile of the product; per row and
//      tile the partial (max, sum exp(x - max)); every logit >= thr is appended
//      to its row's candidate list.
//   4. lmh_select_kernel       per row: lse from the partials (fp64), the exact
//      k-th largest (logit desc, id asc) among the candidates, those k sorted.
//
// Tiles: 128 rows x 256 vocabulary columns per 256-thread workgroup, two
// workgroups per CU, k in steps of 32 through double-buffered, XOR-swizzled LDS
// (global loads two steps ahead), four waves of 64 x 128 each built
// from v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  Each product element is
// computed from the same operands in the same k order in both tile launches,
// so the sample and main launches see identical logits.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kBM = 128, kBK = 32, kNT = 256;
constexpr int kLdk = kBK;  // bf16 per LDS row: 64 bytes, four 16-byte chunks, XOR-swizzled

// Physical chunk of logical chunk q (16 bytes, k-offset 8q) in LDS row r.  The
// swizzle f(r) = ((r >> 1) ^ (r >> 3)) & 3 differs over rows of equal parity
// among 8 consecutive rows and over rows of equal r % 4 among 16, so the
// 16-byte fragment reads of 8 or 16 consecutive rows at one k-offset, and the
// staging writes of 2 or 4 consecutive rows' 4 chunks, fall in distinct bank
// groups whether a pass serves 8 lanes over 32 banks or 16 lanes over 64.
__device__ __forceinline__ int lds_chunk(int r, int q) { return q ^ (((r >> 1) ^ (r >> 3)) & 3); }
constexpr int kSampleCols = 8192;  // vocabulary columns in the threshold sample
constexpr int kSmallM = 256;       // up to this many rows, tiles are 128 columns wide

// Tile shapes.  The four waves of a workgroup split its 128 rows x BN columns
// as WGM (rows) x WGN (columns) waves of (128 / WGM) x 128; a wave's part is
// IM x 4 blocks of 32 x 32.  WGM = 2: 128 x 256 tiles (large M: the head tile
// serves more rows per fetch).  WGM = 4: 128 x 128 tiles (few rows: twice the
// tiles, so one tree's 1187 tiles spread over the CUs in fewer idle rounds).
template <int WGM>
struct TileShape {
  static constexpr int WGN = 4 / WGM, BN = WGN * 128, IM = 4 / WGM, GPT = WGN * 32, NB = BN / 64;
};
constexpr int kThrNT = 256;   // threshold kernel: 2048 sample keys per row
constexpr int kSelNT = 1024;  // select kernel: thousands of candidates per row
constexpr int kSelLdsCap = 8192;  // candidates a select workgroup holds in LDS

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct LmhArgs {
  const uint16_t* H;  // [M, D] bf16 bits
  const uint16_t* W;  // [V, D] bf16 bits
  int M, D, V, T, S, rows_per_tree;
  int gpt;              // groups of 4 columns per tile (WGN * 32)
  int wgn;              // waves across a tile's columns
  uint32_t* samp;       // [M, S * gpt] group-maximum keys (0 = empty group)
  uint32_t* thr;        // [M] candidate threshold keys
  float2* part;         // [M, wgn * T] (max, sum exp(x - max)) per tile and wave column
  uint64_t* cand;       // [M, C] candidate composites
  int* cand_count;      // [M]
  int C;
  int32_t* status;      // [N] or null
  const int32_t* vocab_map;  // [V] full-vocabulary id of column v (increasing), or null
  int packed;                // W in the packed layout of lmh_pack_kernel (else row-major [V, D])
};

__device__ __forceinline__ uint64_t cand_composite(uint32_t key, uint32_t col) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - col);
}

// Tile t of the XCD-aware order: workgroup b runs on XCD b % 8 and takes the
// (b / 8)-th tile of that XCD's contiguous share.  The shares cut a linear
// order of (row group, vocabulary tile, row tile in group), a row group being
// ceil(nM / 8) row tiles, so one XCD works through few row tiles and all their
// vocabulary tiles: the weight tile is fetched once into that XCD's L2 for the
// row tiles of its group, and the group's hidden rows stay warm.
__device__ __forceinline__ bool tile_of(int b, int nM, int nVt, int* m_out, int* v_out) {
  const long long ntiles = (long long)nM * nVt;
  const long long per = (ntiles + 7) / 8;
  const long long t = (long long)(b & 7) * per + (b >> 3);
  if (t >= ntiles) return false;
  const int G = (nM + 7) / 8;
  const long long gsz_full = (long long)G * nVt;
  const int mg = (int)(t / gsz_full);
  const long long r = t - (long long)mg * gsz_full;
  const int gsz = min(G, nM - mg * G);
  *v_out = (int)(r / gsz);
  *m_out = mg * G + (int)(r % gsz);
  return true;
}

template <bool SAMPLE, int WGM>
__global__ void __launch_bounds__(kNT, 2) lmh_tile_kernel(LmhArgs a) {
  using TS = TileShape<WGM>;
  constexpr int BN = TS::BN, WGN = TS::WGN, IM = TS::IM, GPT = TS::GPT;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM][kLdk];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN][kLdk];
  __shared__ uint32_t sthr[kBM];

  const int nM = (a.M + kBM - 1) / kBM;
  const int nVt = SAMPLE ? a.S : a.T;
  int mt, vt_i;
  if (!tile_of((int)blockIdx.x, nM, nVt, &mt, &vt_i)) return;  // whole workgroup, before any barrier
  const int vt = SAMPLE ? (int)(((long long)vt_i * a.T) / a.S) : vt_i;
  const int row0 = mt * kBM, col0 = vt * BN;
  const int tid = (int)threadIdx.x, lane = lane_id(), w = wave_id();
  const int wm = w / WGN, wn = w % WGN;
  const int D = a.D;

  if (!SAMPLE) {
    for (int i = tid; i < kBM; i += kNT) sthr[i] = row0 + i < a.M ? a.thr[row0 + i] : 0xFFFFFFFFu;
  }

  // global -> register chunks of 8 bf16: A 512 per stage (2 per thread), B 4 BN
  // (BN / 64 per thread).  Chunk c is row c / 4, k-offset 8 (c % 4) of the stage.
  // Rows past the matrix read its last row (their results are dropped).
  const int q8 = (tid & 3) * 8, r0 = tid >> 2;
  const int qs8 = lds_chunk(r0, tid & 3) * 8;  // rows r0 + 64 j share r0's swizzle
  const uint16_t* a0p = a.H + (size_t)min(row0 + r0, a.M - 1) * D + q8;
  const uint16_t* a1p = a.H + (size_t)min(row0 + r0 + 64, a.M - 1) * D + q8;
  // Head rows: row-major (rows past V read row V - 1), or packed: the 64 rows x
  // 32 k of block (col0 / 64 + j, step s) are one contiguous 4 KB run at
  // ((col0 / 64 + j) * nS + s) * 2048 elements, thread t's chunk at 8 t.
  const int nSt = D / kBK;
  const size_t bmul = a.packed ? 64 : 1;  // elements per unit of k0
  const uint16_t* b0p = a.packed ? a.W + ((size_t)(col0 / 64 + 0) * nSt) * 2048 + tid * 8
                                 : a.W + (size_t)min(col0 + r0, a.V - 1) * D + q8;
  const uint16_t* b1p = a.packed ? a.W + ((size_t)(col0 / 64 + 1) * nSt) * 2048 + tid * 8
                                 : a.W + (size_t)min(col0 + r0 + 64, a.V - 1) * D + q8;
  const uint16_t* b2p = a.packed ? a.W + ((size_t)(col0 / 64 + 2) * nSt) * 2048 + tid * 8
                                 : a.W + (size_t)min(col0 + r0 + 128, a.V - 1) * D + q8;
  const uint16_t* b3p = a.packed ? a.W + ((size_t)(col0 / 64 + 3) * nSt) * 2048 + tid * 8
                                 : a.W + (size_t)min(col0 + r0 + 192, a.V - 1) * D + q8;
  // Register staging, NSET stages deep: stage j's chunks sit in register set
  // j % NSET from their global load (issued at step j - NSET) until they are
  // copied to LDS at the end of step j - 1.  Narrow tiles have the registers
  // for four sets (loads three steps ahead of their use); wide tiles two.
  constexpr int NSET = WGM == 4 ? 4 : 2;
  uint4 p0a0, p0a1, p0b0, p0b1, p0b2, p0b3;
  uint4 p1a0, p1a1, p1b0, p1b1, p1b2, p1b3;
  uint4 p2a0, p2a1, p2b0, p2b1, p2b2, p2b3;
  uint4 p3a0, p3a1, p3b0, p3b1, p3b2, p3b3;
#define LMH_GLOAD(P, k0)                                       \
  do {                                                         \
    P##a0 = *reinterpret_cast<const uint4*>(a0p + (k0));       \
    P##a1 = *reinterpret_cast<const uint4*>(a1p + (k0));       \
    P##b0 = *reinterpret_cast<const uint4*>(b0p + (k0) * bmul);       \
    P##b1 = *reinterpret_cast<const uint4*>(b1p + (k0) * bmul);       \
    if constexpr (TS::NB == 4) {                               \
      P##b2 = *reinterpret_cast<const uint4*>(b2p + (k0) * bmul);     \
      P##b3 = *reinterpret_cast<const uint4*>(b3p + (k0) * bmul);     \
    }                                                          \
  } while (0)
#define LMH_LSTORE(P, buf)                                          \
  do {                                                              \
    *reinterpret_cast<uint4*>(&sA[buf][r0][qs8]) = P##a0;            \
    *reinterpret_cast<uint4*>(&sA[buf][r0 + 64][qs8]) = P##a1;       \
    *reinterpret_cast<uint4*>(&sB[buf][r0][qs8]) = P##b0;            \
    *reinterpret_cast<uint4*>(&sB[buf][r0 + 64][qs8]) = P##b1;       \
    if constexpr (TS::NB == 4) {                                    \
      *reinterpret_cast<uint4*>(&sB[buf][r0 + 128][qs8]) = P##b2;    \
      *reinterpret_cast<uint4*>(&sB[buf][r0 + 192][qs8]) = P##b3;    \
    }                                                               \
  } while (0)

  f32x16 acc[IM][4];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // lane l feeds row (or column) l % 32 of a 32 x 16 operand, k-half l / 32;
  // every operand row starts at a multiple of 32, so its swizzle is lds_chunk(l % 32, .)
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  const int nS = D / kBK;
#define LMH_COMPUTE(buf)                                                                          \
  do {                                                                                            \
    _Pragma("unroll") for (int kk = 0; kk < kBK; kk += 16) {                                      \
      bf16x8 af[IM], bfv[4];                                                                      \
      const int kc = (lds_chunk(lr, ((kk + lk) >> 3))) * 8;                                       \
      _Pragma("unroll") for (int i = 0; i < IM; ++i)                                              \
        af[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][wm * 32 * IM + i * 32 + lr][kc]);       \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                               \
        bfv[j] = *reinterpret_cast<const bf16x8*>(&sB[buf][wn * 128 + j * 32 + lr][kc]);          \
      _Pragma("unroll") for (int i = 0; i < IM; ++i)                                              \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                             \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0); \
    }                                                                                             \
  } while (0)
  // Steady state: the prefetch load is unconditional (past the last stage it
  // re-reads that stage, unused), so the compiler can count the loads in
  // flight and wait only for the stage it stores, never for the prefetch.
#define LMH_STEP(CUR, NXT)                                  \
  {                                                         \
    const int buf = s & 1;                                  \
    LMH_GLOAD(CUR, min(s + NSET, nS - 1) * kBK);            \
    LMH_COMPUTE(buf);                                       \
    if (s + 1 < nS) LMH_LSTORE(NXT, buf ^ 1);               \
    __syncthreads();                                        \
    ++s;                                                    \
  }
#define LMH_TAIL_STEP(NXT)                                  \
  if (s < nS) {                                             \
    const int buf = s & 1;                                  \
    LMH_COMPUTE(buf);                                       \
    if (s + 1 < nS) LMH_LSTORE(NXT, buf ^ 1);               \
    __syncthreads();                                        \
    ++s;                                                    \
  }

  LMH_GLOAD(p0, 0);
  LMH_GLOAD(p1, min(1, nS - 1) * kBK);
  if constexpr (NSET == 4) {
    LMH_GLOAD(p2, min(2, nS - 1) * kBK);
    LMH_GLOAD(p3, min(3, nS - 1) * kBK);
  }
  LMH_LSTORE(p0, 0);
  __syncthreads();
  int s = 0;
  if constexpr (NSET == 4) {
    while (s + 4 <= nS) {
      LMH_STEP(p0, p1)
      LMH_STEP(p1, p2)
      LMH_STEP(p2, p3)
      LMH_STEP(p3, p0)
    }
    LMH_TAIL_STEP(p1)
    LMH_TAIL_STEP(p2)
    LMH_TAIL_STEP(p3)
  } else {
    while (s + 2 <= nS) {
      LMH_STEP(p0, p1)
      LMH_STEP(p1, p0)
    }
    LMH_TAIL_STEP(p1)
  }
#undef LMH_TAIL_STEP
#undef LMH_STEP
#undef LMH_COMPUTE
#undef LMH_GLOAD
#undef LMH_LSTORE

  // Epilogue.  Accumulator element e of block (i, j) is row
  // wm*32*IM + i*32 + 8*(e/4) + 4*(lane/32) + e%4 and column wn*128 + j*32 + lane%32
  // of the tile.  For one (i, e) a lane holds 4 columns of one row (j = 0..3):
  // a group; the 32 lanes of a half-wave hold that row's other groups.
  const uint64_t half = lane < 32 ? 0x00000000FFFFFFFFull : 0xFFFFFFFF00000000ull;
  const uint64_t lt = (1ull << lane) - 1ull;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < IM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rt = wm * 32 * IM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const int grow = row0 + rt;
      float x[4];
      bool ok[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = acc[i][j][e];
        ok[j] = col0 + wn * 128 + j * 32 + lr < a.V;
      }
      if (SAMPLE) {
        uint32_t g = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (ok[j]) g = max(g, f32_key(__float_as_uint(x[j])));
        if (grow < a.M)
          a.samp[(size_t)grow * ((size_t)a.S * GPT) + (size_t)vt_i * GPT + wn * 32 + lr] = g;
      } else {
        // partial log-sum-exp over this wave's 128 columns of the row
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ok[j]) {
            bad |= !__builtin_isfinite(x[j]);
            mx = fmaxf(mx, x[j]);
          }
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
        float sm = 0.0f;
        if (mx > -INFINITY) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (ok[j]) sm += __expf(x[j] - mx);
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) sm += __shfl_xor(sm, o, kWave);
        if (lr == 0 && grow < a.M) a.part[(size_t)grow * (WGN * (size_t)a.T) + WGN * vt + wn] = make_float2(mx, sm);

        // candidates: logits at or above the row's threshold
        const uint32_t th = sthr[rt];
        bool p[4];
        uint32_t kx[4];
        int before = 0, total = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kx[j] = f32_key(__float_as_uint(x[j]));
          p[j] = ok[j] && kx[j] >= th;
          const uint64_t b = __ballot(p[j]);
          before += __popcll(b & half & lt);
          total += __popcll(b & half);
        }
        int base = 0;
        if (lr == 0 && total > 0 && grow < a.M) base = atomicAdd(&a.cand_count[grow], total);
        base = __shfl(base, lane & 32, kWave);
        if (grow < a.M) {
          int pos = base + before;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (p[j]) {
              if (pos < a.C) a.cand[(size_t)grow * a.C + pos] = cand_composite(kx[j], (uint32_t)(col0 + wn * 128 + j * 32 + lr));
              ++pos;
            }
          }
        }
      }
    }
  }
  if (!SAMPLE && bad && a.status != nullptr) {
    // rows of this lane's tile part: flag every tree the tile touches that holds a bad value
#pragma unroll
    for (int i = 0; i < IM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int grow = row0 + wm * 32 * IM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        bool rb_ = false;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          rb_ |= (col0 + wn * 128 + j * 32 + lr < a.V) && !__builtin_isfinite(acc[i][j][e]);
        if (rb_ && grow < a.M) atomicOr(&a.status[grow / a.rows_per_tree], MFD_TREE_NONFINITE);
      }
    }
  }
}

// Per row: the candidate threshold (k-th largest group maximum, or 0 = take
// every column when the sample holds fewer than k groups); resets the row's
// candidate count.
__global__ void __launch_bounds__(kThrNT) lmh_threshold_kernel(LmhArgs a, int k) {
  __shared__ uint32_t hist[256];
  __shared__ int sh[2];
  __shared__ int red[kThrNT / kWave];
  const int row = (int)blockIdx.x;
  const int n = a.S * a.gpt;
  const uint32_t* g = a.samp + (size_t)row * n;
  int cnt = 0;
  for (int i = threadIdx.x; i < n; i += kThrNT) cnt += g[i] != 0u ? 1 : 0;
  cnt = block_sum<kThrNT>(cnt, red);
  uint32_t thr = 0;
  if (cnt >= k) {
    thr = (uint32_t)block_kth_largest<kThrNT, 32>(
        n, k,
        [&](int i, uint64_t* key) {
          *key = g[i];
          return g[i] != 0u;
        },
        hist, sh);
  }
  if (threadIdx.x == 0) {
    a.thr[row] = thr;
    a.cand_count[row] = 0;
  }
}

// Per row: log-normaliser from the tile partials, then the exact top-k of the
// candidate list (largest composites = largest logits, ties by lower id),
// written in descending order.
__global__ void __launch_bounds__(kSelNT) lmh_select_kernel(LmhArgs a, int k, double* __restrict__ lse,
                                                            int32_t* __restrict__ topk_id,
                                                            float* __restrict__ topk_raw,
                                                            float* __restrict__ topk_logp) {
  extern __shared__ __attribute__((aligned(16))) uint64_t lds[];  // kSelLdsCap candidates, then the sort area
  __shared__ uint32_t hist[256];
  __shared__ int sh[2];
  __shared__ int red[kSelNT / kWave];
  __shared__ float redf[kSelNT / kWave];
  __shared__ double redd[kSelNT / kWave];
  __shared__ int nsel;
  const int row = (int)blockIdx.x;
  const int tid = (int)threadIdx.x, lane = lane_id(), w = wave_id();
  const int np = a.wgn * a.T;
  const float2* part = a.part + (size_t)row * np;

  // 1. lse = M + log sum_t s_t exp(m_t - M), fp64, fixed reduction order
  float mx = -INFINITY;
  for (int i = tid; i < np; i += kSelNT) mx = fmaxf(mx, part[i].x);
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  if (lane == 0) redf[w] = mx;
  __syncthreads();
  mx = redf[0];
#pragma unroll
  for (int i = 1; i < kSelNT / kWave; ++i) mx = fmaxf(mx, redf[i]);
  double s = 0.0;
  if (mx > -INFINITY) {
    for (int i = tid; i < np; i += kSelNT) {
      const float2 p = part[i];
      if (p.x > -INFINITY) s += (double)p.y * exp((double)p.x - (double)mx);
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (lane == 0) redd[w] = s;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < kSelNT / kWave; ++i) tot += redd[i];
  const double l = mx > -INFINITY ? (double)mx + log(tot) : -INFINITY;
  if (tid == 0) lse[row] = l;

  // 2. candidates
  const int cnt = a.cand_count[row];
  int32_t* oid = topk_id + (size_t)row * k;
  float* oraw = topk_raw + (size_t)row * k;
  float* olp = topk_logp ? topk_logp + (size_t)row * k : nullptr;
  if (cnt > a.C || cnt < k) {
    // more candidates than the workspace holds (or, defensively, too few)
    for (int j = tid; j < k; j += kSelNT) {
      oid[j] = -1;
      oraw[j] = -INFINITY;
      if (olp) olp[j] = -INFINITY;
    }
    if (tid == 0 && a.status) atomicOr(&a.status[row / a.rows_per_tree], MFD_TREE_CAPACITY);
    return;
  }
  const uint64_t* cg = a.cand + (size_t)row * a.C;
  const bool in_lds = cnt <= kSelLdsCap;
  uint64_t* sortb = lds + kSelLdsCap;
  if (in_lds)
    for (int i = tid; i < cnt; i += kSelNT) lds[i] = cg[i];
  __syncthreads();
  const uint64_t* src = in_lds ? lds : cg;

  // 3. The k-th largest key.  Every candidate's key is >= the row's threshold
  //    key, so the search runs on rel = key - thr from the highest byte that is
  //    not zero in every rel: candidates spread over the histogram bins instead
  //    of piling into the one or two bins of their shared top byte.
  const uint32_t thr = a.thr[row];
  uint32_t mr = 0;
  for (int i = tid; i < cnt; i += kSelNT) mr = max(mr, (uint32_t)(src[i] >> 32) - thr);
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) mr = max(mr, (uint32_t)__shfl_xor((int)mr, o, kWave));
  if (lane == 0) red[w] = (int)mr;
  __syncthreads();
  mr = 0;
#pragma unroll
  for (int i = 0; i < kSelNT / kWave; ++i) mr = max(mr, (uint32_t)red[i]);
  const int top = mr == 0 ? 0 : 31 - __clz((int)mr);
  uint32_t prefix = 0;
  int remaining = k, ties = 0;
  for (int shift = (top / 8) * 8; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelNT) hist[i] = 0;
    __syncthreads();
    const uint64_t hi = (uint64_t)prefix >> (shift + 8);
    for (int i = tid; i < cnt; i += kSelNT) {
      const uint32_t rel = (uint32_t)(src[i] >> 32) - thr;
      if (((uint64_t)rel >> (shift + 8)) == hi) atomicAdd(&hist[(rel >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      int digit = 0, above = 0;
      wave_pick_digit(hist, remaining, &digit, &above);
      int d = digit, ab = above;
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        d = max(d, __shfl_xor(d, o, kWave));
        ab = max(ab, __shfl_xor(ab, o, kWave));
      }
      if (tid == 0) {
        sh[0] = d;
        sh[1] = ab;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh[0] << shift;
    remaining -= sh[1];
    ties = (int)hist[sh[0]];
    __syncthreads();
  }
  // candidates above the k-th key all make the list (k - remaining of them);
  // of the `ties` candidates at it, the `remaining` with the lowest ids do
  const uint32_t kkey = thr + prefix;
  uint64_t kth = (uint64_t)kkey << 32;  // every tie is taken
  if (ties > remaining) {
    kth = block_kth_largest<kSelNT, 32>(
              cnt, remaining,
              [&](int i, uint64_t* key) {
                *key = (uint32_t)src[i];
                return (uint32_t)(src[i] >> 32) == kkey;
              },
              hist, sh) |
          ((uint64_t)kkey << 32);
  }

  // 4. gather the k composites >= kth (composites are distinct), sort, write descending
  const int P = next_pow2(k);
  for (int i = tid; i < P; i += kSelNT) sortb[i] = 0ull;
  if (tid == 0) nsel = 0;
  __syncthreads();
  for (int i = tid; i < cnt; i += kSelNT) {
    const uint64_t c = src[i];
    if (c >= kth) {
      const int slot = atomicAdd(&nsel, 1);
      if (slot < k) sortb[P - k + slot] = c;
    }
  }
  __syncthreads();
  block_sort_keys<kSelNT>(sortb, P);
  for (int j = tid; j < k; j += kSelNT) {
    const uint64_t c = sortb[P - 1 - j];
    const uint32_t key = (uint32_t)(c >> 32);
    const float raw = __uint_as_float(f32_from_key(key));
    const int32_t col = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
    oid[j] = a.vocab_map ? a.vocab_map[col] : col;
    oraw[j] = raw;
    if (olp) olp[j] = (float)((double)raw - l);
  }
}

// Packed head: rows padded to a multiple of 256 (zeros), cut into blocks of 64
// rows x 32 k, block (vb, s) stored contiguously at ((vb * nS) + s) * 2048
// elements, row-major inside (row r, k-chunk q of 8 at (4 r + q) * 8).  One
// thread copies one 16-byte chunk.
__global__ void __launch_bounds__(256) lmh_pack_kernel(const uint16_t* __restrict__ W, int V, int D,
                                                      uint16_t* __restrict__ Wp, long long nchunks) {
  const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int nS = D / kBK;
  const long long blk = c >> 8;
  const int t = (int)(c & 255);
  const long long vb = blk / nS;
  const int s = (int)(blk - vb * nS);
  const long long row = vb * 64 + (t >> 2);
  const int k = s * kBK + (t & 3) * 8;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < V) v = *reinterpret_cast<const uint4*>(W + row * (long long)D + k);
  *reinterpret_cast<uint4*>(Wp + c * 8) = v;
}

}  // namespace

size_t lmhead_packed_bytes(int V, int D) { return (size_t)((V + 255) / 256) * 256 * (size_t)D * 2; }

hipError_t launch_lmhead_pack(const void* weight, int V, int D, void* packed, hipStream_t stream) {
  const long long nchunks = (long long)((V + 255) / 256) * 256 * D / 8;
  const long long blocks = (nchunks + 255) / 256;
  hipLaunchKernelGGL(lmh_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(weight), V, D, static_cast<uint16_t*>(packed), nchunks);
  return hipGetLastError();
}

LmhWorkspace lmhead_workspace(long long M, int V, int k) {
  LmhWorkspace w{};
  w.small = M <= kSmallM;
  const int BN = w.small ? TileShape<4>::BN : TileShape<2>::BN;
  w.gpt = w.small ? TileShape<4>::GPT : TileShape<2>::GPT;
  w.wgn = w.small ? TileShape<4>::WGN : TileShape<2>::WGN;
  w.T = (V + BN - 1) / BN;
  w.S = w.T < kSampleCols / BN ? w.T : kSampleCols / BN;
  // about k V / (S * BN) candidates per row for rows of independent logits;
  // four times that leaves room for rows of uneven spread
  const long long expect = ((long long)k * V + (long long)w.S * BN - 1) / ((long long)w.S * BN);
  long long C = 4 * expect;
  if (C < 2LL * k) C = 2LL * k;
  if (C < 4096) C = 4096;
  C = (C + 255) / 256 * 256;
  const long long vcap = ((long long)V + 255) / 256 * 256;
  if (C > vcap) C = vcap;
  w.C = (int)C;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.off_samp = take((size_t)M * w.S * w.gpt * sizeof(uint32_t));
  w.off_thr = take((size_t)M * sizeof(uint32_t));
  w.off_count = take((size_t)M * sizeof(int));
  w.off_part = take((size_t)M * w.wgn * w.T * sizeof(float2));
  w.off_cand = take((size_t)M * w.C * sizeof(uint64_t));
  w.bytes = off;
  return w;
}

hipError_t launch_lmhead_topk(const void* hidden, const void* weight, bool packed, const int32_t* vocab_map, int M,
                              int rows_per_tree, int D, int V, int k, double* lse, int32_t* topk_id, float* topk_raw,
                              float* topk_logp, int32_t* status, void* ws, hipStream_t stream) {
  const LmhWorkspace wsl = lmhead_workspace(M, V, k);
  char* base = static_cast<char*>(ws);
  LmhArgs a;
  a.H = static_cast<const uint16_t*>(hidden);
  a.W = static_cast<const uint16_t*>(weight);
  a.M = M;
  a.D = D;
  a.V = V;
  a.T = wsl.T;
  a.S = wsl.S;
  a.gpt = wsl.gpt;
  a.wgn = wsl.wgn;
  a.rows_per_tree = rows_per_tree;
  a.samp = reinterpret_cast<uint32_t*>(base + wsl.off_samp);
  a.thr = reinterpret_cast<uint32_t*>(base + wsl.off_thr);
  a.cand_count = reinterpret_cast<int*>(base + wsl.off_count);
  a.part = reinterpret_cast<float2*>(base + wsl.off_part);
  a.cand = reinterpret_cast<uint64_t*>(base + wsl.off_cand);
  a.C = wsl.C;
  a.status = status;
  a.vocab_map = vocab_map;
  a.packed = packed ? 1 : 0;
  const int nM = (M + kBM - 1) / kBM;
  const long long ns = (long long)nM * a.S, nm = (long long)nM * a.T;
  const long long gs = (ns + 7) / 8 * 8, gm = (nm + 7) / 8 * 8;
  if (wsl.small) {
    hipLaunchKernelGGL((lmh_tile_kernel<true, 4>), dim3((unsigned)gs), dim3(kNT), 0, stream, a);
    hipLaunchKernelGGL(lmh_threshold_kernel, dim3(M), dim3(kThrNT), 0, stream, a, k);
    hipLaunchKernelGGL((lmh_tile_kernel<false, 4>), dim3((unsigned)gm), dim3(kNT), 0, stream, a);
  } else {
    hipLaunchKernelGGL((lmh_tile_kernel<true, 2>), dim3((unsigned)gs), dim3(kNT), 0, stream, a);
    hipLaunchKernelGGL(lmh_threshold_kernel, dim3(M), dim3(kThrNT), 0, stream, a, k);
    hipLaunchKernelGGL((lmh_tile_kernel<false, 2>), dim3((unsigned)gm), dim3(kNT), 0, stream, a);
  }
  const size_t lds = (size_t)(kSelLdsCap + next_pow2(k)) * sizeof(uint64_t);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lmh_select_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lmh_select_kernel, dim3(M), dim3(kSelNT), lds, stream, a, k, lse, topk_id, topk_raw, topk_logp);
  return hipGetLastError();
}

}  // namespace mfd
