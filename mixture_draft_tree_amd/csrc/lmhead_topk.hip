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
//   1. sample  S spread vocabulary blocks of the product; per row the maximum
//      of every disjoint group of 4 columns goes to `samp`.
//   2. lmh_threshold_kernel    per row: thr = the k-th largest of those group
//      maxima.  They are k distinct elements of the row, so the row's k-th
//      largest logit is >= thr: every top-k element passes x >= thr.  Rows with
//      fewer than k groups take thr = "everything".
//   3. main    every column of the product; per row and tile (or wave) the
//      partial (max, sum exp(x - max)); every logit >= thr is appended to its
//      row's candidate list.
//   4. lmh_select_kernel       per row: lse from the partials (fp64), the exact
//      k-th largest (logit desc, id asc) among the candidates, those k sorted.
//
// Launches 1 and 3 run one of two kernels, both on the matrix cores with fp32
// accumulation:
//   - up to 128 rows (one tree): lmh_skinny_kernel, one workgroup per CU, each
//     wave streaming its own head columns through an LDS ring (below);
//   - more rows: lmh_tile_kernel, 128 rows x 256 vocabulary columns per
//     256-thread workgroup (128 x 128 up to 256 rows), two workgroups per CU,
//     k in steps of 32 through double-buffered, XOR-swizzled LDS (global loads
//     two steps ahead), four waves of 64 x 128 each built from
//     v_mfma_f32_32x32x16_bf16.
// Each product element is computed from the same operands in the same k order
// in both launches of a call, so the sample and main launches see identical
// logits.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

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
constexpr int kCountStride = 32;   // ints between row counters: one 128-byte line per row, so
                                   // the many adds to different rows do not meet on one line
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
constexpr int kThrNT = 1024;  // threshold kernel: up to 2048 sample keys per row, two per thread
constexpr int kSelNT = 1024;  // select kernel: thousands of candidates per row
constexpr int kSelLdsCap = 8192;  // candidates a select workgroup holds in LDS

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
  int* cand_count;      // [M * kCountStride]: row r's count at r * kCountStride
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
        if (lr == 0 && total > 0 && grow < a.M) base = atomicAdd(&a.cand_count[(size_t)grow * kCountStride], total);
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

// ---------------------------------------------------------------------------
// Few rows (M <= 128, one tree): the head streamed once, through a per-wave
// LDS ring filled by loads that write LDS directly.  At one tree the
// contraction needs ~1/3 of the matrix cores' rate to keep pace with the head
// read, so what sets the pace is how many head bytes are in flight per CU:
// the accumulators of a wave's 128 rows x 80 columns hold 160 of its 256
// registers, which leaves room for about one 32-deep step of head fragments
// in registers, and a step then waits out a full memory latency.  Loads
// straight into LDS (global_load_lds_dwordx4) hold no registers while in
// flight.  Here:
//   - one 512-thread workgroup per CU; each wave owns up to kSkNB blocks of 16
//     consecutive head rows (vocabulary columns), so a launch covers the
//     vocabulary in one round with at most one block of imbalance per wave;
//   - each wave keeps its head fragments for the next R steps in its own LDS
//     ring (R x blocks x 1 KB; R = 2 for the main launch, 8 for the one-block
//     sample waves) and reads a step's fragments back as the MFMA A operand
//     (v_mfma_f32_16x16x32_bf16: lane l holds column 16 b + l % 16, k-offset
//     8 (l / 16) .. + 7); the loads fill a slot with the block's 16 rows x
//     64 bytes row-major, chunks swizzled as for the hidden rows; the packed
//     layout makes each block's step one contiguous 1 KB run;
//   - the hidden rows (B operand, all 128 rows) sit in a ring of eight 32-deep
//     steps, four chunks of two: at the start of a chunk each wave loads its
//     16 rows of the chunk three ahead, and one barrier per chunk publishes
//     the next one.
// The loop issues no other vector memory loads, so each wait counts exactly
// the ring loads issued after the one it needs.
// Accumulator element r of block (b, rb) in lane l is column 16 b + 4 (l / 16)
// + r and row 16 rb + l % 16: a lane holds groups of 4 consecutive columns of
// one row, and the 4 lanes l % 16 = j share row j.
constexpr int kSkWaves = 8;      // waves per workgroup of the main launch
constexpr int kSkSampleWaves = 2;  // ... and of the sample launch
constexpr int kSkRows = 128, kSkRB = kSkRows / 16;
constexpr int kSkNB = 5;      // 16-column blocks per wave (at most)
constexpr int kSkSampleBlocks = kSampleCols / 16;
constexpr int kSkCUs = 256;   // MI355X compute units: workgroups of one launch round
template <int NB, int WV>
struct SkRing {
  static constexpr int R = NB == 1 ? 8 : 2;  // head steps in flight per wave
  static constexpr int HS = 8;               // 32-deep steps of hidden rows in LDS: 4 chunks of 2
  static constexpr int HD = kSkRows / 16 / WV;  // 16-row hidden loads per wave and step
  static constexpr size_t rings = (size_t)WV * R * NB * 1024 + (size_t)HS * kSkRows * 64;
  // then per row: threshold key, this workgroup's candidate count, its base in
  // the row's list; per wave its staged candidate count; per wave and row its
  // partial (max, sum exp(x - max))
  static constexpr size_t lds = rings + (3 * kSkRows + WV) * sizeof(uint32_t) + (size_t)WV * kSkRows * sizeof(float2);
  // after the loop the rings hold the staged candidates, a run of wave_cap
  // per wave: composites, then (row | offset in the workgroup's run << 8)
  static constexpr int wave_cap = (int)(rings / 12 / WV);
};
static_assert(SkRing<kSkNB, kSkWaves>::lds <= 160 * 1024 && SkRing<1, kSkSampleWaves>::lds <= 160 * 1024,
              "LDS of a CU");

// One 16-byte-per-lane load straight into LDS (buffer_load_dwordx4 ... lds):
// lane l reads bytes [soff + voff, + 16) of the buffer described by rsrc
// (reads past its size return zeros) and its 16 bytes land at LDS byte
// address lds + 16 l (lds wave-uniform, passed in M0).  Written as assembly
// because the compiler waits for every load in flight before any LDS read
// that follows the builtin form; the waits here are sk_vm_wait's.  The
// instruction has no register result.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void sk_dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
               : "memory", "m0");
}
// Raw buffer descriptor: base, no stride, `bytes` long (gfx9 word 3).
__device__ __forceinline__ i32x4 sk_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// Wait until at most N vector memory loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void sk_vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// The same with N = (loads per step) * S + H for a wave of nb head blocks
// (nb wave-uniform; NB or NB - 1 in a launch that spreads blocks evenly, 0
// or other values only for tiny vocabularies, which wait for everything).
template <int NB, int S, int H>
__device__ __forceinline__ void sk_vm_wait_nb(int nb) {
  if (nb == NB)
    sk_vm_wait<NB * S + H>();
  else if (NB > 1 && nb == NB - 1)
    sk_vm_wait<(NB > 1 ? NB - 1 : 0) * S + H>();
  else
    sk_vm_wait<0>();
}

// f32_key of a logit as the matrix cores produce it (adding +0 turns -0
// into +0; a NaN stays quiet, so its bits and key are those f32_key gives).
__device__ __forceinline__ uint32_t sk_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ ((uint32_t)((int)u >> 31) | 0x80000000u);
}

// Vocabulary block of work item i: every block in the main launch, nwork
// spread ones in the sample launch.
__device__ __forceinline__ int sk_vblock(bool sample, int i, int nblk, int nwork) {
  return sample ? (int)(((long long)i * nblk) / nwork) : i;
}

template <bool SAMPLE, int NB, int WV>
__global__ void __launch_bounds__(WV * kWave, 1) lmh_skinny_kernel(LmhArgs a, int nwork, int nw_total) {
  using Cfg = SkRing<NB, WV>;
  constexpr int R = Cfg::R, HS = Cfg::HS, HD = Cfg::HD, NT = WV * kWave;
  static_assert(HS % 2 == 0 && HS >= 4 && (HS & (HS - 1)) == 0, "whole chunks of two steps, power of two");
  // [wave][slot][block] 1 KB head fragments, then [HS][128 rows x 4 chunks] hidden rows
  extern __shared__ __attribute__((aligned(16))) uint4 sk_lds[];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int gw = (int)blockIdx.x * WV + w;
  const int D = a.D, nS = D / 32;
  const int nblk = (a.V + 15) / 16;
  const int b0 = (int)(((long long)gw * nwork) / nw_total);
  const int nbc = (int)(((long long)(gw + 1) * nwork) / nw_total) - b0;  // blocks of this wave, 0..NB
  const int lj = lane & 15, lq = lane >> 4;

  // byte offset of this lane's 16 bytes of each block's head fragment at step
  // 0 (V D and the packed size are below 2^31 elements).  Lane l loads head
  // row 16 vbk + l / 4, the 16-byte chunk that lds_chunk puts at position
  // l % 4 of the row's 64 bytes, so a slot holds the 16 rows x 64 bytes
  // row-major and swizzled like the hidden rows, and a quarter-wave of a
  // row-major load reads 4 rows x 64 bytes
  const int wr_ = lane >> 2, wq_ = (lane & 3) ^ lds_chunk(wr_, 0);
  uint32_t woff[NB];
  int vbk[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    vbk[b] = sk_vblock(SAMPLE, min(b0 + b, nwork - 1), nblk, nwork);
    if (a.packed) {
      // block (vbk / 4, step) of 64 rows x 32 k is 2048 contiguous elements,
      // row-major; this 16-row block is its (vbk % 4)-th 512
      woff[b] = 2u * ((uint32_t)(vbk[b] >> 2) * (uint32_t)nS * 2048u + (uint32_t)(vbk[b] & 3) * 512u + (uint32_t)(4 * wr_ + wq_) * 8u);
    } else {
      woff[b] = 2u * ((uint32_t)min(16 * vbk[b] + wr_, a.V - 1) * (uint32_t)D + (uint32_t)(8 * wq_));
    }
  }
  const uint32_t wstep = a.packed ? 4096u : 64u;  // bytes per 32-deep step
  const uint32_t wbytes = 2u * (a.packed ? (uint32_t)((a.V + 255) / 256) * 256u * (uint32_t)D : (uint32_t)a.V * (uint32_t)D);
  const i32x4 wrs = sk_rsrc(a.W, wbytes);
  const i32x4 hrs = sk_rsrc(a.H, 2u * (uint32_t)a.M * (uint32_t)D);
  // hidden rows: load j of this wave brings rows 16 (HD w + j) .. + 15, lane l
  // row 16 (HD w + j) + l / 4, the 16-byte chunk that the swizzle lds_chunk
  // puts at position l % 4 of the row's 64 bytes
  uint32_t hoff[HD];
#pragma unroll
  for (int j = 0; j < HD; ++j) {
    const int hr = 16 * (HD * w + j) + (lane >> 2);
    hoff[j] = 2u * ((uint32_t)min(hr, a.M - 1) * (uint32_t)D + 8u * (uint32_t)((lane & 3) ^ lds_chunk(hr, 0)));
  }

  const uint32_t lds0 = (uint32_t)(uintptr_t)sk_lds;
  const uint32_t ring = lds0 + (uint32_t)(w * R * NB) * 1024u;
  const uint32_t hbase = lds0 + (uint32_t)(WV * R * NB) * 1024u;
  // uint4 index of this lane's A operand (column lj, k-chunk lq) in slot 0, block 0
  const int ring_u4 = w * R * NB * 64 + 4 * lj + lds_chunk(lj, lq);
  const int hbase_u4 = WV * R * NB * 64;
  auto wdma = [&](int g) {  // head fragments of step g into slot g mod R (g outside [0, nS): a
                            // real step again, whose data is overwritten or never read)
    const int gs = min(max(g, 0), nS - 1);
    const uint32_t slot = ring + (uint32_t)((((g % R) + R) % R) * NB) * 1024u;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < nbc) sk_dma16(wrs, woff[b], (uint32_t)gs * wstep, slot + (uint32_t)b * 1024u);
  };
  auto hdma = [&](int g) {  // this wave's hidden rows of step g into slot g mod HS (g < 0: step 0, unused)
#pragma unroll
    for (int j = 0; j < HD; ++j)
      sk_dma16(hrs, hoff[j], 64u * (uint32_t)min(max(g, 0), nS - 1),
               hbase + (uint32_t)(g & (HS - 1)) * 8192u + (uint32_t)(HD * w + j) * 1024u);
  };

  f32x4 acc[NB][kSkRB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int rb = 0; rb < kSkRB; ++rb) acc[b][rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Step g: (B) wait for head step g; (C) read it from the ring, refill the
  // slot with step g + R; (A, even g) load the hidden rows of the chunk
  // HS / 2 - 1 ahead (steps g + HS - 2, g + HS - 1) into the slots of the
  // previous chunk (steps g - 2, g - 1); (D) the MFMAs of step g; (E, odd g)
  // wait for the hidden rows of the next chunk, loaded at step g + 3 - HS,
  // and publish them.
  // The prologue issues the loads of steps -S0 .. -1 (S0 = max(R, HS - 2)) in
  // that order, so every count below holds from step 0: head step s + R (for
  // s + R < 0, step 0 again into the slot of s + R, overwritten in order
  // later), and at even s the hidden rows of steps s + HS - 2 and s + HS - 1
  // (negative ones: step 0 again, into slots that are refilled in order later).
  constexpr int S0 = R > HS - 2 ? R : HS - 2;
#pragma unroll
  for (int s = -S0; s < 0; ++s) {
    wdma(s + R);
    if ((s & 1) == 0) {
      hdma(s + HS - 2);
      hdma(s + HS - 1);
    }
  }
  // chunk 0 (loaded at step 2 - HS) is followed by HS - 3 steps' head loads
  // and (HS - 4) HD hidden-row loads
  sk_vm_wait_nb<NB, HS - 3, (HS - 4) * HD>(nbc);
  uint32_t* sthr = reinterpret_cast<uint32_t*>(sk_lds + Cfg::rings / 16);
  int* wg_cnt = reinterpret_cast<int*>(sthr + kSkRows);
  int* wg_base = wg_cnt + kSkRows;
  int* wv_staged = wg_base + kSkRows;
  float2* wv_part = reinterpret_cast<float2*>(wv_staged + WV);  // [WV][kSkRows]
  if (!SAMPLE && (int)threadIdx.x < kSkRows) {
    // (this load completes before the barrier: no load of the compiler's is
    // in flight in the loop, whose waits count only the ring loads)
    sthr[threadIdx.x] = (int)threadIdx.x < a.M ? a.thr[threadIdx.x] : 0xFFFFFFFFu;
    wg_cnt[threadIdx.x] = 0;
  }
  __syncthreads();

  // (B) Loads issued after head step g's: head steps g + 1 .. g + R - 1, and
  // 2 HD hidden-row loads for each even step in [g - R, g - 1]: R / 2 such
  // steps for even R; (R - 1) / 2 for even g and (R + 1) / 2 for odd g when R
  // is odd.  (E) After the next chunk's hidden rows (issued at step
  // g + 3 - HS, even): HS - 3 steps' head loads and (HS - 4) HD hidden-row
  // loads.  nS is even (D is a multiple of 64), so chunks are whole.
  constexpr int kEvenH = 2 * HD * (R % 2 == 0 ? R / 2 : (R - 1) / 2);
  constexpr int kOddH = 2 * HD * (R % 2 == 0 ? R / 2 : (R + 1) / 2);
  for (int g0 = 0; g0 < nS; g0 += 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int g = g0 + p;
      if (p == 0)
        sk_vm_wait_nb<NB, R - 1, kEvenH>(nbc);
      else
        sk_vm_wait_nb<NB, R - 1, kOddH>(nbc);
      const int slot_u4 = ring_u4 + (g % R) * NB * 64;
      const int hs_u4 = hbase_u4 + (g & (HS - 1)) * 512;
      bf16x8 wf[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) wf[b] = __builtin_bit_cast(bf16x8, sk_lds[slot_u4 + b * 64]);
      // one-block waves have few MFMAs to hide LDS latency behind: all the
      // step's hidden-row fragments are read before the one wait
      bf16x8 hf1[NB == 1 ? kSkRB : 1];
      if constexpr (NB == 1) {
#pragma unroll
        for (int rb = 0; rb < kSkRB; ++rb) {
          const int r = rb * 16 + lj;
          hf1[rb] = __builtin_bit_cast(bf16x8, sk_lds[hs_u4 + 4 * r + lds_chunk(r, lq)]);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // ring reads done before the slot is refilled
      __builtin_amdgcn_sched_barrier(0);
      wdma(g + R);
      if (p == 0) {
        hdma(g + HS - 2);
        hdma(g + HS - 1);
      }
#pragma unroll
      for (int rb = 0; rb < kSkRB; ++rb) {
        const int r = rb * 16 + lj;
        const bf16x8 hf = NB == 1 ? hf1[NB == 1 ? rb : 0] : __builtin_bit_cast(bf16x8, sk_lds[hs_u4 + 4 * r + lds_chunk(r, lq)]);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[b], hf, acc[b][rb], 0, 0, 0);
      }
      if (p == 1) {
        sk_vm_wait_nb<NB, HS - 3, (HS - 4) * HD>(nbc);
        __syncthreads();
      }
    }
  }
  sk_vm_wait<0>();  // no load may still write this workgroup's LDS when it ends


  // Epilogue.  Column validity is the same for every block row: bit 4 b + r of
  // vmask says whether column 16 vbk[b] + 4 lq + r exists (b < nbc, below V).
  static_assert(NB * 4 <= 32, "validity bits");
  uint32_t vmask = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (b < nbc && 16 * vbk[b] + 4 * lq + r < a.V) vmask |= 1u << (4 * b + r);

  if (SAMPLE) {
    // per row, the maximum of each group of 4 columns (0 = no column)
#pragma unroll
    for (int rb = 0; rb < kSkRB; ++rb) {
      const int row = rb * 16 + lj;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        uint32_t gmax = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gmax = max(gmax, (vmask >> (4 * b + r)) & 1u ? sk_key(acc[b][rb][r]) : 0u);
        }
        if (b < nbc && row < a.M) a.samp[(size_t)row * ((size_t)a.S * 4) + (size_t)(b0 + b) * 4 + lq] = gmax;
      }
    }
    return;
  }

  // Main launch, per block row: the partial log-sum-exp over this wave's
  // columns of the row, the non-finite flag, and the candidates (logits at or
  // above the row's threshold), staged in LDS (the rings are free once every
  // wave has drained its loads) with their offsets in the workgroup's run of
  // the row's list.
  constexpr int kWCap = Cfg::wave_cap;
  constexpr int kOver = 0x40000000;  // in wg_cnt: a candidate of the row did not fit the stage
  uint64_t* stage_c = reinterpret_cast<uint64_t*>(sk_lds);
  uint32_t* stage_m = reinterpret_cast<uint32_t*>(stage_c + WV * kWCap);
  int staged = 0;  // this wave's candidates so far (wave-uniform)
  // every column of every lane exists: all waves but the last few
  const bool all_valid = __ballot(vmask != (NB * 4 == 32 ? 0xFFFFFFFFu : (1u << (NB * 4)) - 1u)) == 0ull;
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < kSkRB; ++rb) {
    const int row = rb * 16 + lj;
    const bool rok = row < a.M;
    float mx = -INFINITY, sm = 0.0f;
    bool bad = false;
    if (all_valid) {
      // a NaN logit turns the sum NaN, +inf the maximum, -inf the minimum
      float mn = INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mx = fmaxf(mx, acc[b][rb][r]);
          mn = fminf(mn, acc[b][rb][r]);
        }
      mx = fmaxf(mx, xor_lanes(mx, 16));
      mx = fmaxf(mx, xor_lanes(mx, 32));
      const float mxl = mx * 1.44269504088896341f;  // log2(e)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm += __builtin_amdgcn_exp2f(fmaf(acc[b][rb][r], 1.44269504088896341f, -mxl));
      sm += xor_lanes(sm, 16);
      sm += xor_lanes(sm, 32);
      mn = fminf(mn, xor_lanes(mn, 16));
      mn = fminf(mn, xor_lanes(mn, 32));
      bad = !__builtin_isfinite(sm) || !__builtin_isfinite(mx) || mn == -INFINITY;
      if (bad && !(mx > -INFINITY)) sm = 0.0f;
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = acc[b][rb][r];
          const bool v = (vmask >> (4 * b + r)) & 1u;
          bad |= v && !__builtin_isfinite(x);
          mx = fmaxf(mx, v ? x : -INFINITY);
        }
      mx = fmaxf(mx, xor_lanes(mx, 16));
      mx = fmaxf(mx, xor_lanes(mx, 32));
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool v = (vmask >> (4 * b + r)) & 1u;
          sm += v && mx > -INFINITY ? __expf(acc[b][rb][r] - mx) : 0.0f;
        }
      sm += xor_lanes(sm, 16);
      sm += xor_lanes(sm, 32);
      bad = __ballot(bad) != 0ull ? (xor_lanes((int)bad, 16) | xor_lanes((int)bad, 32) | xor_lanes(xor_lanes((int)bad, 16), 32) | (int)bad) != 0 : false;
    }
    if (lq == 0) wv_part[w * kSkRows + row] = make_float2(mx, sm);
    if (lq == 0 && bad && rok && a.status != nullptr) atomicOr(&a.status[row / a.rows_per_tree], MFD_TREE_NONFINITE);

    // candidate bits: key >= th, as a float compare where the lane's values
    // are finite (the key order is the float order there, -0 = +0); th = 0
    // (the sample held fewer than k groups) takes every column
    const uint32_t th = sthr[row];
    uint32_t pm = 0;
    if (th == 0u) {
      pm = 0xFFFFFFFFu;
    } else if (!bad) {
      const float tf = __uint_as_float(f32_from_key(th));
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) pm |= acc[b][rb][r] >= tf ? 1u << (4 * b + r) : 0u;
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) pm |= sk_key(acc[b][rb][r]) >= th ? 1u << (4 * b + r) : 0u;
    }
    pm &= rok ? vmask : 0u;
    // offsets: in the wave's stage run, a prefix over the wave; in the
    // workgroup's run of the row, one LDS add per row and wave (lane group 0)
    // plus a prefix over the row's 4 lanes (lanes l ^ 16, l ^ 32, l ^ 48 hold
    // lane groups lq ^ 1, lq ^ 2, lq ^ 3); a candidate's place in either is
    // then the count of candidate bits below its own
    const int cnt = __popc(pm);
    const int incl = wave_inclusive_scan(cnt);
    const int wtot = __builtin_amdgcn_readlane(incl, kWave - 1);
    if (wtot != 0) {
      const int c16 = xor_lanes(cnt, 16), c32 = xor_lanes(cnt, 32), c48 = xor_lanes(c16, 32);
      const int rtot = cnt + c16 + c32 + c48;
      int roff = 0;
      if (lq == 0 && rtot > 0) roff = atomicAdd(&wg_cnt[row], rtot) & (kOver - 1);
      const int r16 = xor_lanes(roff, 16), r32 = xor_lanes(roff, 32), r48 = xor_lanes(r16, 32);
      const int off = roff + r16 + r32 + r48 + ((lq ^ 1) < lq ? c16 : 0) + ((lq ^ 2) < lq ? c32 : 0) + ((lq ^ 3) < lq ? c48 : 0);
      const int gi = staged + incl - cnt;
      const bool fits = staged + wtot <= kWCap;  // wave-uniform
      if (!fits && cnt > 0 && gi + cnt > kWCap) atomicOr(&wg_cnt[row], kOver);
      const int sbase = w * kWCap;
      // this lane's candidates, lowest bit first (a lane holds few: the loop
      // runs as often as the wave's busiest lane needs)
      uint32_t m = pm;
      for (int j = 0; m != 0u; ++j) {
        const int bit = __builtin_ctz(m);
        m &= m - 1u;
        const int bb = bit >> 2, rr = bit & 3;
        f32x4 v = acc[0][rb];
#pragma unroll
        for (int b = 1; b < NB; ++b) v = bb == b ? acc[b][rb] : v;
        const float x = rr == 0 ? v[0] : rr == 1 ? v[1] : rr == 2 ? v[2] : v[3];
        int vb = vbk[0];
#pragma unroll
        for (int b = 1; b < NB; ++b) vb = bb == b ? vbk[b] : vb;
        if (fits || gi + j < kWCap) {
          stage_c[sbase + gi + j] = cand_composite(sk_key(x), (uint32_t)(16 * vb + 4 * lq + rr));
          stage_m[sbase + gi + j] = (uint32_t)row | ((uint32_t)(off + j) << 8);
        }
      }
      staged += wtot;
    }
  }
  if (lane == 0) wv_staged[w] = min(staged, kWCap);

  // one add per row and workgroup reserves the workgroup's run of the row's
  // list (a row with unstaged candidates is pushed past the capacity, which
  // the select kernel reports); then the stage is copied out
  __syncthreads();
  if ((int)threadIdx.x < kSkRows) {
    // the workgroup's partial of the row: its waves' partials combined
    const int row = (int)threadIdx.x;
    float pm = -INFINITY;
#pragma unroll
    for (int i = 0; i < WV; ++i) pm = fmaxf(pm, wv_part[i * kSkRows + row].x);
    float ps = 0.0f;
    if (pm > -INFINITY) {
#pragma unroll
      for (int i = 0; i < WV; ++i) {
        const float2 q = wv_part[i * kSkRows + row];
        if (q.x > -INFINITY) ps += q.y * __expf(q.x - pm);
      }
    }
    if (row < a.M) a.part[(size_t)row * gridDim.x + blockIdx.x] = make_float2(pm, ps);
    const int n = wg_cnt[threadIdx.x];
    int base = 0;
    if (n != 0 && (int)threadIdx.x < a.M) {
      int* cc = &a.cand_count[(size_t)threadIdx.x * kCountStride];
      base = (n & kOver) ? atomicAdd(cc, a.C + 1) + a.C + 1 : atomicAdd(cc, n);
    }
    wg_base[threadIdx.x] = base;
  }
  __syncthreads();
  for (int i = (int)threadIdx.x; i < WV * kWCap; i += NT) {
    const int sw = i / kWCap;
    if (i - sw * kWCap >= wv_staged[sw]) continue;
    const uint32_t m = stage_m[i];
    const int row = (int)(m & 255u);
    const int pos = wg_base[row] + (int)(m >> 8);
    if (pos < a.C) a.cand[(size_t)row * a.C + pos] = stage_c[i];
  }
}

// Per row: the candidate threshold, or 0 = take every column when the sample
// holds fewer than k groups; resets the row's candidate count.  The threshold
// is the lower edge of the histogram bin that holds the k-th largest group
// maximum, in 4096 bins over the row's range of group-maximum keys: at least
// k of those maxima (k distinct elements of the row) lie at or above it, so
// the row's k-th largest logit does too.  One pass over keys held in
// registers; the bins are a 4096th of the range, so the threshold sits at
// most that far below the k-th largest maximum.
constexpr int kThrBins = 4096;
static_assert(kSampleCols / 4 <= 2 * kThrNT && kThrBins == 4 * kThrNT, "keys and bins per thread");
__global__ void __launch_bounds__(kThrNT) lmh_threshold_kernel(LmhArgs a, int k) {
  __shared__ uint32_t hist[kThrBins];
  __shared__ uint32_t red[3][kThrNT / kWave];
  __shared__ int found;
  const int row = (int)blockIdx.x, tid = (int)threadIdx.x, lane = lane_id(), w = wave_id();
  const int n = a.S * a.gpt;
  const uint32_t* g = a.samp + (size_t)row * n;
  uint32_t kv[2];
  int cnt = 0;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + j * kThrNT;
    kv[j] = i < n ? g[i] : 0u;  // 0: a group with no column
    if (kv[j] != 0u) {
      ++cnt;
      lo = min(lo, kv[j]);
      hi = max(hi, kv[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) hist[4 * tid + j] = 0u;
  cnt = wave_allreduce(cnt, [](int x, int y) { return x + y; });
  lo = wave_allreduce(lo, [](uint32_t x, uint32_t y) { return min(x, y); });
  hi = wave_allreduce(hi, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (lane == 0) {
    red[0][w] = (uint32_t)cnt;
    red[1][w] = lo;
    red[2][w] = hi;
  }
  if (tid == 0) found = 0;
  __syncthreads();
  cnt = 0;
  lo = 0xFFFFFFFFu;
  hi = 0u;
#pragma unroll
  for (int i = 0; i < kThrNT / kWave; ++i) {
    cnt += (int)red[0][i];
    lo = min(lo, red[1][i]);
    hi = max(hi, red[2][i]);
  }
  uint32_t thr = 0u;
  if (cnt >= k) {
    const uint32_t range = hi - lo;
    const int bits = range == 0u ? 0 : 32 - __clz((int)range);
    const int shift = bits > 12 ? bits - 12 : 0;  // (range >> shift) < kThrBins
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (kv[j] != 0u) atomicAdd(&hist[(kv[j] - lo) >> shift], 1u);
    __syncthreads();
    // thread t holds bins 4095 - 4 t .. 4092 - 4 t (thread 0 the highest):
    // a prefix over threads counts the keys in higher bins
    uint32_t hb[4];
    int c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hb[j] = hist[kThrBins - 1 - 4 * tid - j];
      c += (int)hb[j];
    }
    const int incl = wave_inclusive_scan(c);
    __syncthreads();  // hist reads done; red is reused
    if (lane == kWave - 1) red[0][w] = (uint32_t)incl;
    __syncthreads();
    int above = incl - c;
    for (int i = 0; i < w; ++i) above += (int)red[0][i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int now = above + (int)hb[j];
      if (above < k && now >= k) found = kThrBins - 1 - 4 * tid - j;  // exactly one bin
      above = now;
    }
    __syncthreads();
    thr = lo + ((uint32_t)found << shift);
  }
  if (tid == 0) {
    a.thr[row] = thr;
    a.cand_count[(size_t)row * kCountStride] = 0;
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
  // the row maximum's own term is about 1, but exp2-domain rounding can leave
  // the sum just under it; the normaliser is kept at or above the maximum
  // (a NaN sum stays NaN)
  double lg = log(tot);
  lg = lg < 0.0 ? 0.0 : lg;
  const double l = mx > -INFINITY ? (double)mx + lg : -INFINITY;
  if (tid == 0) lse[row] = l;

  // 2. candidates
  const int cnt = a.cand_count[(size_t)row * kCountStride];
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
  if (in_lds) {
    // all of this thread's loads in flight at once, then the LDS writes
    constexpr int kPer = kSelLdsCap / kSelNT;
    uint64_t cv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) cv[j] = tid + j * kSelNT < cnt ? cg[tid + j * kSelNT] : 0ull;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (tid + j * kSelNT < cnt) lds[tid + j * kSelNT] = cv[j];
  }
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
  w.skinny = M <= kSkRows;
  w.small = !w.skinny && M <= kSmallM;
  int BN;
  if (w.skinny) {
    // one workgroup per CU (256 on MI355X), more when a wave would need more
    // than kSkNB blocks; partials per row: one per wave
    const int nblk = (V + 15) / 16;
    const int by_cu = std::min(kSkCUs, (nblk + kSkWaves - 1) / kSkWaves);
    const int by_nb = (nblk + kSkWaves * kSkNB - 1) / (kSkWaves * kSkNB);
    w.nwg = std::max(by_cu, by_nb);
    BN = 16;
    w.gpt = 4;
    w.wgn = 1;
    w.T = w.nwg;  // partials per row: one per workgroup
    w.S = std::min(nblk, kSkSampleBlocks);
  } else {
    BN = w.small ? TileShape<4>::BN : TileShape<2>::BN;
    w.gpt = w.small ? TileShape<4>::GPT : TileShape<2>::GPT;
    w.wgn = w.small ? TileShape<4>::WGN : TileShape<2>::WGN;
    w.T = (V + BN - 1) / BN;
    w.S = w.T < kSampleCols / BN ? w.T : kSampleCols / BN;
  }
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
  w.off_count = take((size_t)M * kCountStride * sizeof(int));
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
  if (wsl.skinny) {
    auto* sk_sample = &lmh_skinny_kernel<true, 1, kSkSampleWaves>;
    auto* sk_main = &lmh_skinny_kernel<false, kSkNB, kSkWaves>;
    constexpr size_t lds_sample = SkRing<1, kSkSampleWaves>::lds, lds_main = SkRing<kSkNB, kSkWaves>::lds;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sk_sample),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_sample);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(sk_main), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_main);
    if (e != hipSuccess) return e;
    const int swg = (a.S + kSkSampleWaves - 1) / kSkSampleWaves;
    hipLaunchKernelGGL(sk_sample, dim3(swg), dim3(kSkSampleWaves * kWave), lds_sample, stream, a, a.S,
                       swg * kSkSampleWaves);
    hipLaunchKernelGGL(lmh_threshold_kernel, dim3(M), dim3(kThrNT), 0, stream, a, k);
    const int nblk = (V + 15) / 16;
    hipLaunchKernelGGL(sk_main, dim3(wsl.nwg), dim3(kSkWaves * kWave), lds_main, stream, a, nblk,
                       wsl.nwg * kSkWaves);
  } else if (wsl.small) {
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
