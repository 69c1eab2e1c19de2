// Tree-verification inputs: ancestor-or-self bitmask and position ids.
//
// The target verifies the whole tree in one pass with standard tree
// verification (MFD-Qwen3.5-4B model card, summary paragraph): node i may
// attend to itself and to its ancestors, and sits at position pos_base +
// depth(i).
//
// One wavefront per mask row.  Lane d holds the ancestor of row i at depth d
// (a walk up the parent chain, at most L steps).  For a 64-column word, lane l
// tests column j = 64w + l: j is an ancestor-or-self of i exactly when
// depth(j) <= depth(i) and the ancestor of i at depth(j) is j, which is one
// cross-lane read (ds_bpermute) of the chain.  A ballot turns the 64 answers
// into the mask word; lane w keeps word w so each row is stored with one
// coalesced write.
#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

constexpr int kMaskThreads = 1024;
constexpr int kRowsPerBlock = kMaskThreads / kWave;

__global__ void __launch_bounds__(kMaskThreads)
    tree_mask_kernel(const int32_t* __restrict__ parent, const int32_t* __restrict__ depth,
                     const int32_t* __restrict__ n_nodes, const int64_t* __restrict__ pos_base, int Bp1, int W,
                     uint64_t* __restrict__ mask_words, int64_t* __restrict__ position_ids,
                     uint8_t* __restrict__ dense_mask) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  int16_t* sp = reinterpret_cast<int16_t*>(smem_raw);       // parent (Bp1 <= 16384)
  int8_t* sd = reinterpret_cast<int8_t*>(sp + Bp1);          // depth (<= 32)
  const int n = blockIdx.x;
  int nn = n_nodes[n];
  nn = nn < 0 ? 0 : (nn > Bp1 ? Bp1 : nn);
  const size_t tb = (size_t)n * Bp1;
  for (int j = threadIdx.x; j < Bp1; j += kMaskThreads) {
    sp[j] = (int16_t)(j < nn ? parent[tb + j] : -1);
    sd[j] = (int8_t)(j < nn ? depth[tb + j] : 127);
  }
  __syncthreads();

  const int lane = lane_id();
  const int i = blockIdx.y * kRowsPerBlock + wave_id();
  if (i >= Bp1) return;
  uint64_t* out = mask_words + (tb + i) * (size_t)W;
  uint8_t* dout = dense_mask ? dense_mask + (tb + i) * (size_t)Bp1 : nullptr;
  if (i >= nn) {
    for (int w = lane; w < W; w += kWave) out[w] = 0ull;
    if (dout)
      for (int j = lane; j < Bp1; j += kWave) dout[j] = 0;
    if (lane == 0) position_ids[tb + i] = -1;
    return;
  }
  const int di = sd[i];
  int chain = -1;
  {
    int a = i;
    for (int d = di; d >= 0 && a >= 0 && a < Bp1; --d) {
      if (lane == d) chain = a;
      a = sp[a];
    }
  }
  for (int w0 = 0; w0 < W; w0 += kWave) {
    uint64_t mine = 0ull;
    const int wend = (W - w0 < kWave) ? W - w0 : kWave;
    for (int ww = 0; ww < wend; ++ww) {
      const int j = (w0 + ww) * kWave + lane;
      const int dj = (j < nn) ? (int)sd[j] : 127;
      const int anc = __shfl(chain, dj < kWave ? dj : 0, kWave);
      const bool take = (j < nn) && (dj <= di) && (anc == j);
      const uint64_t word = __ballot(take);
      if (lane == ww) mine = word;
      if (dout && j < Bp1) dout[j] = take ? 1 : 0;
    }
    if (lane < wend) out[w0 + lane] = mine;
  }
  if (lane == 0) position_ids[tb + i] = pos_base[n] + di;
}

}  // namespace

hipError_t launch_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* n_nodes,
                            const int64_t* pos_base, int N, int Bp1, uint64_t* mask_words, int64_t* position_ids,
                            uint8_t* dense_mask, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int W = (Bp1 + 63) / 64;
  const size_t lds = (size_t)Bp1 * 3 + 16;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&tree_mask_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(N, (Bp1 + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(tree_mask_kernel, grid, dim3(kMaskThreads), lds, stream, parent, depth, n_nodes, pos_base, Bp1,
                     W, mask_words, position_ids, dense_mask);
  return hipGetLastError();
}

}  // namespace mfd
