// Host-side launchers of the libmfdtree kernels (one per C-ABI call).  The
// C-ABI layer validates arguments, then calls these; they only size LDS and
// grids and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mfdtree.h"

namespace mfd {

// modes (device [N] or null): rows of mode m >= modes[n] are skipped
hipError_t launch_logsoftmax_topk(const void* logits, bool bf16, int rows, int rows_per_tree, int L, long long V,
                                  int k, const int32_t* vocab_map, const int32_t* modes, double* lse,
                                  int32_t* topk_id, float* topk_raw, float* topk_logp, int32_t* status,
                                  hipStream_t stream);

// Working capacities of the tree search for one tree (shared by the threshold
// and build calls, and by the workspace query).
struct TreeCaps {
  int sort_cap;   // children of one level that fit the LDS sort (power of two)
  int ent_cap;    // per-mode entries over all levels
  int node_cap;   // unique prefixes over all levels
  size_t ws_bytes_per_tree;
  size_t lds_bytes;
};
TreeCaps tree_caps(int K, int L, int k, int B);

// modes (device [N] or null): tree n uses its first clamp(modes[n], 1, K) modes
hipError_t launch_mixture_threshold(const int32_t* topk_id, const float* topk_raw, const double* lse, int N, int K,
                                    int L, int k, int B, const int32_t* modes, double* cutoff, int32_t* n_select,
                                    int32_t* per_mode_kept, int32_t* status, void* ws, hipStream_t stream);

hipError_t launch_tree_build(const int32_t* topk_id, const float* topk_raw, const double* lse, const double* cutoff,
                             const int32_t* n_select, const int32_t* anchor, int N, int K, int L, int k, int B,
                             const int32_t* modes, int32_t* node_token, int32_t* parent, int32_t* depth,
                             double* score, int32_t* best_mode, int32_t* n_nodes, int32_t* status, void* ws,
                             hipStream_t stream);

// The cut-off and the tree from one search (threshold and build outputs both)
hipError_t launch_mixture_tree(const int32_t* topk_id, const float* topk_raw, const double* lse, const int32_t* anchor,
                               int N, int K, int L, int k, int B, const int32_t* modes, double* cutoff,
                               int32_t* n_select, int32_t* per_mode_kept, int32_t* node_token, int32_t* parent,
                               int32_t* depth, double* score, int32_t* best_mode, int32_t* n_nodes, int32_t* status,
                               void* ws, hipStream_t stream);

hipError_t launch_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* n_nodes,
                            const int64_t* pos_base, int N, int Bp1, uint64_t* mask_words, int64_t* position_ids,
                            uint8_t* dense_mask, hipStream_t stream);

size_t walk_ws_bytes(int N, int L);
// With the speculative pass (N trees of Bp1 nodes over rows of V elements):
// the workspace size mfd_workspace_size reports.
size_t walk_ws_bytes_full(int N, int L, int Bp1, long long V);
// The walk's built-in workspace (mfd_verify_walk_noalloc): its size, and its
// device address on the current device (looked up once per device).
size_t walk_scratch_bytes();
hipError_t walk_scratch(void** out);

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

size_t covered_mass_ws_bytes(int N, int Bp1);
hipError_t launch_covered_mass(const void* target, bool bf16, int N, int Bp1, long long V,
                               const int32_t* node_token, const int32_t* parent, const int32_t* n_nodes,
                               const float* temperature, double* mass, int32_t* status, void* ws,
                               hipStream_t stream);
hipError_t launch_chimera_count(const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                                const int32_t* n_nodes, int N, int Bp1, int L, const int32_t* future_a,
                                const int32_t* future_b, int32_t* count, hipStream_t stream);

hipError_t launch_verify_walk(const void* target, bool bf16, int N, int Bp1, long long V, int L,
                              const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                              const int32_t* n_nodes, const float* temperature, const uint64_t* seed, int32_t* tau,
                              int32_t* out_tokens, int32_t* path_nodes, int32_t* status, void* ws, size_t ws_bytes,
                              hipStream_t stream);


// Fused LM head + log-softmax/top-k: workspace layout (byte offsets into the
// caller's buffer) and launcher.
struct LmhWorkspace {
  bool skinny;  // at most 128 rows: head streamed into registers, one workgroup per CU
  int nwg;      // skinny: workgroups of the main launch
  bool small;   // 128-column tiles (up to 256 rows) instead of 256-column ones
  int gpt;     // groups of 4 columns per tile
  int wgn;     // partials per row and tile
  int T;       // vocabulary tiles
  int S;       // tiles in the threshold sample
  int C;       // candidate capacity per row
  size_t off_samp, off_thr, off_count, off_part, off_cand, bytes;
};
LmhWorkspace lmhead_workspace(long long M, int V, int k);
// vocab_map (device [V] or null): topk_id reports vocab_map[column];
// packed: weight in the layout written by launch_lmhead_pack
size_t lmhead_packed_bytes(int V, int D);
hipError_t launch_lmhead_pack(const void* weight, int V, int D, void* packed, hipStream_t stream);
hipError_t launch_lmhead_topk(const void* hidden, const void* weight, bool packed, const int32_t* vocab_map, int M,
                              int rows_per_tree, int D, int V, int k, double* lse, int32_t* topk_id, float* topk_raw,
                              float* topk_logp, int32_t* status, void* ws, hipStream_t stream);

}  // namespace mfd
