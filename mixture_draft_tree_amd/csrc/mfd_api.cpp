// C ABI of libmfdtree: argument checks, workspace sizes, error text, launches.
// Every check happens before any HIP call, so a rejected call launches nothing
// and touches no device state.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mfdtree.h"
#include "mfd_launch.hpp"

namespace {

thread_local char g_err[512] = "";

mfd_status fail(mfd_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mfd_status ok() {
  g_err[0] = 0;
  return MFD_OK;
}

mfd_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MFD_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxLmhD = 16384;
constexpr int kMaxK = 32, kMaxL = 32, kMaxV = (1 << 20) - 1, kMaxB = 16383, kMaxTopk = 2048, kMaxKk = 16384;

mfd_status check_dims(int N, int K, int L, int V) {
  if (N < 0) return fail(MFD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
  if (K < 1 || K > kMaxK) return fail(MFD_ERR_INVALID_ARG, "K must be in [1, %d] (got %d)", kMaxK, K);
  if (L < 1 || L > kMaxL) return fail(MFD_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", kMaxL, L);
  if (V < 1 || V > kMaxV) return fail(MFD_ERR_INVALID_ARG, "V must be in [1, %d] (got %d)", kMaxV, V);
  return MFD_OK;
}

mfd_status check_tree_dims(int N, int K, int L, int k, int B) {
  if (N < 0) return fail(MFD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
  if (K < 1 || K > kMaxK) return fail(MFD_ERR_INVALID_ARG, "K must be in [1, %d] (got %d)", kMaxK, K);
  if (L < 1 || L > kMaxL) return fail(MFD_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", kMaxL, L);
  if (B < 0 || B > kMaxB) return fail(MFD_ERR_INVALID_ARG, "B must be in [0, %d] (got %d)", kMaxB, B);
  if (k < 1 || k > kMaxTopk) return fail(MFD_ERR_INVALID_ARG, "k must be in [1, %d] (got %d)", kMaxTopk, k);
  if ((long long)K * k > kMaxKk) return fail(MFD_ERR_INVALID_ARG, "K*k must be <= %d (got %lld)", kMaxKk, (long long)K * k);
  return MFD_OK;
}

#define REQUIRE_PTR(p)                                                        \
  do {                                                                        \
    if ((p) == nullptr) return fail(MFD_ERR_INVALID_ARG, "%s is NULL", #p); \
  } while (0)

}  // namespace

extern "C" {

const char* mfd_last_error(void) { return g_err; }

const char* mfd_version(void) { return "libmfdtree 0.1 (gfx950)"; }

mfd_status mfd_workspace_size(mfd_op op, int N, int K, int L, int V, int B, size_t* bytes) {
  REQUIRE_PTR(bytes);
  *bytes = 0;
  switch (op) {
    case MFD_OP_LOGSOFTMAX_TOPK:
    case MFD_OP_TREE_MASK:
      if (N < 0) return fail(MFD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
      return ok();
    case MFD_OP_VERIFY_WALK:
      if (N < 0) return fail(MFD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
      // L outside [1, kMaxL] sizes for the longest walk
      *bytes = N == 0 ? 0
                      : mfd::walk_ws_bytes_full(N, L < 1 || L > kMaxL ? kMaxL : L, B < 0 || B > kMaxB ? 0 : B + 1,
                                                V < 1 || V > kMaxV ? 0 : V);
      return ok();
    case MFD_OP_COVERED_MASS:
      if (N < 0) return fail(MFD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
      if (B < 0 || B > kMaxB) return fail(MFD_ERR_INVALID_ARG, "B must be in [0, %d] (got %d)", kMaxB, B);
      *bytes = N == 0 ? 0 : mfd::covered_mass_ws_bytes(N, B + 1);
      return ok();
    case MFD_OP_LMHEAD_TOPK: {
      mfd_status s = check_dims(N, K, L, V);
      if (s != MFD_OK) return s;
      if (B < 0 || B > kMaxB) return fail(MFD_ERR_INVALID_ARG, "B must be in [0, %d] (got %d)", kMaxB, B);
      const int k = B < V ? (B < 1 ? 1 : B) : V;
      if (k > kMaxTopk) return fail(MFD_ERR_INVALID_ARG, "k = min(B, V) must be <= %d (got %d)", kMaxTopk, k);
      const long long M = (long long)N * K * L;
      *bytes = M == 0 ? 0 : mfd::lmhead_workspace(M, V, k).bytes;
      return ok();
    }
    case MFD_OP_MIXTURE_THRESHOLD:
    case MFD_OP_TREE_BUILD:
    case MFD_OP_MIXTURE_TREE: {
      mfd_status s = check_dims(N, K, L, V);
      if (s != MFD_OK) return s;
      if (B < 0 || B > kMaxB) return fail(MFD_ERR_INVALID_ARG, "B must be in [0, %d] (got %d)", kMaxB, B);
      const int k = B < V ? (B < 1 ? 1 : B) : V;
      s = check_tree_dims(N, K, L, k, B);
      if (s != MFD_OK) return s;
      *bytes = (size_t)N * mfd::tree_caps(K, L, k, B).ws_bytes_per_tree;
      return ok();
    }
  }
  return fail(MFD_ERR_INVALID_ARG, "unknown op %d", (int)op);
}

static mfd_status logsoftmax_topk_impl(const char* call, const void* logits, mfd_dtype dtype, int N, int K, int L,
                                       int V, const int32_t* vocab_map, const int32_t* modes, int k, double* lse,
                                       int32_t* topk_id, float* topk_raw, float* topk_logp, int32_t* status,
                                       hipStream_t stream) {
  mfd_status s = check_dims(N, K, L, V);
  if (s != MFD_OK) return s;
  if (dtype != MFD_BF16 && dtype != MFD_F32) return fail(MFD_ERR_DTYPE, "dtype must be MFD_BF16 or MFD_F32");
  if (k < 1 || k > kMaxTopk || k > V) return fail(MFD_ERR_INVALID_ARG, "k must be in [1, min(V, %d)] (got %d)", kMaxTopk, k);
  if (N == 0) return ok();
  REQUIRE_PTR(logits);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(topk_id);
  REQUIRE_PTR(topk_raw);
  const size_t esz = dtype == MFD_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(logits) % esz) return fail(MFD_ERR_INVALID_ARG, "logits not aligned to its element size");
  const long long rows = (long long)N * K * L;
  if (rows > 0x7FFFFFFFLL) return fail(MFD_ERR_INVALID_ARG, "too many rows (%lld)", rows);
  return from_hip(mfd::launch_logsoftmax_topk(logits, dtype == MFD_BF16, (int)rows, K * L, L, V, k, vocab_map, modes,
                                              lse, topk_id, topk_raw, topk_logp, status, stream),
                  call);
}

mfd_status mfd_logsoftmax_topk(const void* logits, mfd_dtype dtype, int N, int K, int L, int V, int k, double* lse,
                               int32_t* topk_id, float* topk_raw, float* topk_logp, int32_t* status, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return logsoftmax_topk_impl("mfd_logsoftmax_topk launch", logits, dtype, N, K, L, V, nullptr, nullptr, k, lse,
                              topk_id, topk_raw, topk_logp, status, stream);
}

mfd_status mfd_logsoftmax_topk_mapped(const void* logits, mfd_dtype dtype, int N, int K, int L, int V,
                                      const int32_t* vocab_map, int V_full, int k, double* lse, int32_t* topk_id,
                                      float* topk_raw, float* topk_logp, int32_t* status, hipStream_t stream) {
  if (V_full < V || V_full > kMaxV)
    return fail(MFD_ERR_INVALID_ARG, "V_full must be in [V, %d] (got %d, V = %d)", kMaxV, V_full, V);
  if (N > 0) REQUIRE_PTR(vocab_map);
  return logsoftmax_topk_impl("mfd_logsoftmax_topk_mapped launch", logits, dtype, N, K, L, V, vocab_map, nullptr, k,
                              lse, topk_id, topk_raw, topk_logp, status, stream);
}

mfd_status mfd_logsoftmax_topk_modes(const void* logits, mfd_dtype dtype, int N, int K, int L, int V,
                                     const int32_t* modes, int k, double* lse, int32_t* topk_id, float* topk_raw,
                                     float* topk_logp, int32_t* status, hipStream_t stream) {
  if (N > 0) REQUIRE_PTR(modes);
  return logsoftmax_topk_impl("mfd_logsoftmax_topk_modes launch", logits, dtype, N, K, L, V, nullptr, modes, k, lse,
                              topk_id, topk_raw, topk_logp, status, stream);
}

static mfd_status check_head(int V, int D) {
  if (V < 1 || V > kMaxV) return fail(MFD_ERR_INVALID_ARG, "V must be in [1, %d] (got %d)", kMaxV, V);
  if (D < 64 || D > kMaxLmhD || D % 64 != 0)
    return fail(MFD_ERR_INVALID_ARG, "D must be a multiple of 64 in [64, %d] (got %d)", kMaxLmhD, D);
  if ((long long)((V + 255) / 256) * 256 * D > 0x7FFFFFFFLL)
    return fail(MFD_ERR_INVALID_ARG, "V*D must be < 2^31 (got %lld)", (long long)V * D);
  return MFD_OK;
}

mfd_status mfd_lmhead_packed_size(int V, int D, size_t* bytes) {
  REQUIRE_PTR(bytes);
  mfd_status s = check_head(V, D);
  if (s != MFD_OK) return s;
  *bytes = mfd::lmhead_packed_bytes(V, D);
  return ok();
}

mfd_status mfd_lmhead_pack_weight(const void* weight, int V, int D, void* packed, size_t packed_bytes,
                                  hipStream_t stream) {
  mfd_status s = check_head(V, D);
  if (s != MFD_OK) return s;
  REQUIRE_PTR(weight);
  REQUIRE_PTR(packed);
  if (reinterpret_cast<uintptr_t>(weight) % 16 || reinterpret_cast<uintptr_t>(packed) % 16)
    return fail(MFD_ERR_INVALID_ARG, "weight and packed must be 16-byte aligned");
  const size_t need = mfd::lmhead_packed_bytes(V, D);
  if (packed_bytes < need) return fail(MFD_ERR_INVALID_ARG, "packed needs %zu bytes (got %zu)", need, packed_bytes);
  return from_hip(mfd::launch_lmhead_pack(weight, V, D, packed, stream), "mfd_lmhead_pack_weight launch");
}

static mfd_status lmhead_impl(const char* call, const void* hidden, const void* weight, mfd_head_layout layout,
                              const int32_t* vocab_map, int N, int K, int L, int D, int V, int k, double* lse,
                              int32_t* topk_id, float* topk_raw, float* topk_logp, int32_t* status, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  mfd_status s = check_dims(N, K, L, V);
  if (s != MFD_OK) return s;
  if (layout != MFD_HEAD_ROWS && layout != MFD_HEAD_PACKED)
    return fail(MFD_ERR_INVALID_ARG, "layout must be MFD_HEAD_ROWS or MFD_HEAD_PACKED (got %d)", (int)layout);
  if (D < 64 || D > kMaxLmhD || D % 64 != 0)
    return fail(MFD_ERR_INVALID_ARG, "D must be a multiple of 64 in [64, %d] (got %d)", kMaxLmhD, D);
  if (k < 1 || k > kMaxTopk || k > V) return fail(MFD_ERR_INVALID_ARG, "k must be in [1, min(V, %d)] (got %d)", kMaxTopk, k);
  const long long M = (long long)N * K * L;
  if (M * D > 0x7FFFFFFFLL) return fail(MFD_ERR_INVALID_ARG, "N*K*L*D must be < 2^31 (got %lld)", M * D);
  if ((long long)((V + 255) / 256) * 256 * D > 0x7FFFFFFFLL)
    return fail(MFD_ERR_INVALID_ARG, "V*D must be < 2^31 (got %lld)", (long long)V * D);
  if (N == 0) return ok();
  REQUIRE_PTR(hidden);
  REQUIRE_PTR(weight);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(topk_id);
  REQUIRE_PTR(topk_raw);
  if (reinterpret_cast<uintptr_t>(hidden) % 16 || reinterpret_cast<uintptr_t>(weight) % 16)
    return fail(MFD_ERR_INVALID_ARG, "hidden and weight must be 16-byte aligned");
  const size_t need = mfd::lmhead_workspace(M, V, k).bytes;
  if (ws == nullptr || ws_bytes < need)
    return fail(MFD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws == nullptr ? (size_t)0 : ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MFD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return from_hip(mfd::launch_lmhead_topk(hidden, weight, layout == MFD_HEAD_PACKED, vocab_map, (int)M, K * L, D, V,
                                          k, lse, topk_id, topk_raw, topk_logp, status, ws, stream),
                  call);
}

mfd_status mfd_lmhead_logsoftmax_topk(const void* hidden, const void* weight, mfd_head_layout layout, int N, int K,
                                      int L, int D, int V, int k, double* lse, int32_t* topk_id, float* topk_raw,
                                      float* topk_logp, int32_t* status, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  return lmhead_impl("mfd_lmhead_logsoftmax_topk launch", hidden, weight, layout, nullptr, N, K, L, D, V, k, lse,
                     topk_id, topk_raw, topk_logp, status, ws, ws_bytes, stream);
}

mfd_status mfd_lmhead_logsoftmax_topk_mapped(const void* hidden, const void* weight, mfd_head_layout layout,
                                             const int32_t* vocab_map, int V_full, int N, int K, int L, int D, int V,
                                             int k, double* lse, int32_t* topk_id, float* topk_raw,
                                             float* topk_logp, int32_t* status, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
  if (V_full < V || V_full > kMaxV)
    return fail(MFD_ERR_INVALID_ARG, "V_full must be in [V, %d] (got %d, V = %d)", kMaxV, V_full, V);
  if (N > 0) REQUIRE_PTR(vocab_map);
  return lmhead_impl("mfd_lmhead_logsoftmax_topk_mapped launch", hidden, weight, layout, vocab_map, N, K, L, D, V, k,
                     lse, topk_id, topk_raw, topk_logp, status, ws, ws_bytes, stream);
}

static mfd_status mixture_threshold_impl(const char* call, const int32_t* topk_id, const float* topk_raw,
                                         const double* lse, int N, int K, int L, int k, int B, const int32_t* modes,
                                         double* cutoff, int32_t* n_select, int32_t* per_mode_kept, int32_t* status,
                                         void* ws, size_t ws_bytes, hipStream_t stream) {
  mfd_status s = check_tree_dims(N, K, L, k, B);
  if (s != MFD_OK) return s;
  if (N == 0) return ok();
  REQUIRE_PTR(topk_id);
  REQUIRE_PTR(topk_raw);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(cutoff);
  REQUIRE_PTR(n_select);
  const size_t need = (size_t)N * mfd::tree_caps(K, L, k, B).ws_bytes_per_tree;
  if (ws == nullptr || ws_bytes < need)
    return fail(MFD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws == nullptr ? (size_t)0 : ws_bytes);
  return from_hip(mfd::launch_mixture_threshold(topk_id, topk_raw, lse, N, K, L, k, B, modes, cutoff, n_select,
                                                per_mode_kept, status, ws, stream),
                  call);
}

mfd_status mfd_mixture_threshold(const int32_t* topk_id, const float* topk_raw, const double* lse, int N, int K, int L,
                                 int k, int B, double* cutoff, int32_t* n_select, int32_t* per_mode_kept,
                                 int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream) {
  return mixture_threshold_impl("mfd_mixture_threshold launch", topk_id, topk_raw, lse, N, K, L, k, B, nullptr, cutoff,
                                n_select, per_mode_kept, status, ws, ws_bytes, stream);
}

mfd_status mfd_mixture_threshold_modes(const int32_t* topk_id, const float* topk_raw, const double* lse, int N, int K,
                                       int L, int k, int B, const int32_t* modes, double* cutoff, int32_t* n_select,
                                       int32_t* per_mode_kept, int32_t* status, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  if (N > 0) REQUIRE_PTR(modes);
  return mixture_threshold_impl("mfd_mixture_threshold_modes launch", topk_id, topk_raw, lse, N, K, L, k, B, modes,
                                cutoff, n_select, per_mode_kept, status, ws, ws_bytes, stream);
}

static mfd_status tree_build_impl(const char* call, const int32_t* topk_id, const float* topk_raw, const double* lse,
                                  const double* cutoff, const int32_t* n_select, const int32_t* anchor_token, int N,
                                  int K, int L, int k, int B, const int32_t* modes, int32_t* node_token,
                                  int32_t* parent, int32_t* depth, double* score, int32_t* best_mode,
                                  int32_t* n_nodes, int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream) {
  mfd_status s = check_tree_dims(N, K, L, k, B);
  if (s != MFD_OK) return s;
  if (N == 0) return ok();
  REQUIRE_PTR(topk_id);
  REQUIRE_PTR(topk_raw);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(cutoff);
  REQUIRE_PTR(n_select);
  REQUIRE_PTR(anchor_token);
  REQUIRE_PTR(node_token);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(score);
  REQUIRE_PTR(best_mode);
  REQUIRE_PTR(n_nodes);
  const size_t need = (size_t)N * mfd::tree_caps(K, L, k, B).ws_bytes_per_tree;
  if (ws == nullptr || ws_bytes < need)
    return fail(MFD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws == nullptr ? (size_t)0 : ws_bytes);
  return from_hip(mfd::launch_tree_build(topk_id, topk_raw, lse, cutoff, n_select, anchor_token, N, K, L, k, B, modes,
                                         node_token, parent, depth, score, best_mode, n_nodes, status, ws, stream),
                  call);
}

mfd_status mfd_tree_build(const int32_t* topk_id, const float* topk_raw, const double* lse, const double* cutoff,
                          const int32_t* n_select, const int32_t* anchor_token, int N, int K, int L, int k, int B,
                          int32_t* node_token, int32_t* parent, int32_t* depth, double* score, int32_t* best_mode,
                          int32_t* n_nodes, int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream) {
  return tree_build_impl("mfd_tree_build launch", topk_id, topk_raw, lse, cutoff, n_select, anchor_token, N, K, L, k,
                         B, nullptr, node_token, parent, depth, score, best_mode, n_nodes, status, ws, ws_bytes,
                         stream);
}

mfd_status mfd_tree_build_modes(const int32_t* topk_id, const float* topk_raw, const double* lse, const double* cutoff,
                                const int32_t* n_select, const int32_t* anchor_token, int N, int K, int L, int k,
                                int B, const int32_t* modes, int32_t* node_token, int32_t* parent, int32_t* depth,
                                double* score, int32_t* best_mode, int32_t* n_nodes, int32_t* status, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  if (N > 0) REQUIRE_PTR(modes);
  return tree_build_impl("mfd_tree_build_modes launch", topk_id, topk_raw, lse, cutoff, n_select, anchor_token, N, K,
                         L, k, B, modes, node_token, parent, depth, score, best_mode, n_nodes, status, ws, ws_bytes,
                         stream);
}

static mfd_status mixture_tree_impl(const char* call, const int32_t* topk_id, const float* topk_raw,
                                    const double* lse, const int32_t* anchor_token, int N, int K, int L, int k, int B,
                                    const int32_t* modes, double* cutoff, int32_t* n_select, int32_t* per_mode_kept,
                                    int32_t* node_token, int32_t* parent, int32_t* depth, double* score,
                                    int32_t* best_mode, int32_t* n_nodes, int32_t* status, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  mfd_status s = check_tree_dims(N, K, L, k, B);
  if (s != MFD_OK) return s;
  if (N == 0) return ok();
  REQUIRE_PTR(topk_id);
  REQUIRE_PTR(topk_raw);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(anchor_token);
  REQUIRE_PTR(cutoff);
  REQUIRE_PTR(n_select);
  REQUIRE_PTR(node_token);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(score);
  REQUIRE_PTR(best_mode);
  REQUIRE_PTR(n_nodes);
  const size_t need = (size_t)N * mfd::tree_caps(K, L, k, B).ws_bytes_per_tree;
  if (ws == nullptr || ws_bytes < need)
    return fail(MFD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws == nullptr ? (size_t)0 : ws_bytes);
  return from_hip(mfd::launch_mixture_tree(topk_id, topk_raw, lse, anchor_token, N, K, L, k, B, modes, cutoff,
                                           n_select, per_mode_kept, node_token, parent, depth, score, best_mode,
                                           n_nodes, status, ws, stream),
                  call);
}

mfd_status mfd_mixture_tree(const int32_t* topk_id, const float* topk_raw, const double* lse,
                            const int32_t* anchor_token, int N, int K, int L, int k, int B, double* cutoff,
                            int32_t* n_select, int32_t* per_mode_kept, int32_t* node_token, int32_t* parent,
                            int32_t* depth, double* score, int32_t* best_mode, int32_t* n_nodes, int32_t* status,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  return mixture_tree_impl("mfd_mixture_tree launch", topk_id, topk_raw, lse, anchor_token, N, K, L, k, B, nullptr,
                           cutoff, n_select, per_mode_kept, node_token, parent, depth, score, best_mode, n_nodes,
                           status, ws, ws_bytes, stream);
}

mfd_status mfd_mixture_tree_modes(const int32_t* topk_id, const float* topk_raw, const double* lse,
                                  const int32_t* anchor_token, int N, int K, int L, int k, int B,
                                  const int32_t* modes, double* cutoff, int32_t* n_select, int32_t* per_mode_kept,
                                  int32_t* node_token, int32_t* parent, int32_t* depth, double* score,
                                  int32_t* best_mode, int32_t* n_nodes, int32_t* status, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (N > 0) REQUIRE_PTR(modes);
  return mixture_tree_impl("mfd_mixture_tree_modes launch", topk_id, topk_raw, lse, anchor_token, N, K, L, k, B,
                           modes, cutoff, n_select, per_mode_kept, node_token, parent, depth, score, best_mode,
                           n_nodes, status, ws, ws_bytes, stream);
}

mfd_status mfd_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* n_nodes, const int64_t* pos_base,
                         int N, int Bp1, uint64_t* mask_words, int64_t* position_ids, uint8_t* dense_mask,
                         hipStream_t stream) {
  if (N < 0) return fail(MFD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
  if (Bp1 < 1 || Bp1 > kMaxB + 1) return fail(MFD_ERR_INVALID_ARG, "Bp1 must be in [1, %d] (got %d)", kMaxB + 1, Bp1);
  if (N == 0) return ok();
  REQUIRE_PTR(parent);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(n_nodes);
  REQUIRE_PTR(pos_base);
  REQUIRE_PTR(mask_words);
  REQUIRE_PTR(position_ids);
  return from_hip(
      mfd::launch_tree_mask(parent, depth, n_nodes, pos_base, N, Bp1, mask_words, position_ids, dense_mask, stream),
      "mfd_tree_mask launch");
}

static mfd_status verify_walk_checks(const void* target_logits, mfd_dtype dtype, int N, int Bp1, int V, int L,
                                     const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                                     const int32_t* n_nodes, const float* temperature, const uint64_t* seed,
                                     int32_t* tau, int32_t* out_tokens, int32_t* path_nodes) {
  if (N < 0) return fail(MFD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
  if (Bp1 < 1 || Bp1 > kMaxB + 1) return fail(MFD_ERR_INVALID_ARG, "Bp1 must be in [1, %d] (got %d)", kMaxB + 1, Bp1);
  if (V < 1 || V > kMaxV) return fail(MFD_ERR_INVALID_ARG, "V must be in [1, %d] (got %d)", kMaxV, V);
  if (L < 1 || L > kMaxL) return fail(MFD_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", kMaxL, L);
  if (dtype != MFD_BF16 && dtype != MFD_F32) return fail(MFD_ERR_DTYPE, "dtype must be MFD_BF16 or MFD_F32");
  if (N == 0) return ok();
  REQUIRE_PTR(target_logits);
  REQUIRE_PTR(node_token);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(n_nodes);
  REQUIRE_PTR(temperature);
  REQUIRE_PTR(seed);
  REQUIRE_PTR(tau);
  REQUIRE_PTR(out_tokens);
  REQUIRE_PTR(path_nodes);
  const size_t esz = dtype == MFD_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(target_logits) % esz)
    return fail(MFD_ERR_INVALID_ARG, "target_logits not aligned to its element size");
  return MFD_OK;
}

mfd_status mfd_verify_walk(const void* target_logits, mfd_dtype dtype, int N, int Bp1, int V, int L,
                           const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                           const int32_t* n_nodes, const float* temperature, const uint64_t* seed, int32_t* tau,
                           int32_t* out_tokens, int32_t* path_nodes, int32_t* status, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  mfd_status s = verify_walk_checks(target_logits, dtype, N, Bp1, V, L, node_token, parent, depth, n_nodes,
                                    temperature, seed, tau, out_tokens, path_nodes);
  if (s != MFD_OK || N == 0) return s == MFD_OK ? ok() : s;
  const size_t need = mfd::walk_ws_bytes(N, L);
  if (ws == nullptr || ws_bytes < need)
    return fail(MFD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws == nullptr ? (size_t)0 : ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 8) return fail(MFD_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  return from_hip(mfd::launch_verify_walk(target_logits, dtype == MFD_BF16, N, Bp1, V, L, node_token, parent, depth,
                                          n_nodes, temperature, seed, tau, out_tokens, path_nodes, status, ws, ws_bytes,
                                          stream),
                  "mfd_verify_walk launch");
}

static int walk_noalloc_max_trees(int L) {
  int lo = 0, hi = 1 << 20;  // the largest N whose workspace fits the built-in scratch
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (mfd::walk_ws_bytes(mid, L) <= mfd::walk_scratch_bytes()) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

mfd_status mfd_verify_walk_noalloc(const void* target_logits, mfd_dtype dtype, int N, int Bp1, int V, int L,
                                   const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                                   const int32_t* n_nodes, const float* temperature, const uint64_t* seed,
                                   int32_t* tau, int32_t* out_tokens, int32_t* path_nodes, int32_t* status,
                                   hipStream_t stream) {
  mfd_status s = verify_walk_checks(target_logits, dtype, N, Bp1, V, L, node_token, parent, depth, n_nodes,
                                    temperature, seed, tau, out_tokens, path_nodes);
  if (s != MFD_OK || N == 0) return s == MFD_OK ? ok() : s;
  const size_t need = mfd::walk_ws_bytes(N, L);
  if (need > mfd::walk_scratch_bytes())
    return fail(MFD_ERR_WORKSPACE, "N = %d trees need %zu bytes of walk workspace; the built-in one holds %zu (N <= %d)",
                N, need, mfd::walk_scratch_bytes(), walk_noalloc_max_trees(L));
  void* ws = nullptr;
  mfd_status r = from_hip(mfd::walk_scratch(&ws), "mfd_verify_walk_noalloc scratch lookup");
  if (r != MFD_OK) return r;
  return from_hip(mfd::launch_verify_walk(target_logits, dtype == MFD_BF16, N, Bp1, V, L, node_token, parent, depth,
                                          n_nodes, temperature, seed, tau, out_tokens, path_nodes, status, ws,
                                          mfd::walk_scratch_bytes(), stream),
                  "mfd_verify_walk_noalloc launch");
}

mfd_status mfd_covered_mass(const void* target_logits, mfd_dtype dtype, int N, int Bp1, int V,
                            const int32_t* node_token, const int32_t* parent, const int32_t* n_nodes,
                            const float* temperature, double* mass, int32_t* status, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (N < 0 || N > 65535) return fail(MFD_ERR_INVALID_ARG, "N must be in [0, 65535] (got %d)", N);
  if (Bp1 < 1 || Bp1 > kMaxB + 1) return fail(MFD_ERR_INVALID_ARG, "Bp1 must be in [1, %d] (got %d)", kMaxB + 1, Bp1);
  if (V < 1 || V > kMaxV) return fail(MFD_ERR_INVALID_ARG, "V must be in [1, %d] (got %d)", kMaxV, V);
  if (dtype != MFD_BF16 && dtype != MFD_F32) return fail(MFD_ERR_DTYPE, "dtype must be MFD_BF16 or MFD_F32");
  if (N == 0) return ok();
  REQUIRE_PTR(target_logits);
  REQUIRE_PTR(node_token);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(n_nodes);
  REQUIRE_PTR(temperature);
  REQUIRE_PTR(mass);
  const size_t esz = dtype == MFD_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(target_logits) % esz)
    return fail(MFD_ERR_INVALID_ARG, "target_logits not aligned to its element size");
  const size_t need = mfd::covered_mass_ws_bytes(N, Bp1);
  if (ws == nullptr || ws_bytes < need)
    return fail(MFD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws == nullptr ? (size_t)0 : ws_bytes);
  return from_hip(mfd::launch_covered_mass(target_logits, dtype == MFD_BF16, N, Bp1, V, node_token, parent, n_nodes,
                                           temperature, mass, status, ws, stream),
                  "mfd_covered_mass launch");
}

mfd_status mfd_chimera_count(const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                             const int32_t* n_nodes, int N, int Bp1, int L, const int32_t* future_a,
                             const int32_t* future_b, int32_t* count, hipStream_t stream) {
  if (N < 0) return fail(MFD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
  if (Bp1 < 1 || Bp1 > kMaxB + 1) return fail(MFD_ERR_INVALID_ARG, "Bp1 must be in [1, %d] (got %d)", kMaxB + 1, Bp1);
  if (L < 1 || L > kMaxL) return fail(MFD_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", kMaxL, L);
  if (N == 0) return ok();
  REQUIRE_PTR(node_token);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(n_nodes);
  REQUIRE_PTR(future_a);
  REQUIRE_PTR(future_b);
  REQUIRE_PTR(count);
  return from_hip(mfd::launch_chimera_count(node_token, parent, depth, n_nodes, N, Bp1, L, future_a, future_b, count,
                                            stream),
                  "mfd_chimera_count launch");
}

mfd_status mfd_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes % 16) return fail(MFD_ERR_INVALID_ARG, "bytes must be a multiple of 16 (got %zu)", bytes);
  if (bytes == 0) return ok();
  REQUIRE_PTR(buf);
  REQUIRE_PTR(sink);
  if (reinterpret_cast<uintptr_t>(buf) % 16) return fail(MFD_ERR_INVALID_ARG, "buf is not 16-byte aligned");
  return from_hip(mfd::launch_stream_read(buf, bytes, sink, stream), "mfd_stream_read launch");
}

}  // extern "C"
