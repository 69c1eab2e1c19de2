/*
 * The C ABI used from plain C: no Python, no torch.  Test infrastructure.
 *
 *   abi_smoke cpu
 *       Library version, workspace sizes and argument errors (nothing is
 *       launched, no GPU needed).  Exit status 0 when every check holds.
 *   abi_smoke gpu IN OUT
 *       Reads one batch of drafter logits and target rows from IN, runs the
 *       five calls of a decoding round on the current HIP device with buffers
 *       from hipMalloc, and writes the tree, mask, position ids and walk
 *       results to OUT for the caller to compare.
 *
 * IN (little-endian): int32 N, K, L, V, B; float32 logits [N,K,L,V];
 * int32 anchor [N]; int64 pos_base [N]; float32 target [N,B+1,V];
 * float32 temperature [N]; uint64 seed [N].
 * OUT: int32 n_nodes [N]; int32 node_token, parent, depth [N,B+1];
 * uint64 mask words [N,B+1,W]; int64 position ids [N,B+1]; int32 tau [N];
 * int32 out_tokens [N,L+1]; int32 status [N].
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mfdtree.h"

static int fails = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAIL: %s (last error: %s)\n", what, mfd_last_error());
    ++fails;
  }
}

static int cpu_checks(void) {
  size_t b = 0;
  void* fake = (void*)(uintptr_t)0x100000; /* rejected before any launch: never dereferenced */
  void* odd = (void*)(uintptr_t)0x100004;  /* 4-byte aligned only */
  expect(strstr(mfd_version(), "gfx950") != NULL, "version names gfx950");

  /* workspace sizes */
  expect(mfd_workspace_size(MFD_OP_TREE_BUILD, 64, 8, 15, 151936, 256, &b) == MFD_OK && b > 0,
         "tree workspace for 64 trees");
  const size_t many = b;
  expect(mfd_workspace_size(MFD_OP_TREE_BUILD, 1, 8, 15, 151936, 256, &b) == MFD_OK && 64 * b == many,
         "tree workspace is per tree");
  expect(mfd_workspace_size(MFD_OP_MIXTURE_THRESHOLD, 64, 8, 15, 151936, 256, &b) == MFD_OK && b == many,
         "threshold and build share the tree workspace");
  expect(mfd_workspace_size(MFD_OP_LOGSOFTMAX_TOPK, 64, 8, 15, 151936, 256, &b) == MFD_OK && b == 0,
         "logits pass needs no workspace");
  expect(mfd_workspace_size(MFD_OP_TREE_MASK, 64, 8, 15, 151936, 256, &b) == MFD_OK && b == 0,
         "mask needs no workspace");
  expect(mfd_workspace_size(MFD_OP_VERIFY_WALK, 64, 8, 15, 151936, 256, &b) == MFD_OK && b > 0, "walk workspace");
  expect(mfd_workspace_size(MFD_OP_VERIFY_WALK, 0, 8, 15, 151936, 256, &b) == MFD_OK && b == 0, "no trees, no bytes");
  expect(mfd_workspace_size(MFD_OP_COVERED_MASS, 64, 0, 0, 0, 256, &b) == MFD_OK && b > 0, "covered-mass workspace");
  expect(mfd_workspace_size(MFD_OP_LMHEAD_TOPK, 1, 8, 15, 151936, 256, &b) == MFD_OK && b > 0,
         "fused LM-head workspace");
  expect(mfd_workspace_size(MFD_OP_TREE_BUILD, 1, 33, 15, 100, 8, &b) == MFD_ERR_INVALID_ARG &&
             strstr(mfd_last_error(), "K must be") != NULL,
         "K = 33 rejected with a message");
  expect(mfd_workspace_size((mfd_op)99, 1, 8, 15, 100, 8, &b) == MFD_ERR_INVALID_ARG, "unknown op rejected");
  expect(mfd_workspace_size((mfd_op)-3, 1, 8, 15, 100, 8, &b) == MFD_ERR_INVALID_ARG, "negative op rejected");
  expect(mfd_workspace_size(MFD_OP_VERIFY_WALK, -1, 8, 15, 100, 8, &b) == MFD_ERR_INVALID_ARG, "N < 0 rejected");
  expect(mfd_workspace_size(MFD_OP_TREE_BUILD, 1, 8, 15, 100, 8, NULL) == MFD_ERR_INVALID_ARG, "NULL bytes rejected");
  expect(mfd_workspace_size(MFD_OP_LMHEAD_TOPK, 1, 8, 15, 151936, 4096, &b) == MFD_ERR_INVALID_ARG,
         "fused LM head: k above 2048 rejected");
  expect(mfd_workspace_size(MFD_OP_TREE_BUILD, 1, 8, 15, 100, 8, &b) == MFD_OK && mfd_last_error()[0] == 0,
         "a successful call clears the message");

  /* logits pass */
  expect(mfd_logsoftmax_topk(fake, MFD_BF16, 1, 8, 15, 1000, 2049, fake, fake, fake, NULL, NULL, NULL, 0, 0) ==
             MFD_ERR_INVALID_ARG,
         "k > 2048 rejected");
  expect(mfd_logsoftmax_topk(fake, MFD_BF16, 1, 8, 15, 100, 101, fake, fake, fake, NULL, NULL, NULL, 0, 0) ==
             MFD_ERR_INVALID_ARG,
         "k > V rejected");
  expect(mfd_logsoftmax_topk(fake, (mfd_dtype)7, 1, 8, 15, 1000, 8, fake, fake, fake, NULL, NULL, NULL, 0, 0) ==
             MFD_ERR_DTYPE,
         "unknown dtype rejected");
  expect(mfd_logsoftmax_topk(fake, (mfd_dtype)-1, 1, 8, 15, 1000, 8, fake, fake, fake, NULL, NULL, NULL, 0, 0) ==
             MFD_ERR_DTYPE,
         "negative dtype rejected");
  expect(mfd_logsoftmax_topk(fake, MFD_BF16, 1, 8, 15, 1000, 8, NULL, fake, fake, NULL, NULL, NULL, 0, 0) ==
             MFD_ERR_INVALID_ARG,
         "NULL lse rejected");
  expect(mfd_logsoftmax_topk((void*)(uintptr_t)0x100001, MFD_BF16, 1, 8, 15, 1000, 8, fake, fake, fake, NULL, NULL,
                             NULL, 0, 0) == MFD_ERR_INVALID_ARG,
         "misaligned logits rejected");
  expect(mfd_logsoftmax_topk(fake, MFD_BF16, 1, 8, 0, 1000, 8, fake, fake, fake, NULL, NULL, NULL, 0, 0) ==
             MFD_ERR_INVALID_ARG,
         "L = 0 rejected");
  expect(mfd_logsoftmax_topk(fake, MFD_BF16, 1, 8, 15, 1 << 20, 8, fake, fake, fake, NULL, NULL, NULL, 0, 0) ==
             MFD_ERR_INVALID_ARG,
         "V = 2^20 rejected");
  expect(mfd_logsoftmax_topk(NULL, MFD_BF16, 0, 8, 15, 1000, 8, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0) == MFD_OK,
         "logits pass: N = 0 is a no-op");
  expect(mfd_logsoftmax_topk_mapped(fake, MFD_BF16, 1, 8, 15, 1000, fake, 999, 8, fake, fake, fake, NULL, NULL, 0) ==
             MFD_ERR_INVALID_ARG,
         "mapped: V_full < V rejected");
  expect(mfd_logsoftmax_topk_mapped(fake, MFD_BF16, 1, 8, 15, 1000, NULL, 2000, 8, fake, fake, fake, NULL, NULL, 0) ==
             MFD_ERR_INVALID_ARG,
         "mapped: NULL map rejected");
  expect(mfd_logsoftmax_topk_modes(fake, MFD_BF16, 1, 8, 15, 1000, NULL, 8, fake, fake, fake, NULL, NULL, 0) ==
             MFD_ERR_INVALID_ARG,
         "modes: NULL modes rejected");

  /* cut-off and tree */
  expect(mfd_mixture_threshold(fake, fake, fake, 1, 8, 15, 256, 256, fake, fake, NULL, NULL, fake, 16, 0) ==
             MFD_ERR_WORKSPACE,
         "small workspace rejected");
  expect(mfd_mixture_threshold(fake, fake, fake, 1, 8, 15, 256, 256, fake, fake, NULL, NULL, NULL, 1 << 30, 0) ==
             MFD_ERR_WORKSPACE,
         "NULL workspace rejected");
  expect(mfd_mixture_threshold(fake, fake, fake, 1, 17, 15, 1024, 1024, fake, fake, NULL, NULL, fake, 1 << 30, 0) ==
             MFD_ERR_INVALID_ARG,
         "K*k > 16384 rejected");
  expect(mfd_mixture_threshold(fake, fake, fake, 1, 8, 15, 256, 16384, fake, fake, NULL, NULL, fake, 1 << 30, 0) ==
             MFD_ERR_INVALID_ARG,
         "B > 16383 rejected");
  expect(mfd_mixture_threshold(fake, fake, fake, 1, 8, 15, 256, 256, NULL, fake, NULL, NULL, fake, 1 << 30, 0) ==
             MFD_ERR_INVALID_ARG,
         "NULL cutoff rejected");
  expect(mfd_mixture_threshold_modes(fake, fake, fake, 1, 8, 15, 256, 256, NULL, fake, fake, NULL, NULL, fake,
                                     1 << 30, 0) == MFD_ERR_INVALID_ARG,
         "threshold modes: NULL modes rejected");
  expect(mfd_tree_build(fake, fake, fake, fake, fake, fake, 1, 8, 15, 256, 256, fake, fake, fake, fake, fake, NULL,
                        NULL, fake, 1 << 30, 0) == MFD_ERR_INVALID_ARG &&
             strstr(mfd_last_error(), "n_nodes") != NULL,
         "NULL n_nodes rejected with its name");
  expect(mfd_tree_build_modes(fake, fake, fake, fake, fake, fake, 1, 8, 15, 256, 256, NULL, fake, fake, fake, fake,
                              fake, fake, NULL, fake, 1 << 30, 0) == MFD_ERR_INVALID_ARG,
         "build modes: NULL modes rejected");
  expect(mfd_tree_build(NULL, NULL, NULL, NULL, NULL, NULL, 0, 8, 15, 256, 256, NULL, NULL, NULL, NULL, NULL, NULL,
                        NULL, NULL, 0, 0) == MFD_OK,
         "build: N = 0 is a no-op");

  /* mask */
  expect(mfd_tree_mask(NULL, NULL, NULL, NULL, 0, 9, NULL, NULL, NULL, 0) == MFD_OK, "N = 0 is a no-op");
  expect(mfd_tree_mask(fake, fake, fake, fake, 1, 0, fake, fake, NULL, 0) == MFD_ERR_INVALID_ARG, "Bp1 = 0 rejected");
  expect(mfd_tree_mask(fake, fake, fake, NULL, 1, 9, fake, fake, NULL, 0) == MFD_ERR_INVALID_ARG,
         "NULL pos_base rejected");

  /* walk */
  expect(mfd_verify_walk(fake, (mfd_dtype)5, 1, 9, 16, 4, fake, fake, fake, fake, fake, fake, fake, fake, fake, NULL,
                         NULL, 0, 0) == MFD_ERR_DTYPE,
         "walk: unknown dtype rejected");
  expect(mfd_verify_walk(fake, MFD_F32, 1, 9, 16, 0, fake, fake, fake, fake, fake, fake, fake, fake, fake, NULL, NULL,
                         0, 0) == MFD_ERR_INVALID_ARG,
         "walk: L = 0 rejected");
  expect(mfd_verify_walk(fake, MFD_F32, 1, 9, 16, 4, NULL, fake, fake, fake, fake, fake, fake, fake, fake, NULL, NULL,
                         0, 0) == MFD_ERR_INVALID_ARG,
         "walk: NULL node_token rejected");
  expect(mfd_verify_walk(fake, MFD_F32, 1, 9, 16, 4, fake, fake, fake, fake, fake, fake, fake, fake, fake, NULL, NULL,
                         0, 0) == MFD_ERR_WORKSPACE,
         "walk: missing workspace rejected");
  expect(mfd_verify_walk(fake, MFD_F32, 1, 9, 16, 4, fake, fake, fake, fake, fake, fake, fake, fake, fake, NULL, odd,
                         1 << 20, 0) == MFD_ERR_INVALID_ARG,
         "walk: misaligned workspace rejected");
  /* at L = 4 the built-in 16 MiB holds the walk workspace of 1637 trees */
  expect(mfd_verify_walk_noalloc(fake, MFD_F32, 1638, 9, 16, 4, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                 NULL, 0) == MFD_ERR_WORKSPACE &&
             strstr(mfd_last_error(), "N <= 1637") != NULL,
         "walk without workspace: 1638 trees rejected with the limit");
  expect(mfd_verify_walk_noalloc(NULL, MFD_F32, 0, 9, 16, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                 NULL, 0) == MFD_OK,
         "walk without workspace: N = 0 is a no-op");

  /* diagnostics and the streaming reference */
  expect(mfd_covered_mass(fake, MFD_F32, 65536, 9, 16, fake, fake, fake, fake, fake, NULL, fake, 1 << 30, 0) ==
             MFD_ERR_INVALID_ARG,
         "covered mass: N > 65535 rejected");
  expect(mfd_covered_mass(fake, MFD_F32, 2, 9, 16, fake, fake, fake, fake, fake, NULL, NULL, 0, 0) ==
             MFD_ERR_WORKSPACE,
         "covered mass: missing workspace rejected");
  expect(mfd_chimera_count(fake, fake, fake, fake, 1, 9, 0, fake, fake, fake, 0) == MFD_ERR_INVALID_ARG,
         "chimera count: L = 0 rejected");
  expect(mfd_chimera_count(NULL, NULL, NULL, NULL, 0, 9, 4, NULL, NULL, NULL, 0) == MFD_OK,
         "chimera count: N = 0 is a no-op");
  expect(mfd_stream_read(fake, 17, fake, 0) == MFD_ERR_INVALID_ARG, "stream read: ragged size rejected");
  expect(mfd_stream_read(odd, 32, fake, 0) == MFD_ERR_INVALID_ARG, "stream read: misaligned buffer rejected");

  /* fused LM head */
  expect(mfd_lmhead_packed_size(151936, 2560, &b) == MFD_OK && b == (size_t)151936 * 2560 * 2 + (size_t)128 * 2560 * 2,
         "packed head size: rows padded to 256");
  expect(mfd_lmhead_packed_size(1000, 100, &b) == MFD_ERR_INVALID_ARG, "packed head: D not a multiple of 64");
  expect(mfd_lmhead_pack_weight(fake, 1000, 128, fake, 16, 0) == MFD_ERR_INVALID_ARG, "pack: small output rejected");
  expect(mfd_lmhead_logsoftmax_topk(fake, fake, (mfd_head_layout)5, 1, 8, 15, 128, 1000, 8, fake, fake, fake, NULL,
                                    NULL, fake, 1 << 30, 0) == MFD_ERR_INVALID_ARG,
         "fused head: unknown layout rejected");
  expect(mfd_lmhead_logsoftmax_topk(fake, fake, MFD_HEAD_ROWS, 1, 8, 15, 100, 1000, 8, fake, fake, fake, NULL, NULL,
                                    fake, 1 << 30, 0) == MFD_ERR_INVALID_ARG,
         "fused head: D not a multiple of 64 rejected");
  expect(mfd_lmhead_logsoftmax_topk(fake, fake, MFD_HEAD_ROWS, 1, 8, 15, 128, 1000, 8, fake, fake, fake, NULL, NULL,
                                    fake, 16, 0) == MFD_ERR_WORKSPACE,
         "fused head: small workspace rejected");
  expect(mfd_lmhead_logsoftmax_topk_mapped(fake, fake, MFD_HEAD_ROWS, fake, 999, 1, 8, 15, 128, 1000, 8, fake, fake,
                                           fake, NULL, NULL, fake, 1 << 30, 0) == MFD_ERR_INVALID_ARG,
         "fused head mapped: V_full < V rejected");
  return fails == 0 ? 0 : 1;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      exit(3);                                                                 \
    }                                                                          \
  } while (0)
#define MFD_OK_OR_DIE(x)                                                       \
  do {                                                                         \
    mfd_status s_ = (x);                                                       \
    if (s_ != MFD_OK) {                                                        \
      fprintf(stderr, "%s: status %d: %s\n", #x, (int)s_, mfd_last_error());   \
      exit(4);                                                                 \
    }                                                                          \
  } while (0)

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes < 8 ? 8 : bytes));
  return p;
}

static void* read_n(FILE* f, size_t bytes) {
  void* p = malloc(bytes < 8 ? 8 : bytes);
  if (p == NULL || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
  return p;
}

static void* to_dev(const void* h, size_t bytes) {
  void* d = dev_alloc(bytes);
  HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

static void dump(FILE* f, const void* d, size_t bytes) {
  void* h = malloc(bytes < 8 ? 8 : bytes);
  HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  fwrite(h, 1, bytes, f);
  free(h);
}

static int gpu_round(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  if (f == NULL) return 2;
  int32_t* dims = (int32_t*)read_n(f, 5 * sizeof(int32_t));
  const int N = dims[0], K = dims[1], L = dims[2], V = dims[3], B = dims[4];
  const int Bp1 = B + 1, W = (Bp1 + 63) / 64, k = B < V ? (B < 1 ? 1 : B) : V;
  const size_t rows = (size_t)N * K * L;
  void* logits = read_n(f, rows * V * sizeof(float));
  void* anchor = read_n(f, (size_t)N * sizeof(int32_t));
  void* pos = read_n(f, (size_t)N * sizeof(int64_t));
  void* target = read_n(f, (size_t)N * Bp1 * V * sizeof(float));
  void* temp = read_n(f, (size_t)N * sizeof(float));
  void* seed = read_n(f, (size_t)N * sizeof(uint64_t));
  fclose(f);

  void* d_logits = to_dev(logits, rows * V * sizeof(float));
  void* d_anchor = to_dev(anchor, (size_t)N * sizeof(int32_t));
  void* d_pos = to_dev(pos, (size_t)N * sizeof(int64_t));
  void* d_target = to_dev(target, (size_t)N * Bp1 * V * sizeof(float));
  void* d_temp = to_dev(temp, (size_t)N * sizeof(float));
  void* d_seed = to_dev(seed, (size_t)N * sizeof(uint64_t));
  double* lse = (double*)dev_alloc(rows * sizeof(double));
  int32_t* topk_id = (int32_t*)dev_alloc(rows * k * sizeof(int32_t));
  float* topk_raw = (float*)dev_alloc(rows * k * sizeof(float));
  double* cutoff = (double*)dev_alloc((size_t)N * sizeof(double));
  int32_t* n_select = (int32_t*)dev_alloc((size_t)N * sizeof(int32_t));
  int32_t* node_token = (int32_t*)dev_alloc((size_t)N * Bp1 * sizeof(int32_t));
  int32_t* parent = (int32_t*)dev_alloc((size_t)N * Bp1 * sizeof(int32_t));
  int32_t* depth = (int32_t*)dev_alloc((size_t)N * Bp1 * sizeof(int32_t));
  double* score = (double*)dev_alloc((size_t)N * Bp1 * sizeof(double));
  int32_t* best_mode = (int32_t*)dev_alloc((size_t)N * Bp1 * sizeof(int32_t));
  int32_t* n_nodes = (int32_t*)dev_alloc((size_t)N * sizeof(int32_t));
  uint64_t* mask = (uint64_t*)dev_alloc((size_t)N * Bp1 * W * sizeof(uint64_t));
  int64_t* pos_ids = (int64_t*)dev_alloc((size_t)N * Bp1 * sizeof(int64_t));
  int32_t* tau = (int32_t*)dev_alloc((size_t)N * sizeof(int32_t));
  int32_t* out_tokens = (int32_t*)dev_alloc((size_t)N * (L + 1) * sizeof(int32_t));
  int32_t* path_nodes = (int32_t*)dev_alloc((size_t)N * (L + 1) * sizeof(int32_t));
  int32_t* status = (int32_t*)dev_alloc((size_t)N * sizeof(int32_t));
  HIP_OK(hipMemset(status, 0, (size_t)N * sizeof(int32_t)));
  size_t wt = 0, ww = 0;
  MFD_OK_OR_DIE(mfd_workspace_size(MFD_OP_TREE_BUILD, N, K, L, V, B, &wt));
  MFD_OK_OR_DIE(mfd_workspace_size(MFD_OP_VERIFY_WALK, N, K, L, V, B, &ww));
  const size_t wsb = wt > ww ? wt : ww;
  void* ws = dev_alloc(wsb);
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  MFD_OK_OR_DIE(mfd_logsoftmax_topk(d_logits, MFD_F32, N, K, L, V, k, lse, topk_id, topk_raw, NULL, status, NULL, 0,
                                    st));
  MFD_OK_OR_DIE(mfd_mixture_threshold(topk_id, topk_raw, lse, N, K, L, k, B, cutoff, n_select, NULL, status, ws, wsb,
                                      st));
  MFD_OK_OR_DIE(mfd_tree_build(topk_id, topk_raw, lse, cutoff, n_select, (const int32_t*)d_anchor, N, K, L, k, B,
                               node_token, parent, depth, score, best_mode, n_nodes, status, ws, wsb, st));
  MFD_OK_OR_DIE(mfd_tree_mask(parent, depth, n_nodes, (const int64_t*)d_pos, N, Bp1, mask, pos_ids, NULL, st));
  MFD_OK_OR_DIE(mfd_verify_walk(d_target, MFD_F32, N, Bp1, V, L, node_token, parent, depth, n_nodes,
                                (const float*)d_temp, (const uint64_t*)d_seed, tau, out_tokens, path_nodes, status, ws, wsb,
                                st));
  HIP_OK(hipStreamSynchronize(st));

  FILE* o = fopen(out_path, "wb");
  if (o == NULL) return 2;
  dump(o, n_nodes, (size_t)N * sizeof(int32_t));
  dump(o, node_token, (size_t)N * Bp1 * sizeof(int32_t));
  dump(o, parent, (size_t)N * Bp1 * sizeof(int32_t));
  dump(o, depth, (size_t)N * Bp1 * sizeof(int32_t));
  dump(o, mask, (size_t)N * Bp1 * W * sizeof(uint64_t));
  dump(o, pos_ids, (size_t)N * Bp1 * sizeof(int64_t));
  dump(o, tau, (size_t)N * sizeof(int32_t));
  dump(o, out_tokens, (size_t)N * (L + 1) * sizeof(int32_t));
  dump(o, status, (size_t)N * sizeof(int32_t));
  fclose(o);
  HIP_OK(hipStreamDestroy(st));
  printf("abi_smoke gpu: %d trees done\n", N);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "cpu") == 0) {
    const int rc = cpu_checks();
    printf("abi_smoke cpu: %s\n", rc == 0 ? "ok" : "FAILED");
    return rc;
  }
  if (argc >= 4 && strcmp(argv[1], "gpu") == 0) return gpu_round(argv[2], argv[3]);
  fprintf(stderr, "usage: abi_smoke cpu | abi_smoke gpu IN OUT\n");
  return 2;
}
