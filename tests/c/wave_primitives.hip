// Checks the wave-level primitives of the kernels (mfd_device.hpp) against
// results computed on the host: lane exchanges at every stride and type, the
// wave and block scans, and the sorting networks at every size they serve.
// One block per check; every write stays inside its output array.  Prints
// one line per check and ALL OK / FAIL; exit status 0 only if all agree.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <algorithm>
#include <vector>
#include "mfd_device.hpp"
using namespace mfd;

__global__ void xor_test(const uint64_t* in, uint64_t* out) {  // out[s_idx * 64 + lane]
  const int lane = threadIdx.x;
  const uint64_t v = in[lane];
  int si = 0;
  for (int s = 1; s < 64; s <<= 1, ++si) {
    out[si * 64 + lane] = xor_lanes(v, s);
    out[(6 + si) * 64 + lane] = (uint64_t)(uint32_t)xor_lanes((int)(uint32_t)v, s);
    const double d = xor_lanes((double)(int64_t)(v & 0xFFFFF), s);
    out[(12 + si) * 64 + lane] = (uint64_t)(int64_t)d;
    const float f = xor_lanes((float)(int)(v & 0xFFF), s);
    out[(18 + si) * 64 + lane] = (uint64_t)(int)f;
  }
}
__global__ void scan_test(const int* in, int* out) {  // 1024 threads: wave scans and a block scan
  const int t = threadIdx.x;
  __shared__ int smem[16];
  out[t] = wave_inclusive_scan(in[t]);
  int tot;
  out[1024 + t] = block_exclusive_scan<1024>(in[t], smem, &tot);
  if (t == 0) out[2048] = tot;
  out[2049 + t] = wave_sum(in[t]);
}
__global__ void sort_test(const uint64_t* in, uint64_t* out, int P) {  // 1024 threads, P <= 4096 keys
  __shared__ uint64_t a[4096];
  for (int i = threadIdx.x; i < P; i += 1024) a[i] = in[i];
  __syncthreads();
  block_sort_keys<1024>(a, P);
  for (int i = threadIdx.x; i < P; i += 1024) out[i] = a[i];
}
__global__ void sort_test256(const uint64_t* in, uint64_t* out, int P) {  // 256 threads, P <= 1024 keys
  __shared__ uint64_t a[1024];
  for (int i = threadIdx.x; i < P; i += 256) a[i] = in[i];
  __syncthreads();
  block_sort_keys<256>(a, P);
  for (int i = threadIdx.x; i < P; i += 256) out[i] = a[i];
}
__global__ void small_sorts(const uint64_t* in, uint64_t* out) {  // 256 threads
  __shared__ uint64_t x[512];
  const int t = threadIdx.x;
  uint64_t a = in[t];
  block_sort_single<256>(a, x);
  out[t] = a;
  __syncthreads();
  uint64_t a0 = in[256 + 2 * t], a1 = in[256 + 2 * t + 1];
  block_sort_pairs<256>(a0, a1, x);
  out[256 + 2 * t] = a0;
  out[256 + 2 * t + 1] = a1;
  uint64_t w = in[768 + t];
  if (t < 64) out[768 + t] = wave_sort_desc(w);
}

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next() { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return rng; }
#define CK(x) do { if ((x) != hipSuccess) { printf("hip error line %d\n", __LINE__); return 1; } } while (0)

int main() {
  int bad = 0;
  {  // xor_lanes
    std::vector<uint64_t> h(64), r(24 * 64);
    for (auto& v : h) v = next();
    uint64_t *din, *dout;
    CK(hipMalloc(&din, 64 * 8)); CK(hipMalloc(&dout, 24 * 64 * 8));
    CK(hipMemcpy(din, h.data(), 64 * 8, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(xor_test, dim3(1), dim3(64), 0, 0, din, dout);
    CK(hipMemcpy(r.data(), dout, 24 * 64 * 8, hipMemcpyDeviceToHost));
    int si = 0;
    for (int s = 1; s < 64; s <<= 1, ++si)
      for (int l = 0; l < 64; ++l) {
        const uint64_t src = h[l ^ s];
        if (r[si * 64 + l] != src) ++bad;
        if (r[(6 + si) * 64 + l] != (uint64_t)(uint32_t)src) ++bad;
        if (r[(12 + si) * 64 + l] != (src & 0xFFFFF)) ++bad;
        if (r[(18 + si) * 64 + l] != (src & 0xFFF)) ++bad;
      }
    printf("xor_lanes mismatches: %d\n", bad);
    CK(hipFree(din)); CK(hipFree(dout));
  }
  {  // scans
    std::vector<int> h(1024), r(2049 + 1024);
    for (auto& v : h) v = (int)(next() % 17);
    int *din, *dout;
    CK(hipMalloc(&din, 1024 * 4)); CK(hipMalloc(&dout, r.size() * 4));
    CK(hipMemcpy(din, h.data(), 1024 * 4, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(scan_test, dim3(1), dim3(1024), 0, 0, din, dout);
    CK(hipMemcpy(r.data(), dout, r.size() * 4, hipMemcpyDeviceToHost));
    int b = 0, acc = 0;
    for (int w = 0; w < 16; ++w) {
      int wa = 0, ws = 0;
      for (int l = 0; l < 64; ++l) ws += h[w * 64 + l];
      for (int l = 0; l < 64; ++l) {
        wa += h[w * 64 + l];
        if (r[w * 64 + l] != wa) ++b;
        if (r[2049 + w * 64 + l] != ws) ++b;
      }
    }
    for (int t = 0; t < 1024; ++t) { if (r[1024 + t] != acc) ++b; acc += h[t]; }
    if (r[2048] != acc) ++b;
    printf("scan mismatches: %d\n", b);
    bad += b;
    CK(hipFree(din)); CK(hipFree(dout));
  }
  for (int P : {64, 128, 256, 512, 1024, 2048, 4096}) {  // block_sort_keys
    std::vector<uint64_t> h(P), r(P);
    for (auto& v : h) v = next() % 1000;  // many equal keys
    uint64_t *din, *dout;
    CK(hipMalloc(&din, P * 8)); CK(hipMalloc(&dout, P * 8));
    CK(hipMemcpy(din, h.data(), P * 8, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(sort_test, dim3(1), dim3(1024), 0, 0, din, dout, P);
    CK(hipMemcpy(r.data(), dout, P * 8, hipMemcpyDeviceToHost));
    std::sort(h.begin(), h.end());
    int b = 0;
    for (int i = 0; i < P; ++i) b += r[i] != h[i];
    printf("block_sort_keys P=%d mismatches: %d\n", P, b);
    bad += b;
    CK(hipFree(din)); CK(hipFree(dout));
  }
  for (int P : {64, 128, 256, 512, 1024}) {  // block_sort_keys with 256 threads
    std::vector<uint64_t> h(P), r(P);
    for (auto& v : h) v = next() % 1000;
    uint64_t *din, *dout;
    CK(hipMalloc(&din, P * 8)); CK(hipMalloc(&dout, P * 8));
    CK(hipMemcpy(din, h.data(), P * 8, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(sort_test256, dim3(1), dim3(256), 0, 0, din, dout, P);
    CK(hipMemcpy(r.data(), dout, P * 8, hipMemcpyDeviceToHost));
    std::sort(h.begin(), h.end());
    int b = 0;
    for (int i = 0; i < P; ++i) b += r[i] != h[i];
    printf("block_sort_keys<256> P=%d mismatches: %d\n", P, b);
    bad += b;
    CK(hipFree(din)); CK(hipFree(dout));
  }
  {  // block_sort_single, block_sort_pairs, wave_sort_desc
    std::vector<uint64_t> h(1024), r(1024);
    for (auto& v : h) v = next();
    uint64_t *din, *dout;
    CK(hipMalloc(&din, 1024 * 8)); CK(hipMalloc(&dout, 1024 * 8));
    CK(hipMemcpy(din, h.data(), 1024 * 8, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(small_sorts, dim3(1), dim3(256), 0, 0, din, dout);
    CK(hipMemcpy(r.data(), dout, 1024 * 8, hipMemcpyDeviceToHost));
    std::vector<uint64_t> a(h.begin(), h.begin() + 256), p(h.begin() + 256, h.begin() + 768), w(h.begin() + 768, h.begin() + 832);
    std::sort(a.begin(), a.end()); std::sort(p.begin(), p.end()); std::sort(w.begin(), w.end(), std::greater<uint64_t>());
    int b = 0;
    for (int i = 0; i < 256; ++i) b += r[i] != a[i];
    for (int i = 0; i < 512; ++i) b += r[256 + i] != p[i];
    for (int i = 0; i < 64; ++i) b += r[768 + i] != w[i];
    printf("single/pairs/wave sorts mismatches: %d\n", b);
    bad += b;
    CK(hipFree(din)); CK(hipFree(dout));
  }
  printf(bad ? "FAIL\n" : "ALL OK\n");
  return bad ? 4 : 0;
}
