// hop_probe: latency of the all-to-all exchange the batch-1 persistent decode
// kernel performs three times per layer, measured alone.  A cooperative grid
// of workgroups (one per CU) runs 2000 exchanges back to back; in each, every
// workgroup publishes its words (64-bit {value, exchange number}, relaxed
// device-scope stores into R replicas) and then reads every workgroup's words
// from its replica with relaxed device-scope loads until all are fresh.
// Consecutive exchanges alternate between two buffers, so a buffer is
// rewritten only after every reader has passed it.  Reported: microseconds
// per exchange, for
//   - the kernel's poll (wait on the first stale word, then re-issue every
//     stale word) and a poll that re-issues every stale word each round;
//   - 2, 8 and 16 KB per reader (the B/C, residual and gated-output payloads);
//   - grids of 256 down to 16 workgroups, 16 KB per reader.
// Every workgroup also checks that its hardware XCD id equals blockIdx % 8
// (the dispatch order the persistent kernel's replica choice relies on for
// spreading readers).  Every wait is bounded: a workgroup that polls too long
// raises an abort flag that ends all of them.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);           \
      exit(1);                                                                        \
    }                                                                                 \
  } while (0)

namespace {

constexpr int kT = 256;          // threads per workgroup
constexpr int kMaxG = 256;       // largest grid
constexpr int kWords = 2048;     // words per reader at the largest payload
constexpr int kR = 4;            // replicas
constexpr long kSpin = 1 << 20;  // polls before giving up

__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t word(unsigned v, unsigned e) { return ((uint64_t)e << 32) | v; }
__device__ __forceinline__ bool fresh(uint64_t w, unsigned e) { return (unsigned)(w >> 32) == e; }
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ bool give_up(long spins, int* abort_flag) {
  if (spins > kSpin) {
    __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  return (spins & 63) == 0 && __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// words base[m * kT], m < n; ALL: re-issue every stale word each round, else
// wait on the first stale word alone, then re-issue every stale one
template <int MAXW, bool ALL>
__device__ bool poll(const uint64_t* base, int n, unsigned e, int* abort_flag, uint64_t (&w)[MAXW]) {
#pragma unroll
  for (int m = 0; m < MAXW; ++m) w[m] = m < n ? ld_dev(base + m * kT) : word(0, e);
  long spins = 0;
  for (;;) {
    int first = -1;
#pragma unroll
    for (int m = MAXW - 1; m >= 0; --m)
      if (!fresh(w[m], e)) first = m;
    if (first < 0) return true;
    if (!ALL) {
      uint64_t v = ld_dev(base + first * kT);
      while (!fresh(v, e)) {
        if (give_up(++spins, abort_flag)) return false;
        v = ld_dev(base + first * kT);
      }
    } else if (give_up(++spins, abort_flag)) {
      return false;
    }
#pragma unroll
    for (int m = 0; m < MAXW; ++m)
      if (!fresh(w[m], e)) w[m] = ld_dev(base + m * kT);
  }
}

// n_words words in total, published by gridDim.x workgroups (n_words / grid each)
// and read by every workgroup (n_words / kT per thread, at most 8)
template <bool ALL>
__global__ __launch_bounds__(kT, 1) void exchange_kernel(uint64_t* box, int n_words, int n_ex, int* abort_flag,
                                                         int* errors, int* xcd_mismatch) {
  __shared__ int s_stop;
  if (threadIdx.x == 0) s_stop = 0;
  lds_barrier();
  const int w = blockIdx.x;
  const int per = n_words / gridDim.x, mine = n_words / kT;
  const int xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15;  // HW_REG_XCC_ID
  if (threadIdx.x == 0 && xcc != (w & 7)) atomicAdd(xcd_mismatch, 1);
  uint64_t v[8];
  for (int x = 0; x < n_ex; ++x) {
    const unsigned e = (unsigned)x + 1;
    uint64_t* bx = box + (size_t)(x & 1) * kR * n_words;
    if (threadIdx.x < per)
      for (int r = 0; r < kR; ++r)
        st_dev(bx + (size_t)r * n_words + w * per + threadIdx.x, word((unsigned)(w * per + threadIdx.x) ^ e, e));
    if (!poll<8, ALL>(bx + (size_t)(w % kR) * n_words + threadIdx.x, mine, e, abort_flag, v)) s_stop = 1;
    lds_barrier();
    if (s_stop) return;
    if (x == n_ex - 1)
      for (int m = 0; m < mine; ++m)
        if ((unsigned)v[m] != ((unsigned)(threadIdx.x + m * kT) ^ e)) atomicAdd(errors, 1);
  }
}

template <bool ALL>
void run(uint64_t* box, int grid, int n_words, int* flags, const char* name) {
  int n_ex = 2000;
  CHECK(hipMemset(box, 0, sizeof(uint64_t) * 2 * kR * kWords));
  CHECK(hipMemset(flags, 0, 3 * sizeof(int)));
  int* abort_flag = flags;
  int* errors = flags + 1;
  int* mism = flags + 2;
  void* args[] = {&box, &n_words, &n_ex, &abort_flag, &errors, &mism};
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  CHECK(hipEventRecord(a, 0));
  CHECK(hipLaunchCooperativeKernel((const void*)exchange_kernel<ALL>, dim3(grid), dim3(kT), args, 0, 0));
  CHECK(hipEventRecord(b, 0));
  CHECK(hipEventSynchronize(b));
  float ms = 0.0f;
  CHECK(hipEventElapsedTime(&ms, a, b));
  int h[3];
  CHECK(hipMemcpy(h, flags, sizeof(h), hipMemcpyDeviceToHost));
  printf("%-30s grid %3d  %5d B per reader: %6.3f us per exchange  (abort %d, wrong words %d, XCD != blockIdx %% 8: %d)\n",
         name, grid, n_words * 8, ms * 1000.0f / n_ex, h[0], h[1], h[2]);
  fflush(stdout);
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
}

}  // namespace

int main() {
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  if (cus < kMaxG) {
    printf("needs %d compute units for one workgroup per CU (device has %d)\n", kMaxG, cus);
    return 1;
  }
  uint64_t* box = nullptr;
  int* flags = nullptr;
  CHECK(hipMalloc(&box, sizeof(uint64_t) * 2 * kR * kWords));
  CHECK(hipMalloc(&flags, 3 * sizeof(int)));
  for (int rep = 0; rep < 2; ++rep) {
    printf("-- pass %d\n", rep + 1);
    for (int words : {256, 1024, 2048}) run<false>(box, 256, words, flags, "first-stale poll");
    for (int words : {256, 1024, 2048}) run<true>(box, 256, words, flags, "poll every stale word");
    for (int g : {128, 64, 32, 16}) run<false>(box, g, 2048, flags, "first-stale poll");
  }
  CHECK(hipFree(box));
  CHECK(hipFree(flags));
  return 0;
}
