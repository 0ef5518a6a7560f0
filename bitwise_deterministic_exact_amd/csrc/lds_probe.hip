// LDS atomic throughput probe for the benchmark's roofline (not part of the
// library: bench.py loads it to measure the peak that det_gemm's kernel is
// held to).  No published figure gives the rate of non-returning LDS integer
// atomics on gfx950, so the benchmark measures it with this kernel, shaped
// like the GEMM kernels' accumulate step: every lane adds into its own word
// of a 64-word row (conflict-free, as the cells are laid out), each step into
// another 1 KiB cell of the workgroup's array, with the workgroup size and
// LDS footprint of the kernel it stands for (64-bit adds: 128 KiB and 16
// waves, one workgroup per CU; 32-bit adds: 64 KiB and 8 waves, two per CU).
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

template <typename T, int WAVES, int KIB>
__global__ __launch_bounds__(64 * WAVES) void k_lds_add_rate(int steps, T inc, T* sink) {
  constexpr uint32_t BYTES = KIB * 1024u;
  __shared__ __align__(16) T cells[BYTES / sizeof(T)];
  for (uint32_t i = threadIdx.x; i < BYTES / sizeof(T); i += blockDim.x) cells[i] = 0;
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
  char* const base = reinterpret_cast<char*>(cells);
  uint32_t off = wave * 1024u + lane * static_cast<uint32_t>(sizeof(T));
  constexpr uint32_t STRIDE = WAVES * 1024u;          // the next cell of this wave
  for (int i = 0; i < steps; i += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      atomicAdd(reinterpret_cast<T*>(base + ((off + u * STRIDE) & (BYTES - 1u))), inc);
    off += 8u * STRIDE;
  }
  __syncthreads();
  if (threadIdx.x < 64) atomicAdd(&sink[threadIdx.x], cells[threadIdx.x]);   // keeps the adds observable
}

template <typename T, int WAVES, int KIB>
hipError_t run(int blocks, int steps, hipStream_t s, float* ms) {
  T* sink = nullptr;
  hipError_t e = hipMalloc(&sink, 64 * sizeof(T));
  if (e != hipSuccess) return e;
  hipEvent_t a = nullptr, b = nullptr;
  e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) {
    hipLaunchKernelGGL((k_lds_add_rate<T, WAVES, KIB>), dim3(blocks), dim3(64 * WAVES), 0, s, steps, T(1), sink);
    e = hipEventRecord(a, s);
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL((k_lds_add_rate<T, WAVES, KIB>), dim3(blocks), dim3(64 * WAVES), 0, s, steps, T(1), sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  (void)hipFree(sink);
  return e;
}

}  // namespace

extern "C" {

// One timed launch (after one untimed) of `blocks` workgroups, each wave
// doing `steps` (a multiple of 8) non-returning atomic adds per lane; bits =
// 64 (the f32 GEMM's cells) or 32 (bf16's).  *ms: the launch's duration.
// Returns 0, or a hipError_t.
int lds_probe_add_rate(int bits, int blocks, int steps, void* stream, float* ms) {
  if (blocks < 1 || steps < 8 || steps % 8 != 0 || ms == nullptr) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bits == 64) return static_cast<int>(run<unsigned long long, 16, 128>(blocks, steps, s, ms));
  if (bits == 32) return static_cast<int>(run<unsigned int, 8, 64>(blocks, steps, s, ms));
  return -1;
}

// lane-atomics one launch performs (for the rate)
double lds_probe_lane_ops(int bits, int blocks, int steps) {
  const int waves = bits == 64 ? 16 : 8;
  return static_cast<double>(blocks) * 64.0 * waves * steps;
}

}  // extern "C"
