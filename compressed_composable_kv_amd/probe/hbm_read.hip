// Achievable HBM read rate of the GPU this runs on.
//
// A measurement tool for the benchmark, not part of the C2KV path: a
// streaming read of a caller buffer in which every workgroup reads its own
// contiguous share (its 256 threads read consecutive 16-byte chunks,
// non-temporal, eight in flight per thread), each thread folding what it
// read into one word it writes at the end, so the traffic is the buffer
// read once plus a few KB of writes.  On MI355X this pattern with 256-512
// workgroups streams at about 7.2 TB/s, a grid-stride loop over the same
// buffer at 6.3-7.1 TB/s, and plain (temporal) loads at about 6.0 TB/s.
// Read-dominated kernels (decode reads the whole cache and writes a few
// rows) are compared with this rate rather than with a copy, which also
// writes every byte it reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                            unsigned* __restrict__ out) {
  // this workgroup's share [lo, hi) of the 16-byte units
  const uint64_t per = n16 / gridDim.x;
  const uint64_t lo = (uint64_t)blockIdx.x * per;
  const uint64_t hi = blockIdx.x + 1 == gridDim.x ? n16 : lo + per;
  const u32x4* p = src + lo;
  const uint64_t len = hi - lo;
  u32x4 acc = {0u, 0u, 0u, 0u};
  uint64_t i = threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < len; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) v[j] = __builtin_nontemporal_load(p + i + j * kThreads);
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) acc ^= v[j];
  }
  for (; i < len; i += kThreads) acc ^= p[i];
  out[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the device buffer `buf` with
// `blocks` workgroups of 256 threads, once untimed and `reps` times timed on
// the null stream; `out` is a device buffer of at least blocks * 256 * 4
// bytes.  Writes the best repetition's milliseconds and returns its GB/s
// (bytes read per second), or a negative value on bad arguments or a HIP
// error.
extern "C" double c2kv_probe_hbm_read(const void* buf, uint64_t bytes, void* out, uint64_t out_bytes, int blocks,
                                      int reps, float* ms_out) {
  if (!buf || !out || bytes == 0 || bytes % 16 != 0 || blocks <= 0 || reps <= 0 ||
      out_bytes < (uint64_t)blocks * kThreads * sizeof(unsigned))
    return -1.0;
  const uint64_t n16 = bytes / 16;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  double result = -1.0;
  float best = 0.f;
  if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    hipLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(kThreads), 0, 0, static_cast<const u32x4*>(buf), n16,
                       static_cast<unsigned*>(out));
    bool ok = hipGetLastError() == hipSuccess;
    for (int r = 0; ok && r < reps; ++r) {
      float ms = 0.f;
      hipEventRecord(e0, 0);
      hipLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(kThreads), 0, 0, static_cast<const u32x4*>(buf), n16,
                         static_cast<unsigned*>(out));
      hipEventRecord(e1, 0);
      ok = hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess &&
           hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f;
      if (ok && (best == 0.f || ms < best)) best = ms;
    }
    if (ok && best > 0.f) result = (double)bytes / (best * 1e-3) / 1e9;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (ms_out) *ms_out = best;
  return result;
}
