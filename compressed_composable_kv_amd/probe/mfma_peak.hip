// Achievable dense bf16 MFMA rate of the GPU this runs on.
//
// A measurement tool for the benchmark, not part of the C2KV path: every
// wave runs NCHAIN independent accumulation chains of
// v_mfma_f32_16x16x32_bf16 (16 384 FLOPs each) on register operands, with
// no memory traffic inside the timed loop, so the figure is the rate the
// matrix cores sustain at the clock the chip holds under that load.  The
// published peak assumes the nominal 2.4 GHz; under sustained MFMA load the
// chip runs slower, and this probe measures what is left.
//
// Two operand modes.  "constant": every MFMA of a wave reads the same two
// operand registers, so the matrix datapath sees the same inputs every
// cycle and draws little power.  "data": the chains cycle through 4 x 4
// pairs of operand registers filled with random bf16 values, so consecutive
// MFMAs see different inputs, as they do in an attention tile; the power
// the board may draw then bounds the clock, and this mode measures the
// rate that is left for MFMA work on real data.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 16;

template <bool kData>
__global__ __launch_bounds__(512) void mfma_chain_kernel(float* out, int iters) {
  constexpr int NV = kData ? 4 : 1;
  bf16x8 a[NV], b[NV];
  unsigned h = (blockIdx.x * blockDim.x + threadIdx.x) * 2654435761u + 12345u;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (kData) {
        h = h * 1664525u + 1013904223u;
        a[v][j] = (__bf16)((float)((h >> 8) & 0xFFFF) * (1.f / 32768.f) - 1.f);
        h = h * 1664525u + 1013904223u;
        b[v][j] = (__bf16)((float)((h >> 8) & 0xFFFF) * (1.f / 32768.f) - 1.f);
      } else {
        a[v][j] = (__bf16)(1e-3f * (float)((threadIdx.x + j) & 63));
        b[v][j] = (__bf16)(1e-3f * (float)j);
      }
    }
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c % NV], b[(c / NV) % NV], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps the chains live
}

}  // namespace

template <bool kData>
static double run_probe(int blocks, int threads, int iters, float* ms_out) {
  if (blocks <= 0 || threads <= 0 || threads > 512 || threads % 64 != 0 || iters <= 0) return -1.0;
  float* out = nullptr;
  if (hipMalloc(&out, sizeof(float) * (size_t)blocks * threads) != hipSuccess) return -1.0;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  double result = -1.0;
  float ms = 0.f;
  if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    hipLaunchKernelGGL(mfma_chain_kernel<kData>, dim3(blocks), dim3(threads), 0, 0, out, iters);
    hipEventRecord(e0, 0);
    hipLaunchKernelGGL(mfma_chain_kernel<kData>, dim3(blocks), dim3(threads), 0, 0, out, iters);
    hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess &&
        hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f) {
      const double flops = (double)blocks * (threads / 64) * (double)iters * kChains * 16384.0;
      result = flops / (ms * 1e-3) / 1e12;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (ms_out) *ms_out = ms;
  return result;
}

// Runs `blocks` workgroups of `threads` threads (a multiple of 64, at most
// 512), each wave doing iters * 16 MFMAs, once untimed and once timed on the
// null stream.  Writes the timed kernel's milliseconds and returns the
// achieved TFLOP/s, or a negative value on a HIP error.  Allocates and frees
// its own output buffer.  _data: random operands that change from one MFMA
// to the next (see above).
extern "C" double c2kv_probe_mfma_bf16(int blocks, int threads, int iters, float* ms_out) {
  return run_probe<false>(blocks, threads, iters, ms_out);
}
extern "C" double c2kv_probe_mfma_bf16_data(int blocks, int threads, int iters, float* ms_out) {
  return run_probe<true>(blocks, threads, iters, ms_out);
}
