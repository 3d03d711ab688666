// The extractor layer around the structured attention, on gfx950:
//   * gemm_nt_kernel: C = A * B^T in bf16 with fp32 accumulation on
//     v_mfma_f32_16x16x32_bf16, 128x128 output tiles, K in steps of 64
//     brought into LDS by buffer_load ... lds (two stages, XOR-swizzled
//     16-byte chunks).
//     A row-range table picks the weight matrix per row tile (document rows
//     take the frozen projections, slot rows the C2 ones); the epilogue
//     splits columns over up to three outputs (q | k | v), adds a residual
//     in fp32 and rounds once, or (gate/up rows interleaved in blocks of
//     16) writes silu(gate) * up.
//   * rms_norm_kernel: one workgroup per row, fp32 sum of squares.
//   * slot_fill_kernel: writes the shared slot vector into every slot row.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "c2kv_device.hpp"
#include "c2kv_launch.hpp"

namespace c2kv {

constexpr int kGM = 128, kGN = 128, kGK = 64;
constexpr int kGroupM = 8;   // row tiles per group of the tile order

// Tile order.  The eight XCDs each have their own L2 and receive workgroups
// round robin, so physical workgroup p becomes logical tile
// (p % 8) * (grid / 8) + p / 8: each XCD walks a contiguous slice of the
// logical order.  That order takes groups of kGroupM row tiles with the row
// tile varying fastest, so the 64 workgroups an XCD holds at once cover
// about 8 row tiles x 8 column tiles and share each A and B panel through
// the XCD's L2.  Returns false for the padding workgroups past the last tile.
__device__ __forceinline__ bool gemm_tile(int p, int grid, int m_tiles, int n_tiles, int& mt, int& nt) {
  const int t = (p & 7) * (grid >> 3) + (p >> 3);   // grid is a multiple of 8
  if (t >= m_tiles * n_tiles) return false;
  const int group_tiles = kGroupM * n_tiles;
  const int g = t / group_tiles, local = t % group_tiles;
  const int gm0 = g * kGroupM;
  const int gsz = min(kGroupM, m_tiles - gm0);
  mt = gm0 + local % gsz;
  nt = local / gsz;
  return true;
}

typedef __attribute__((address_space(3))) void lds_void;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) bf16 lds[2][2][kGM * kGK];   // [stage][A, B]: 64 KB
  // the stages are written only by buffer_load ... lds; escape them so the
  // compiler does not treat them as never-stored memory
  asm volatile("" : : "r"(&lds[0][0][0]) : "memory");
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mt, nt;
  if (!gemm_tile((int)blockIdx.x, (int)gridDim.x, p.m_tiles, p.n_tiles, mt, nt)) return;
  int lo = 0, hi = p.num_ranges - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.ranges[mid].tile0 <= mt) lo = mid; else hi = mid - 1;
  }
  const GemmRange rg = p.ranges[lo];
  const int row0 = rg.row0 + (mt - rg.tile0) * kGM;
  const int valid = min(kGM, rg.row0 + rg.rows - row0);
  const bf16* B = rg.sel ? p.b1 : p.b0;
  const int n0 = nt * kGN;

  // LDS DMA: each tile (A or B) is 16 blocks of 1 KB (8 rows of 64 k);
  // wave w fills blocks 4w..4w+3 of both.  Lane l of block b fills LDS slot
  // (row b*8 + l/8, chunk l%8) with logical k chunk (l%8) ^ (row & 7), the
  // XOR swizzle the operand reads undo.  Rows past the range repeat a valid
  // row (their results are not stored).  The K step goes into the
  // wave-uniform offset.
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + (int64_t)row0 * p.lda), 0, (int)((int64_t)valid * p.lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + (int64_t)n0 * p.K), 0, (int)((int64_t)kGN * p.K * 2), 0x00020000);
  int aoff[4], boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave * 4 + j) * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ (row & 7);
    aoff[j] = (int)((int64_t)min(row, valid - 1) * p.lda * 2) + kc * 16;
    boff[j] = row * p.K * 2 + kc * 16;
  }
#define C2KV_DMA(kt, st)                                                                                   \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                        \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void*)&lds[st][0][(wave * 4 + j) * 512], 16, aoff[j], \
                                             (kt) * kGK * 2, 0, 0);                                      \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void*)&lds[st][1][(wave * 4 + j) * 512], 16, boff[j], \
                                             (kt) * kGK * 2, 0, 0);                                      \
  }

  // C^T tiles: the weight rows (n) are the MFMA's A operand and the input
  // rows (m) its B operand, so each lane ends with 4 consecutive columns of
  // one output row.  Wave (wm, wn) owns rows wm*64.. and columns wn*64..
  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / kGK;
  C2KV_DMA(0, 0)
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    // this wave's DMA of step kt has landed; after the barrier every
    // wave's has, and every wave is done reading the other stage
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (kt + 1 < nk) { C2KV_DMA(kt + 1, buf ^ 1) }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kc = s * 4 + (lane >> 4);   // both operands: k elements 8*(lane/16).. of slab s
      bf16x8 wf[4], xf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rn = wn * 64 + i * 16 + (lane & 15);
        const int rm = wm * 64 + i * 16 + (lane & 15);
        wf[i] = *reinterpret_cast<const bf16x8*>(&lds[buf][1][rn * kGK + ((kc ^ (rn & 7)) << 3)]);
        xf[i] = *reinterpret_cast<const bf16x8*>(&lds[buf][0][rm * kGK + ((kc ^ (rm & 7)) << 3)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma16(wf[i], xf[j], acc[i][j]);
    }
  }
#undef C2KV_DMA

  // lane holds C[row0 + wm*64 + j*16 + lane%16][n0 + wn*64 + i*16 + 4*(lane/16) + 0..3]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ml = wm * 64 + j * 16 + (lane & 15);
    if (ml >= valid) continue;
    const int64_t row = row0 + ml;
    if (EPI == kEpiSwiglu) {
      // weight rows come in blocks of 16 gate rows then the matching 16 up
      // rows, so block i (gate) and block i + 1 (up) of this lane hold the
      // same 4 FFN columns f: act[row][f] = silu(gate) * up
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int n = n0 + wn * 64 + i * 16 + 4 * (lane >> 4);
        const int f = (n >> 5) * 16 + (n & 15);
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g = acc[i][j][e];
          o4[e] = from_f32<bf16>(g / (1.0f + expf(-g)) * acc[i + 1][j][e]);
        }
        *reinterpret_cast<bf16x4*>(p.c0 + row * p.ldc0 + f) = o4;
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn * 64 + i * 16 + 4 * (lane >> 4);
      bf16* dst;
      if (n < p.n1) dst = p.c0 + row * p.ldc0 + n;
      else if (n < p.n2) dst = p.c1 + row * p.ldc1 + (n - p.n1);
      else dst = p.c2 + row * p.ldc2 + (n - p.n2);
      float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
      if (EPI == kEpiResidual) {
        const bf16x4 r4 = *reinterpret_cast<const bf16x4*>(p.r + row * p.ldr + n);
        v0 += to_f32(r4[0]);
        v1 += to_f32(r4[1]);
        v2 += to_f32(r4[2]);
        v3 += to_f32(r4[3]);
      }
      bf16x4 o4;
      o4[0] = from_f32<bf16>(v0);
      o4[1] = from_f32<bf16>(v1);
      o4[2] = from_f32<bf16>(v2);
      o4[3] = from_f32<bf16>(v3);
      *reinterpret_cast<bf16x4*>(dst) = o4;
    }
  }
}

hipError_t launch_gemm(const GemmParams& p, int epi, hipStream_t st) {
  const int64_t tiles = (int64_t)p.m_tiles * p.n_tiles;
  if (tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8));   // a multiple of the 8 XCDs
  if (epi == kEpiResidual)
    hipLaunchKernelGGL((gemm_nt_kernel<kEpiResidual>), grid, dim3(256), 0, st, p);
  else if (epi == kEpiSwiglu)
    hipLaunchKernelGGL((gemm_nt_kernel<kEpiSwiglu>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<kEpiStore>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

// ------------------------------------------------------------- RMSNorm
// h[r] = bf16(x[r] / sqrt(mean(x[r]^2) + eps) * gamma), one workgroup per
// row, 8 elements per thread and step.
__global__ __launch_bounds__(256) void rms_norm_kernel(const bf16* __restrict__ x, const bf16* __restrict__ gamma,
                                                       bf16* __restrict__ h, int dm, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int tid = (int)threadIdx.x;
  const bf16* xr = x + row * dm;
  float ss = 0.f;
  for (int c = tid; c < dm / 8; c += 256) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(xr + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += to_f32(v[e]) * to_f32(v[e]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float rs = 1.0f / sqrtf(tot / (float)dm + eps);
  bf16* hr = h + row * dm;
  for (int c = tid; c < dm / 8; c += 256) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(xr + c * 8);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(gamma + c * 8);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = from_f32<bf16>(to_f32(v[e]) * rs * to_f32(g[e]));
    *reinterpret_cast<bf16x8*>(hr + c * 8) = o;
  }
}

hipError_t launch_rms_norm(const void* x, const void* gamma, void* h, int64_t rows, int dm, float eps,
                           hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rms_norm_kernel, dim3((unsigned)rows), dim3(256), 0, st, static_cast<const bf16*>(x),
                     static_cast<const bf16*>(gamma), static_cast<bf16*>(h), dm, eps);
  return hipGetLastError();
}

// ----------------------------------------------------------- slot fill
// One workgroup per slot row of the launch's documents: x[row] = embed.
__global__ __launch_bounds__(256) void slot_fill_kernel(const SlotFillParams p) {
  const int s = (int)blockIdx.x;
  int lo = 0, hi = p.num_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.docs[mid].slot0 <= s) lo = mid; else hi = mid - 1;
  }
  const int64_t row = p.docs[lo].row0 + (s - p.docs[lo].slot0);
  bf16* xr = static_cast<bf16*>(p.x) + row * p.dm;
  const bf16* e = static_cast<const bf16*>(p.embed);
  for (int c = (int)threadIdx.x; c < p.dm / 8; c += 256)
    *reinterpret_cast<uint4*>(xr + c * 8) = *reinterpret_cast<const uint4*>(e + c * 8);
}

hipError_t launch_slot_fill(const SlotFillParams& p, int slots, hipStream_t st) {
  if (slots == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_fill_kernel, dim3((unsigned)slots), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace c2kv
