// Device-side building blocks of the C2KV kernels for gfx950 (CDNA4):
// element traits, MFMA wrappers, RoPE rotation, wave reductions, and the
// kernel parameter blocks shared with the host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "c2kv.h"

namespace c2kv {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- tiling
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kQW = 32;        // query rows per wave (two 16-row MFMA blocks)
constexpr int kWaves = 4;      // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxHalfDim = 64;
static_assert(kBN == C2KV_EXTRACT_TILE_KEYS && kQW == C2KV_EXTRACT_UNIT_ROWS, "tile shape is part of the ABI");

template <typename T> struct ElemTraits;
template <> struct ElemTraits<bf16> {
  using v8 = bf16x8;
  using v4 = bf16x4;
  static constexpr int kChunk = 8;     // elements per 16-byte chunk
};
template <> struct ElemTraits<float> {
  using v8 = f32x8;
  using v4 = f32x4;
  static constexpr int kChunk = 4;
};

// D[16x16] += A[16x32] * B[32x16].  Lane l supplies A row l%16 and B column
// l%16, each with 8 consecutive k-elements of group l/16; the same (group,
// element) -> k assignment holds for A and B, so any k order the hardware
// uses gives the same sum.  Result lane l holds D rows 4*(l/16)+i, column l%16.
__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 operands: eight 16x16x4 steps, step e taking element e of each lane's
// 8-element group as that lane's single k value.
__device__ __forceinline__ f32x4 mma16(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// D[32x32] += A[32x16] * B[16x32].  Lane l supplies A row l%32 and B column
// l%32, each with 8 k-elements of half l/32 (paired alike in A and B, so the
// k order does not matter).  Result register i of lane l holds D row
// 8*(i/4) + 4*(l/32) + i%4, column l%32.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ---------------------------------------------------------------- RoPE
// Rotation of one half-split pair (x_i, x_{i+d/2}) by (c, s) with each
// product and sum rounded to fp32 separately (no contraction).
__device__ __forceinline__ void rope_pair(float x0, float x1, float c, float s,
                                          float& y0, float& y1) {
#pragma clang fp contract(off)
  const float a = x0 * c;
  const float b = x1 * s;
  const float e = x1 * c;
  const float f = x0 * s;
  y0 = a - b;
  y1 = e + f;
}

// cos/sin of the fp32 angle fp32(pos) * inv_freq (one rounded multiply).
__device__ __forceinline__ void rope_cs(int32_t pos, float inv_freq, float& c, float& s) {
#pragma clang fp contract(off)
  const float ang = static_cast<float>(pos) * inv_freq;
  sincosf(ang, &s, &c);
}

struct RopeFreqs {
  float f[kMaxHalfDim];
};

// 16-byte chunks of CE elements, unpacked to and packed from fp32.
template <typename T> struct Chunk;
template <> struct Chunk<bf16> {
  static constexpr int CE = 8;
  __device__ static void unpack(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static uint4 pack(const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16 a = static_cast<bf16>(f[2 * i]);
      const bf16 b = static_cast<bf16>(f[2 * i + 1]);
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Chunk<float> {
  static constexpr int CE = 4;
  __device__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

// Rotate one chunk pair (lo = elements [i0, i0+CE), hi = the same + d/2)
// with per-element (cos, sin).
template <typename T>
__device__ __forceinline__ void rotate_chunk(uint4& lo, uint4& hi, const float* c, const float* s) {
  constexpr int CE = Chunk<T>::CE;
  float a[CE], b[CE], y0[CE], y1[CE];
  Chunk<T>::unpack(lo, a);
  Chunk<T>::unpack(hi, b);
#pragma unroll
  for (int e = 0; e < CE; ++e) rope_pair(a[e], b[e], c[e], s[e], y0[e], y1[e]);
  lo = Chunk<T>::pack(y0);
  hi = Chunk<T>::pack(y1);
}

// Index of the request (or document) that workgroup L belongs to, given
// the entries' first workgroups wg0 (ascending, the first 0) in a
// kernel-argument table of up to 64 entries: one lane-indexed load and a
// ballot, instead of a walk whose every step waits for a kernel-argument
// load.
template <typename Req>
__device__ __forceinline__ int request_of(const Req* reqs, int num_reqs, int L) {
  if (num_reqs == 1) return 0;
  const int lane = threadIdx.x & 63;
  const int w = reqs[min(lane, num_reqs - 1)].wg0;
  const uint64_t le = __ballot(lane < num_reqs && w <= L);
  return __builtin_amdgcn_readfirstlane(__popcll(le) - 1);
}

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS operations (lgkmcnt 0), not for its vector-memory operations,
// so DMA and global loads in flight stay in flight (__syncthreads would
// wait for them too).  The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations (loads,
// stores, LDS DMA) are outstanding; the counter retires in issue order, so
// every older operation has completed.  gfx9 encoding: vmcnt bits [3:0] and
// [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// ---------------------------------------------------------------- waves
// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) with gfx950's VALU lane swaps instead of LDS permutes: with both
// operands equal to x, v_permlane16_swap returns {x[l], x[l^16]} and
// v_permlane32_swap returns {x[l], x[l^32]} across its two results.
__device__ __forceinline__ float wave_max_16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reductions over lanes l and l^32 (one v_permlane32_swap).
__device__ __forceinline__ float half_max_32(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float half_sum_32(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Physical workgroup -> logical workgroup so that each XCD (8 per MI355X,
// dispatched round robin) runs a contiguous slice of the logical order; the
// workgroups that share K/V tiles then share one XCD's L2.
__device__ __forceinline__ int xcd_logical(int p, int grid) {
  const int per = grid >> 3;  // grid is a multiple of 8
  return (p & 7) * per + (p >> 3);
}

// ---------------------------------------------------------------- params
struct ExtractDoc {
  int64_t row0;      // first packed row of the document in the batch
  int32_t n, m;      // document tokens, slots
  int32_t wg0;       // first logical workgroup of the document
  int32_t nwg_doc;   // workgroups per KV head over document rows
  int32_t nwg_slot;  // workgroups per KV head over slot rows
  int32_t pad;
};

struct ExtractParams {
  const void* q;        // [rows][hq][D]   pre-RoPE
  const void* krot;     // [rows][hkv][D]  rotated keys (workspace)
  const void* v;        // [rows][hkv][D] values (input)
  void* o;              // [rows][hq][D]
  float* lse;           // [hq][rows] or null
  const float2* rope;   // [max_n][D/2] (cos, sin)
  uint64_t* counts;     // mask-count mode: 5 counters; tile-dump mode: [0] entries found
  c2kv_tile_entry* entries;  // tile-dump mode: output table
  int64_t entry_cap;    // tile-dump mode: entries that fit
  int64_t total_rows;
  int32_t num_docs, hq, hkv, G, ratio_k, sink_len;
  int32_t total_wg, grid_wg;
  float scale_log2;
  int32_t anchor;       // 1: the anchor-token ablation's mask (documents <-> slots both ways)
  int32_t doc_base;     // index of docs[0] in the caller's document list
  ExtractDoc docs[C2KV_MAX_BATCH];
};

struct CacheReq {
  int32_t wg0;       // first logical workgroup of the request
  int32_t cache_len; // rows before the appended question
  int32_t nsplit;    // key chunks
  int32_t pbase;     // first split partial of the request (when nsplit > 1)
  int32_t pos0;      // position of the first question token
};

// Split partials of a launch are compact: request ri's partial of (head,
// token t, split) has index pbase[ri] + (head * tq + t) * nsplit[ri] + split,
// with its unnormalised o in part_o[index][D] and its (running max m in the
// log2 domain, sum l) in part_ml[index], so the (m, l) pairs of one output
// row are contiguous.
struct CacheParams {
  const void* q;        // [R][tq][hq][D] pre-RoPE question queries
  const void* k_new;    // [R][tq][hkv][D] pre-RoPE question keys
  const void* v_new;    // [R][tq][hkv][D]
  void* kc;             // [R][hkv][cap][D]
  void* vc;
  void* o;              // [R][tq][hq][D]
  float* lse;           // [R][hq][tq] or null
  float* part_o;        // split partials: o
  float2* part_ml;      // split partials: (m, l)
  int64_t cap;
  int32_t req0;         // first request of this launch (global index)
  int32_t num_reqs, tq, hq, hkv, G, nblk_q, nug, chunk;
  int32_t total_wg, grid_wg;
  float scale_log2;
  RopeFreqs freqs;
  CacheReq reqs[C2KV_MAX_BATCH];
};

struct DecodeReq {
  int32_t wg0;       // first workgroup of the request
  int32_t cache_len; // rows before the new token (its row)
  int32_t pos;       // position of the new token
  int32_t nsplit;    // key pieces of the request
  int32_t chunk;     // keys per piece (a multiple of 32)
  int32_t pbase;     // first split partial of the request (when nsplit > 1)
};

struct DecodeParams {
  const void* q;        // [R][hq][D] pre-RoPE
  const void* k_new;    // [R][hkv][D] pre-RoPE
  const void* v_new;
  void* kc;             // [R][hkv][cap][D]
  void* vc;
  void* o;              // [R][hq][D]
  float* lse;           // [R][hq] or null
  float* part_o;        // split partials (see CacheParams)
  float2* part_ml;
  int64_t cap;
  int32_t req0, num_reqs, hq, hkv, G, total_wg;
  float scale_log2;
  RopeFreqs freqs;
  DecodeReq reqs[C2KV_MAX_BATCH];
};

struct MergeParams {
  const float* part_o;
  const float2* part_ml;
  void* o;              // [R][tq][hq][D]
  float* lse;           // [R][hq][tq] or null
  int32_t req0, num_rows, hq, tq;
  int32_t nsplit[C2KV_MAX_BATCH];
  int32_t pbase[C2KV_MAX_BATCH];
};

}  // namespace c2kv
