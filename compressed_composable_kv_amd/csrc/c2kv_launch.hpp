// Host-side launchers of the C2KV kernels (defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "c2kv_device.hpp"

namespace c2kv {

// Document table of the K pre-rotation and V transpose kernels.
struct RotDoc {
  int64_t row0;
  int32_t n, m;
};
struct RotateParams {
  const void* k;
  void* krot;
  const float2* rope;
  int64_t row_begin, row_end;   // packed rows covered by this launch
  int32_t num_docs, hkv, ratio_k, pad;
  RotDoc docs[C2KV_MAX_BATCH];
};

// One document segment of a compose launch (passed as a kernel argument).
struct ComposeSeg {
  const void* k;
  const void* v;
  int32_t stride;      // elements between slot rows
  int32_t n;           // original document length
  int32_t req;         // request index
  int32_t out_row;     // first cache row of this segment
  int32_t pos_off;     // position offset of the document
  int32_t tile0;       // first row tile of this segment within the launch
};
constexpr int kComposeSegs = 64;   // segments per launch (kernel-argument table)
constexpr int kComposeHPT = 2;     // KV heads per thread

struct ComposeParams {
  void* cache_k;
  void* cache_v;
  int32_t* pos_out;
  int64_t cap;
  int32_t num_segs, hkv, ratio_k, total_tiles;
  RopeFreqs freqs;
  ComposeSeg segs[kComposeSegs];
};
static_assert(sizeof(ComposeParams) <= 4096, "compose table must fit the kernel arguments");

// Composed rows per row tile of compose_kernel (one workgroup of 256 threads
// covers a tile of rows, each thread one 16-byte chunk of a half row).
inline int compose_rows_per_tile(int dtype_bytes, int head_dim) {
  return 256 / (head_dim / 2 * dtype_bytes / 16);
}

struct AppendReq {
  int32_t cache_len, pos0;
};
struct AppendParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* qrot;
  void* cache_k;
  void* cache_v;
  int64_t cap;
  int32_t req0, num_reqs, tq, hq, hkv, pad;
  RopeFreqs freqs;
  AppendReq reqs[C2KV_MAX_BATCH];
};

hipError_t launch_rope_table(float2* table, int npos, int head_dim, const RopeFreqs& f, hipStream_t st);
hipError_t launch_rotate_k(const RotateParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_extract_attn(const ExtractParams& p, int dtype, int head_dim, bool count, hipStream_t st);
hipError_t launch_cache_attn(const CacheParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_decode_attn(const DecodeParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_compose(const ComposeParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_append(const AppendParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t st);

}  // namespace c2kv
