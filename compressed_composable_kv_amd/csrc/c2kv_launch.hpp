// Host-side launchers of the C2KV kernels (defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "c2kv_device.hpp"

namespace c2kv {

// Document table of the K pre-rotation kernel.
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

// Compose launch table (kernel arguments, no device-side table): the
// distinct documents of the launch once, each occurrence of a document in a
// request as a one-byte index, and "runs" -- maximal sequences of
// consecutive segments of one request that go to the launch.  The kernel
// rebuilds every occurrence's cache row and position offset with prefix
// sums over the occurrences (cache rows and positions advance by each
// document's slot count and original length within a run) and groups the
// occurrences by document.  total_units is the launch's work units (an
// upper bound is enough: it sizes the grid).
struct ComposeDoc {
  const void* k;
  const void* v;
  int32_t stride;      // elements between slot rows
  int32_t n;           // original document length
};
constexpr int kComposeDocs = 64;     // distinct documents per launch
constexpr int kComposeOcc = 1024;    // document occurrences per launch
constexpr int kComposeRuns = 64;     // runs per launch
constexpr int kComposeNoRealign = 0x80;   // occurrence flag: keep extraction positions (offset = pos_base)
constexpr int kComposeHPT = 2;       // KV heads per thread
constexpr int kComposeGroup = 4;     // occurrences of one document written per work unit

struct ComposeParams {
  void* cache_k;
  void* cache_v;
  int32_t* pos_out;
  int64_t cap;
  int32_t num_docs, num_occ, num_runs, hkv, ratio_k, total_units;
  int32_t rpt, gpb, nblk;   // rows per tile, head pairs per unit, units per tile (ComposeTiling)
  RopeFreqs freqs;
  ComposeDoc docs[kComposeDocs];
  int32_t run_req[kComposeRuns];    // request of the run
  int32_t run_row0[kComposeRuns];   // cache row of the run's first occurrence
  int32_t run_pos0[kComposeRuns];   // realigned position offset of the run's first occurrence
  int32_t run_base[kComposeRuns];   // pos_base of the run's request (offset without realignment)
  uint16_t run_occ0[kComposeRuns + 1];   // first occurrence of each run; [num_runs] = num_occ
  alignas(4) uint8_t occ_doc[kComposeOcc];   // document index | kComposeNoRealign
};
static_assert(sizeof(ComposeParams) <= 4096, "compose table must fit the kernel arguments");

// Tiling of compose_kernel.  A workgroup of 256 threads covers a unit: rpt
// composed rows times gpb pairs of KV heads, each thread one 16-byte chunk
// of the low half of a row (and the matching chunk of the high half) for a
// pair.  gpb is the number of head pairs rounded up to a power of two, capped
// by the threads, so that a unit reads whole source rows (all heads of a
// slot are contiguous) where the threads allow; a tile of rows then takes
// nblk units.
struct ComposeTiling {
  int rpt, gpb, nblk;
};
inline ComposeTiling compose_tiling(int dtype_bytes, int head_dim, int hkv) {
  const int tph = head_dim / 2 * dtype_bytes / 16;   // threads per half row
  const int pairs = (hkv + 1) / 2;
  int gp = 1;
  while (gp < pairs) gp <<= 1;
  const int gpb = gp < 256 / tph ? gp : 256 / tph;
  return ComposeTiling{256 / tph / gpb, gpb, (pairs + gpb - 1) / gpb};
}


// Extractor layer GEMM C = A * B^T (bf16, fp32 accumulation).  A row range
// of A uses weights b0 (sel 0) or b1 (sel 1); tile0 is its first 128-row
// tile.  Epilogues: kEpiStore splits columns [0, n1) to c0, [n1, n2) to c1,
// [n2, N) to c2 (each boundary a multiple of 128); kEpiResidual writes
// C = r + A * B^T to c0; kEpiSwiglu takes weight rows in blocks of 16 gate
// rows then the matching 16 up rows and writes silu(gate) * up to c0
// ([rows][N / 2]).
constexpr int kEpiStore = 0, kEpiResidual = 1, kEpiSwiglu = 2;
struct GemmRange {
  int32_t row0, rows, sel, tile0;
};
constexpr int kGemmRanges = 128;   // two per document of a 64-document chunk
struct GemmParams {
  const bf16* a;
  const bf16* b0;
  const bf16* b1;
  bf16* c0;
  bf16* c1;
  bf16* c2;
  const bf16* r;
  int64_t lda, ldc0, ldc1, ldc2, ldr;
  int32_t K, N, n1, n2, num_ranges, m_tiles, n_tiles, pad;
  GemmRange ranges[kGemmRanges];
};
static_assert(sizeof(GemmParams) <= 4096, "gemm table must fit the kernel arguments");

struct SlotFillDoc {
  int64_t row0;    // first slot row of the document
  int32_t slot0;   // index of its first slot within the launch
  int32_t pad;
};
struct SlotFillParams {
  void* x;
  const void* embed;
  int32_t dm, num_docs;
  SlotFillDoc docs[C2KV_MAX_BATCH];
};

hipError_t launch_rope_table(float2* table, int npos, int head_dim, const RopeFreqs& f, hipStream_t st);
hipError_t launch_rotate_k(const RotateParams& p, int dtype, int head_dim, hipStream_t st);
constexpr int kExtractAttn = 0, kExtractCount = 1, kExtractDump = 2;   // launch_extract_attn modes
hipError_t launch_extract_attn(const ExtractParams& p, int dtype, int head_dim, int mode, hipStream_t st);
hipError_t launch_prefill_attn(const CacheParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_decode_attn(const DecodeParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t st);
hipError_t launch_compose(const ComposeParams& p, int dtype, int head_dim, bool host_src, hipStream_t st);
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t st);
hipError_t launch_gemm(const GemmParams& p, int epi, hipStream_t st);
hipError_t launch_rms_norm(const void* x, const void* gamma, void* h, int64_t rows, int dm, float eps,
                           hipStream_t st);
hipError_t launch_slot_fill(const SlotFillParams& p, int slots, hipStream_t st);

}  // namespace c2kv
