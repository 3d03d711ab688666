// Bandwidth-bound kernels of the C2KV hot path for gfx950:
//   * RoPE cos/sin table and key pre-rotation for extraction,
//   * compose: realigned RoPE of the stored pre-RoPE slot keys fused with the
//     scatter of keys and values into the contiguous per-request cache (the
//     C2KV explainer's positions section: every document keeps its original
//     length in positions, later documents are offset by the lengths before
//     them, slot j sits at its block's last token),
//   * a zero-fill kernel for workspaces.
//
// Every RoPE'd element pair (x_i, x_{i+d/2}) is handled by one thread that
// reads both halves with 16-byte loads, so rotation needs no data exchange;
// a thread covers one 16-byte chunk of each half.
#include "c2kv_device.hpp"
#include "c2kv_launch.hpp"

namespace c2kv {

// ------------------------------------------------------------ RoPE table
__global__ void rope_table_kernel(float2* table, int npos, int half, const RopeFreqs f) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)npos * half) return;
  const int pos = (int)(idx / half), i = (int)(idx % half);
  float c, s;
  rope_cs(pos, f.f[i], c, s);
  table[idx] = make_float2(c, s);
}

hipError_t launch_rope_table(float2* table, int npos, int head_dim, const RopeFreqs& f, hipStream_t st) {
  const int half = head_dim / 2;
  const int64_t n = (int64_t)npos * half;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, st, table, npos, half, f);
  return hipGetLastError();
}

// ------------------------------------------------ extraction key rotation
template <typename T, int D>
__global__ void rotate_k_kernel(const RotateParams p) {
  constexpr int CE = Chunk<T>::CE, H = D / 2, TPH = H / CE;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)p.hkv * TPH;
  const int64_t row = p.row_begin + idx / per_row;
  if (row >= p.row_end) return;
  const int h = (int)((idx % per_row) / TPH), c = (int)(idx % TPH);
  // the row's document: when every wave lies in one row (a multiple of 64
  // threads per row), one lane-indexed load of the 64-entry table and a
  // ballot; otherwise a binary search over the documents' first rows
  int b;
  if (per_row % 64 == 0) {
    static_assert(C2KV_MAX_BATCH == 64, "one table entry per lane");
    const int lane = threadIdx.x & 63;
    const int64_t r0 = p.docs[lane].row0;   // entries past num_docs are masked
    b = (int)__popcll(__ballot(lane < p.num_docs && r0 <= row)) - 1;
  } else {
    int lo = 0, hi = p.num_docs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.docs[mid].row0 <= row) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
  }
  const int local = (int)(row - p.docs[b].row0);
  const int n = p.docs[b].n;
  const int pos = local < n ? local : min((local - n) * p.ratio_k + p.ratio_k - 1, n - 1);
  const int64_t off = (row * p.hkv + h) * D + c * CE;
  const T* src = reinterpret_cast<const T*>(p.k) + off;
  T* dst = reinterpret_cast<T*>(p.krot) + off;
  uint4 lo = *reinterpret_cast<const uint4*>(src);
  uint4 hi = *reinterpret_cast<const uint4*>(src + H);
  float cs[CE], sn[CE];
#pragma unroll
  for (int e = 0; e < CE; ++e) {
    const float2 t = p.rope[(int64_t)pos * H + c * CE + e];
    cs[e] = t.x;
    sn[e] = t.y;
  }
  rotate_chunk<T>(lo, hi, cs, sn);
  *reinterpret_cast<uint4*>(dst) = lo;
  *reinterpret_cast<uint4*>(dst + H) = hi;
}

template <typename T, int D>
static hipError_t launch_rotate_k_t(const RotateParams& p, hipStream_t st) {
  constexpr int TPH = D / 2 / Chunk<T>::CE;
  const int64_t n = (p.row_end - p.row_begin) * p.hkv * TPH;
  const int blocks = (int)((n + 255) / 256);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((rotate_k_kernel<T, D>), dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_rotate_k(const RotateParams& p, int dtype, int head_dim, hipStream_t st) {
  if (dtype == C2KV_BF16) return head_dim == 128 ? launch_rotate_k_t<bf16, 128>(p, st) : launch_rotate_k_t<bf16, 64>(p, st);
  return head_dim == 128 ? launch_rotate_k_t<float, 128>(p, st) : launch_rotate_k_t<float, 64>(p, st);
}

// ---------------------------------------------------------------- compose
// Work unit = (row tile of one DOCUMENT of the launch, block of gpb pairs of
// KV heads (see ComposeTiling), group of up to kComposeGroup occurrences of
// that document).  A thread owns one 16-byte chunk of the low half of a row
// (and the matching chunk of the high half) of one head pair: it loads the
// document's pre-RoPE rows once and, for every occurrence of the group,
// rotates the keys at that occurrence's realigned positions and writes keys
// and values to that occurrence's cache rows.  A document reused by several
// requests is therefore read once per group instead of once per request,
// and the cache writes dominate the traffic.  Consecutive threads take the
// chunks, then the head pairs, then the rows, so a unit reads whole source
// rows.  Each workgroup first rebuilds the launch's tables in LDS (cache row
// and position offset of every occurrence by prefix sums over the runs; the
// occurrences of each document; the units of each document); a unit finds
// its document by a binary search over the documents' first units.  The
// realigned position of slot j of an occurrence is the occurrence's offset
// plus the slot's extraction position.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ void store_nt(T* dst, const uint4& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(dst));
}

struct ComposeTable {
  int row[kComposeOcc];         // cache row of the occurrence's slot 0
  int pos[kComposeOcc];         // position offset of the occurrence
  int req[kComposeOcc];         // request (global index)
  long long scan_n[kComposeOcc];   // global exclusive prefix of original lengths
  int scan_m[kComposeOcc];         // global exclusive prefix of slot counts
  short by_doc[kComposeOcc];    // occurrences grouped by document, in occurrence order
  short rank[kComposeOcc];      // rank of the occurrence among those of its document
  unsigned char occ[kComposeOcc];   // copy of the launch table's occurrence bytes
  int doc_n[kComposeDocs];          // copies of the launch table's small arrays
  int run_occ0[kComposeRuns + 1], run_row0[kComposeRuns], run_pos0[kComposeRuns], run_base[kComposeRuns];
  int run_req[kComposeRuns];
  int doc_occ0[kComposeDocs + 1];   // first entry of each document in by_doc
  int doc_unit0[kComposeDocs + 1];  // first unit of each document; [num_docs] = total units
  int doc_cnt[kComposeDocs];        // occurrences of each document
  int rank_cnt[kComposeDocs];       // running counts of the ranking pass
  long long wsum_n[4];
  int wsum_m[4];
};

// Inclusive scan over the 64 lanes of a wave.
template <typename X>
__device__ __forceinline__ X wave_incl_scan(X x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const X y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// The table is built in two phases.  Phase A (the launch table into LDS,
// each document's occurrence count by an LDS histogram, and each document's
// first occurrence entry and first unit) is all a unit needs to find its
// document and load its rows; phase B (the stable grouping of occurrences
// by document, and each occurrence's cache row, position offset and
// request) is needed only to store.  The kernel issues its first unit's
// loads between the two, so phase B runs while they are in flight.
__device__ void compose_table_a(const ComposeParams& p, ComposeTable& tb) {
  constexpr int PER = kComposeOcc / 256;   // occurrences per thread
  static_assert(PER == 4, "one 32-bit word of occurrence bytes per thread");
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // one round of independent loads of the launch table (kernel arguments),
  // all issued before any is used: indices are clamped so that no load
  // waits behind a branch on another one
  const int td = min(t, kComposeDocs - 1), tr = min(t, kComposeRuns - 1);
  const int ld_n = p.docs[td].n;
  const int ld_occ0 = p.run_occ0[min(t, kComposeRuns)];
  const int ld_row0 = p.run_row0[tr], ld_pos0 = p.run_pos0[tr], ld_base = p.run_base[tr], ld_req = p.run_req[tr];
  const uint32_t ld_occ = *reinterpret_cast<const uint32_t*>(&p.occ_doc[PER * min(t, kComposeOcc / PER - 1)]);
  const int num_docs = p.num_docs, num_runs = p.num_runs, num_occ = p.num_occ;
  // (the empty asm makes every load above complete here, in one wait,
  // instead of each being sunk into the branch that stores it)
  asm volatile("" : : "v"(ld_n), "v"(ld_occ0), "v"(ld_row0), "v"(ld_pos0), "v"(ld_base), "v"(ld_req), "v"(ld_occ),
               "s"(num_docs), "s"(num_runs), "s"(num_occ));
  if (t < kComposeDocs) {
    tb.doc_cnt[t] = 0;
    tb.rank_cnt[t] = 0;
    if (t < num_docs) tb.doc_n[t] = ld_n;
  }
  if (t <= num_runs) tb.run_occ0[t] = ld_occ0;
  if (t < num_runs) {
    tb.run_row0[t] = ld_row0;
    tb.run_pos0[t] = ld_pos0;
    tb.run_base[t] = ld_base;
    tb.run_req[t] = ld_req;
  }
  if (PER * t < num_occ) *reinterpret_cast<uint32_t*>(&tb.occ[PER * t]) = ld_occ;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (PER * t + i < num_occ) atomicAdd(&tb.doc_cnt[(ld_occ >> (8 * i)) & (kComposeNoRealign - 1)], 1);
  __syncthreads();
  // per document (one per lane of wave 0): first by_doc entry and first unit
  static_assert(kComposeDocs == 64, "one wave covers the documents");
  if (wave == 0) {
    int c = 0, nu = 0;
    if (lane < num_docs) {
      const int m = (tb.doc_n[lane] + p.ratio_k - 1) / p.ratio_k;
      c = tb.doc_cnt[lane];
      nu = ((m + p.rpt - 1) / p.rpt) * p.nblk * ((c + kComposeGroup - 1) / kComposeGroup);
    }
    const int ic = wave_incl_scan(c), iu = wave_incl_scan(nu);
    if (lane < num_docs) {
      tb.doc_occ0[lane] = ic - c;
      tb.doc_unit0[lane] = iu - nu;
    }
    if (lane == 63) {
      tb.doc_occ0[num_docs] = ic;
      tb.doc_unit0[num_docs] = iu;
    }
  }
  __syncthreads();
}

// (its barriers order LDS only, so the first unit's loads stay in flight)
__device__ void compose_table_b(const ComposeParams& p, ComposeTable& tb) {
  constexpr int PER = kComposeOcc / 256;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int ml[PER], rl[PER], dl[PER];
  long long nl[PER];
  int sm = 0;
  long long sn = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int o = PER * t + i;
    ml[i] = 0;
    nl[i] = 0;
    rl[i] = 0;
    dl[i] = 0;
    if (o < p.num_occ) {
      dl[i] = tb.occ[o] & (kComposeNoRealign - 1);
      const int n = tb.doc_n[dl[i]];
      ml[i] = (n + p.ratio_k - 1) / p.ratio_k;
      nl[i] = n;
      int lo = 0, hi = p.num_runs - 1;          // run of the occurrence
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tb.run_occ0[mid] <= o) lo = mid; else hi = mid - 1;
      }
      rl[i] = lo;
    }
    sm += ml[i];
    sn += nl[i];
  }
  // exclusive prefixes of the per-thread sums across the workgroup
  const int im = wave_incl_scan(sm);
  const long long in_ = wave_incl_scan(sn);
  if (lane == 63) { tb.wsum_m[wave] = im; tb.wsum_n[wave] = in_; }
  lds_barrier();
  int bm = im - sm;
  long long bn = in_ - sn;
  for (int w = 0; w < wave; ++w) { bm += tb.wsum_m[w]; bn += tb.wsum_n[w]; }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int o = PER * t + i;
    if (o < p.num_occ) {
      tb.scan_m[o] = bm;
      tb.scan_n[o] = bn;
    }
    bm += ml[i];
    bn += nl[i];
  }
  // stable rank of every occurrence among those of its document, so that
  // every workgroup groups the occurrences identically: wave 0 walks them 64
  // at a time; lanes holding the same document find each other by comparing
  // the document index bit by bit through ballots, and the highest such lane
  // advances the document's running count
  if (wave == 0) {
    for (int c0 = 0; c0 < p.num_occ; c0 += 64) {
      const int o = c0 + lane;
      const bool valid = o < p.num_occ;
      const int dd = valid ? (tb.occ[o] & (kComposeNoRealign - 1)) : kComposeNoRealign - 1;
      uint64_t same = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 7; ++b) {
        const bool bit = (dd >> b) & 1;
        const uint64_t mb = __ballot(bit);
        same &= bit ? mb : ~mb;
      }
      const int below = __popcll(same & ((1ull << lane) - 1));
      const int base = valid ? tb.rank_cnt[dd] : 0;
      __builtin_amdgcn_wave_barrier();   // every lane has read its base before any lane updates it
      if (valid) {
        tb.rank[o] = (short)(base + below);
        if ((same >> lane) == 1ull) tb.rank_cnt[dd] = base + __popcll(same);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  lds_barrier();
  // cache rows and position offsets relative to the start of each run; the
  // occurrence lists of the documents
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int o = PER * t + i;
    if (o < p.num_occ) {
      const int r = rl[i], f = tb.run_occ0[r];
      tb.row[o] = tb.run_row0[r] + (tb.scan_m[o] - tb.scan_m[f]);
      tb.pos[o] = (tb.occ[o] & kComposeNoRealign) ? tb.run_base[r]
                                                 : tb.run_pos0[r] + (int)(tb.scan_n[o] - tb.scan_n[f]);
      tb.req[o] = tb.run_req[r];
      tb.by_doc[tb.doc_occ0[dl[i]] + tb.rank[o]] = (short)o;
    }
  }
  lds_barrier();
}

template <typename T, int D>
struct ComposeUnit {
  static constexpr int CE = Chunk<T>::CE, H = D / 2, TPH = H / CE;
  uint4 kl0, kh0, vl0, vh0, kl1, kh1, vl1, vh1;
  float fr[CE];
  int doc, g0, g1, j, c, h0, spos;
  bool live;

  __device__ __forceinline__ void load(const ComposeParams& p, const ComposeTable& tb, int u) {
    const int t = (int)threadIdx.x;
    int lo = 0, hi = p.num_docs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tb.doc_unit0[mid] <= u) lo = mid; else hi = mid - 1;
    }
    doc = __builtin_amdgcn_readfirstlane(lo);   // uniform: every lane searched for the same unit
    const ComposeDoc& dc = p.docs[doc];
    const int m = (dc.n + p.ratio_k - 1) / p.ratio_k;
    const int cnt = tb.doc_cnt[doc];
    const int ngrp = (cnt + kComposeGroup - 1) / kComposeGroup;
    const int local = u - tb.doc_unit0[doc];
    const int grp = local % ngrp, rest = local / ngrp;   // groups of one tile run back to back
    const int tile = rest / p.nblk, blk = rest % p.nblk;
    g0 = tb.doc_occ0[doc] + grp * kComposeGroup;
    g1 = min(g0 + kComposeGroup, tb.doc_occ0[doc] + cnt);
    const int hgrp = blk * p.gpb + (t / TPH) % p.gpb;
    j = tile * p.rpt + t / (TPH * p.gpb);
    c = t % TPH;
    live = j < m && 2 * hgrp < p.hkv;   // padded head pairs load a valid head and store nothing
    const int jj = live ? j : m - 1;     // dead lanes load a valid row
    spos = min(jj * p.ratio_k + p.ratio_k - 1, dc.n - 1);
#pragma unroll
    for (int e = 0; e < CE; e += 4) {
      const f32x4 f4 = *reinterpret_cast<const f32x4*>(&p.freqs.f[c * CE + e]);
      fr[e] = f4[0]; fr[e + 1] = f4[1]; fr[e + 2] = f4[2]; fr[e + 3] = f4[3];
    }
    const T* ksrc = reinterpret_cast<const T*>(dc.k) + (int64_t)jj * dc.stride + c * CE;
    const T* vsrc = reinterpret_cast<const T*>(dc.v) + (int64_t)jj * dc.stride + c * CE;
    h0 = min(hgrp * 2, p.hkv - 1);
    const int h1 = min(h0 + 1, p.hkv - 1);
    kl0 = *reinterpret_cast<const uint4*>(ksrc + h0 * D);
    kh0 = *reinterpret_cast<const uint4*>(ksrc + h0 * D + H);
    vl0 = *reinterpret_cast<const uint4*>(vsrc + h0 * D);
    vh0 = *reinterpret_cast<const uint4*>(vsrc + h0 * D + H);
    kl1 = *reinterpret_cast<const uint4*>(ksrc + h1 * D);
    kh1 = *reinterpret_cast<const uint4*>(ksrc + h1 * D + H);
    vl1 = *reinterpret_cast<const uint4*>(vsrc + h1 * D);
    vh1 = *reinterpret_cast<const uint4*>(vsrc + h1 * D + H);
  }

  __device__ __forceinline__ void store(const ComposeParams& p, const ComposeTable& tb) {
    if (!live) return;
    for (int gi = g0; gi < g1; ++gi) {
      const int o = tb.by_doc[gi];
      const int req = tb.req[o], row0 = tb.row[o];
      const int cpos = tb.pos[o] + spos;
      float cs[CE], sn[CE];
#pragma unroll
      for (int e = 0; e < CE; ++e) rope_cs(cpos, fr[e], cs[e], sn[e]);
      auto put = [&](int h, uint4 kl, uint4 kh, const uint4& vl, const uint4& vh) {
        rotate_chunk<T>(kl, kh, cs, sn);
        const int64_t dst = (((int64_t)req * p.hkv + h) * p.cap + row0 + j) * D + c * CE;
        T* kd = reinterpret_cast<T*>(p.cache_k) + dst;
        T* vd = reinterpret_cast<T*>(p.cache_v) + dst;
        // the composed cache is written once and read by later calls:
        // streaming (non-temporal) stores
        store_nt(kd, kl);
        store_nt(kd + H, kh);
        store_nt(vd, vl);
        store_nt(vd + H, vh);
      };
      put(h0, kl0, kh0, vl0, vh0);
      if (h0 + 1 < p.hkv) put(h0 + 1, kl1, kh1, vl1, vh1);
      if (p.pos_out && h0 == 0 && c == 0) p.pos_out[(int64_t)req * p.cap + row0 + j] = cpos;
    }
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256, 4) void compose_kernel(const ComposeParams p) {
  static_assert(kComposeHPT == 2, "two heads per thread");
  __shared__ ComposeTable tb;
  // the scalar kernel-argument fields, loaded in one round: the empty asm
  // needs them all at once, so they complete at one wait instead of one
  // dependent round per use (the table's per-lane loads follow separately)
  const int total_units = p.total_units, num_docs = p.num_docs, num_occ = p.num_occ, num_runs = p.num_runs;
  const int hkv = p.hkv, ratio_k = p.ratio_k, rpt = p.rpt, gpb = p.gpb, nblk = p.nblk;
  const int64_t cap = p.cap;
  void* const ck = p.cache_k;
  void* const cv = p.cache_v;
  int32_t* const pos_out = p.pos_out;
  asm volatile("" : : "s"(total_units), "s"(num_docs), "s"(num_occ), "s"(num_runs), "s"(hkv), "s"(ratio_k),
               "s"(rpt), "s"(gpb), "s"(nblk), "s"(cap), "s"(ck), "s"(cv), "s"(pos_out));
  int u = blockIdx.x;
  if (u >= total_units) return;
  compose_table_a(p, tb);
  const int total = tb.doc_unit0[p.num_docs];
  // one unit in flight per wave: a unit's loads are amortised over the
  // stores of its whole occurrence group, and four workgroups per CU keep
  // other waves' loads in flight meanwhile.  The first unit's loads are
  // issued before the second phase of the table, which runs under them.
  ComposeUnit<T, D> cur;
  cur.load(p, tb, u);
  compose_table_b(p, tb);
  for (;;) {
    cur.store(p, tb);
    u += gridDim.x;
    if (u >= total) break;
    cur.load(p, tb, u);
  }
}

template <typename T, int D>
static hipError_t launch_compose_t(const ComposeParams& p, bool host_src, hipStream_t st) {
  const int units = p.total_units;
  if (units == 0) return hipSuccess;
  // device sources: four workgroups per CU (16 waves).  Measured on one
  // MI355X: the Qwen2.5 pool (about 6900 units) 101.3-101.6 us against
  // 102.6-104.1 at three and 105-106 at two; the Llama layer (1024 units)
  // 16.6-16.8 us at three or four, 18.6 at two.  Host sources: 16 workgroups (about 1 MB in flight) keep the
  // host link busy; more concurrent readers made its transfers slower
  // (56 GB/s at 12-16 workgroups, 48 GB/s at 192 or more).
  const int blocks = min(units, host_src ? 16 : 4 * 256);
  hipLaunchKernelGGL((compose_kernel<T, D>), dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_compose(const ComposeParams& p, int dtype, int head_dim, bool host_src, hipStream_t st) {
  if (dtype == C2KV_BF16)
    return head_dim == 128 ? launch_compose_t<bf16, 128>(p, host_src, st) : launch_compose_t<bf16, 64>(p, host_src, st);
  return head_dim == 128 ? launch_compose_t<float, 128>(p, host_src, st) : launch_compose_t<float, 64>(p, host_src, st);
}

// --------------------------------------------------------------- zero fill
__global__ void fill_zero_kernel(uint32_t* p, int64_t nwords) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) p[i] = 0u;
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t st) {
  const int64_t nwords = (int64_t)(bytes / 4);
  if (nwords == 0) return hipSuccess;
  const int64_t want = (nwords + 255) / 256;
  const int blocks = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<uint32_t*>(ptr), nwords);
  return hipGetLastError();
}

}  // namespace c2kv
