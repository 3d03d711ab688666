// MFMA flash-attention kernels of the C2KV hot path for gfx950:
//   * extraction attention under the structured-flow mask (the C2KV
//     explainer's "structured information flow" section: documents causal and
//     blind to slots; slot j sees the sink block, its own k-token block and
//     the slots up to itself), enumerating only tiles that hold a visible
//     cell for some wave of the workgroup;
//   * the same enumeration in a counting mode (test support);
//   * split-K attention of question tokens over a composed cache (the
//     explainer's "overall flow" section), writing final rows when a request
//     has one key chunk and log-sum-exp partials for merge_kernel otherwise.
//
// Tile shapes.  A workgroup is 4 waves; each wave owns one "unit" = 32 query
// rows of one query head, and all units of a workgroup share one KV head, so
// the K/V tiles staged in LDS (64 keys, double buffered) serve every wave.
// S^T = K Q^T puts keys on the M side and queries on the N side, so each
// lane's accumulators belong to ONE query and the O^T rescale is a per-lane
// scalar; P^T goes straight from the S^T accumulators into the B operand of
// O^T += V^T P^T.  Two tiles:
//   * XAttn32 (bf16 extraction): v_mfma_f32_32x32x16_bf16, one query per
//     lane, row statistics in one lane swap;
//   * XAttn (fp32 extraction, prefill): v_mfma_f32_16x16x32_bf16 (fp32:
//     16x16x4 steps), two 16-query blocks per wave, row statistics in two
//     lane swaps.
// K and V tiles arrive row-major by LDS DMA (K from the rotated-key
// workspace or the cache, V from the input or the cache), and the V^T
// operand is read with transposing LDS reads.
#include "c2kv_device.hpp"
#include "c2kv_launch.hpp"

namespace c2kv {

// ------------------------------------------------------ visibility rules
// One branch-free formula covers every rule on this path:
//   visible(q, c) = c < kmax && (c <= q + a || (b > 0 && q b <= c < q b + b) || c < sink)
//   document row q, document key c:  a = 0                      (causal)
//   slot j, document key c:          a = -2^30, b = k, sink     (sink block + own block)
//   slot j, slot key j':             a = 0                      (causal)
//   cache query t, cache row c:      a = cache_len              (all cached rows + causal new rows)
//   anchor ablation, slot keys of a document row, any key of a slot row:
//                                    a = 2^30                   (every key below kmax)
struct Pred {
  int kmax, a, b, sink;
  __device__ __forceinline__ bool operator()(int q, int c) const {
    const int qb = q * b;
    const bool causal = c <= q + a;
    const bool own = (c >= qb) & (c < qb + b);
    return (c < kmax) & (causal | own | (c < sink));
  }
};
__host__ __device__ constexpr Pred pred_causal(int kmax, int offset) { return Pred{kmax, offset, 0, 0}; }
__host__ __device__ constexpr Pred pred_slot_doc(int n, int k, int sink) { return Pred{n, -(1 << 30), k, sink}; }

// Load 8 elements (one lane's k-group) of a row as fp32.
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float* out);
template <>
__device__ __forceinline__ void load8_f32<bf16>(const bf16* p, float* out) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = static_cast<float>(v[e]);
}
template <>
__device__ __forceinline__ void load8_f32<float>(const float* p, float* out) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[4 + e] = b[e]; }
}

// ===================================================== extraction kernel
struct ExtractPlan {
  int doc, kvh, slot_region, wvalid, head, q0, qend, anchor;
  int nA0, nA1, nB0, nB1, nS;        // doc tiles [nA0,nA1) u [nB0,nB1), slot tiles [0,nS)
  int64_t row0;
  int n, m, ratio_k, sink;
};

__device__ __forceinline__ ExtractPlan extract_plan(const ExtractParams& p, int L, int wave) {
  ExtractPlan P;
  const int b = request_of(p.docs, p.num_docs, L);
  const ExtractDoc& dc = p.docs[b];
  P.doc = b;
  P.row0 = dc.row0;
  P.n = dc.n;
  P.m = dc.m;
  P.ratio_k = p.ratio_k;
  P.sink = min(p.sink_len, dc.n);
  P.anchor = p.anchor;
  const int per = dc.nwg_doc + dc.nwg_slot;
  const int local = L - dc.wg0;
  P.kvh = local / per;
  int w = local % per;
  P.slot_region = w >= dc.nwg_doc;
  if (P.slot_region) w -= dc.nwg_doc;
  const int G = p.G;
  const int nrows = P.slot_region ? P.m : P.n;
  const int nblk = (nrows + kQW - 1) / kQW;
  const int nunits = nblk * G;
  auto unit_rows = [&](int u, int& q0, int& q1) {
    const int blk = P.slot_region ? u / G : nblk - 1 - u / G;
    q0 = blk * kQW;
    q1 = min(nrows, q0 + kQW);
  };
  const int u = w * kWaves + wave;
  P.wvalid = u < nunits;
  P.head = P.kvh * G + (u % G);
  P.q0 = 0;
  P.qend = 0;
  if (P.wvalid) unit_rows(u, P.q0, P.qend);
  // union of the waves' tile needs (identical in every wave)
  int tmax = 0, j0 = 1 << 30, j1 = 0;
  for (int ww = 0; ww < kWaves; ++ww) {
    const int uu = w * kWaves + ww;
    if (uu >= nunits) break;
    int a0, a1;
    unit_rows(uu, a0, a1);
    tmax = max(tmax, (a1 + kBN - 1) / kBN);
    j0 = min(j0, a0);
    j1 = max(j1, a1);
  }
  if (!P.slot_region) {
    P.nA0 = 0; P.nA1 = tmax; P.nB0 = 0; P.nB1 = 0;
    P.nS = P.anchor ? (P.m + kBN - 1) / kBN : 0;   // anchor ablation: documents also see every slot
  } else if (P.anchor) {
    // anchor ablation: slots see every document token and every slot
    P.nA0 = 0; P.nA1 = (P.n + kBN - 1) / kBN; P.nB0 = P.nB1 = P.nA1;
    P.nS = (P.m + kBN - 1) / kBN;
  } else {
    const int ts = (P.sink + kBN - 1) / kBN;
    const int blo = (j0 * P.ratio_k) / kBN;
    const int bhi = (min(P.n, j1 * P.ratio_k) + kBN - 1) / kBN;
    P.nA0 = 0; P.nA1 = ts;
    P.nB0 = max(ts, blo); P.nB1 = max(P.nB0, bhi);
    P.nS = tmax;
  }
  return P;
}

// Whether every cell of the document key tile [a, a + kBN) is visible to
// every slot row j in [q0, q1) (slot j sees the sink [0, s) and its own block
// [jk, min(n, jk + k))).  A row whose own block starts inside the sink
// (jk <= s) sees one interval [0, max(s, min(n, jk + k))), the smallest such
// row binding; a row whose block starts past the sink sees two separate
// intervals, so the tile must lie in that row's own block, which no two rows
// share.
__device__ __forceinline__ bool slot_doc_tile_full(int a, int n, int k, int s, int q0, int q1) {
  const int b = a + kBN;
  if (b > n) return false;
  if (b <= s) return true;
  const int jm = s / k + 1;                    // rows j < jm start inside the sink
  if (q0 < jm && b > max(s, min(n, q0 * k + k))) return false;
  const int sep0 = max(q0, jm);
  if (q1 - sep0 >= 2) return false;
  if (q1 - sep0 == 1 && (a < sep0 * k || b > min(n, sep0 * k + k))) return false;
  return true;
}

// Tile `it` of the plan: whether it holds a document or slot key range,
// its index, and the visibility predicate / activity of the calling wave.
struct TileSel {
  int is_slot, t, key0, nvalid, active, masked;
  Pred pred;
};

__device__ __forceinline__ TileSel extract_tile(const ExtractPlan& P, int it) {
  TileSel s;
  const int na = P.nA1 - P.nA0, nb = P.nB1 - P.nB0;
  s.is_slot = it >= na + nb;
  s.t = it < na ? P.nA0 + it : (it < na + nb ? P.nB0 + (it - na) : it - na - nb);
  s.key0 = s.t * kBN;
  const int nkeys = s.is_slot ? P.m : P.n;
  s.nvalid = min(kBN, nkeys - s.key0);
  if (P.anchor && (P.slot_region || s.is_slot)) {
    // anchor ablation: every key of the tile's range is visible
    s.active = P.wvalid;
    s.masked = s.key0 + kBN > nkeys;
    s.pred = pred_causal(nkeys, 1 << 30);
  } else if (!P.slot_region) {
    s.active = P.wvalid && s.key0 < P.qend;
    s.masked = (s.key0 + kBN - 1 > P.q0) || (s.key0 + kBN > P.n);
    s.pred = pred_causal(P.n, 0);
  } else if (!s.is_slot) {
    const int ts = (P.sink + kBN - 1) / kBN;
    const int blo = (P.q0 * P.ratio_k) / kBN;
    const int bhi = (min(P.n, P.qend * P.ratio_k) + kBN - 1) / kBN;
    s.active = P.wvalid && (s.t < ts || (s.t >= blo && s.t < bhi));
    s.masked = !slot_doc_tile_full(s.key0, P.n, P.ratio_k, P.sink, P.q0, P.qend);
    s.pred = pred_slot_doc(P.n, P.ratio_k, P.sink);
  } else {
    s.active = P.wvalid && s.key0 < P.qend;
    s.masked = (s.key0 + kBN - 1 > P.q0) || (s.key0 + kBN > P.m);
    s.pred = pred_causal(P.m, 0);
  }
  return s;
}

// ------------------------------------------------- row-major V tiles
// A V tile of 64 keys x D, row-major, filled by LDS DMA.  32-byte pairs of
// a row are XOR-swizzled with vr_swz(row) so that the transposed operand
// reads of a half wave (8 rows x 32 bytes) hit distinct banks.
template <int RB>
__device__ __forceinline__ int vr_swz(int row) {
  if constexpr (RB >= 256) return (row & 3) | (((row >> 3) & 1) << 2);
  else return ((row >> 1) & 1) | (((row >> 3) & 1) << 1);
}

typedef short pf_s4 __attribute__((ext_vector_type(4)));

// V^T operand of O^T += V^T P^T for half c and dims 16 db .. +15: lane
// (r16, g) gets dim 16 db + r16 of keys 32 c + 8 g + e, e = 0..7 (the key
// order of the P^T operand).  bf16: ds_read_b64_tr_b16, where within each
// 16 lanes output lane j element a is element j % 4 of the 4 values
// addressed by source lane 4a + j / 4; fp32: element reads.
template <typename T, int D>
__device__ __forceinline__ typename ElemTraits<T>::v8 vrow_operand(const char* vt, int c, int db, int r16, int g) {
  constexpr int RB = D * (int)sizeof(T);
  if constexpr (sizeof(T) == 2) {
    pf_s4 x[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * c + 8 * g + 4 * h + (r16 >> 2);
      const int off = row * RB + 32 * (db ^ vr_swz<RB>(row)) + 8 * (r16 & 3);
      x[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) pf_s4*)(vt + off));
    }
    typedef short s8 __attribute__((ext_vector_type(8)));
    const s8 v = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  } else {
    f32x8 a;
    const int d = 16 * db + r16;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = 32 * c + 8 * g + e;
      a[e] = *reinterpret_cast<const float*>(vt + row * RB + (((d >> 2) ^ (2 * vr_swz<256>(row))) << 4) + 4 * (d & 3));
    }
    return a;
  }
}

// ------------------------------------------------------- tile layout
// A stage holds one 64-key tile: K [64 keys][D] and V [64 keys][D], both
// row-major and filled by buffer_load ... lds (16 bytes per lane,
// consecutive lanes to consecutive LDS slots).  Bank conflicts are avoided
// by XOR-swizzling: a lane that fills K slot (row, pc) loads logical chunk
// pc ^ k_swz(row); V rows swizzle 32-byte pairs with vr_swz(row).
//
// S^T blocks use a permuted key order: in block kb, MFMA row r reads key
// 32(kb/2) + 8(r/4) + 4(kb%2) + r%4.  Then a lane's 8 scores of a 32-key
// half are 8 consecutive keys, the k-order of the V^T operand read
// transposed from the V rows for O^T += V^T P^T.
template <typename T, int D>
struct XTile {
  static constexpr int ES = sizeof(T);
  static constexpr int RB = D * ES;            // bytes of one K or V row
  static constexpr int CPR = RB / 16;          // 16-byte chunks per row
  static constexpr int KBYTES = kBN * RB;      // one K (or V) tile
  static constexpr int STAGE = 2 * KBYTES;
  static constexpr int KBLK = KBYTES / 1024;   // 1 KB DMA blocks per tile
  static_assert(KBLK % kWaves == 0, "DMA blocks must split over the waves");
};

template <int CPR>
__device__ __forceinline__ int k_swz(int row) { return ((row & 3) | (((row >> 3) & 3) << 2)) & (CPR - 1); }

__device__ __forceinline__ int s_key_row(int kb, int r) {
  return 32 * (kb >> 1) + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3);
}

// Wait for this wave's outstanding vector-memory operations (the LDS DMA).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef __attribute__((address_space(3))) void lds_void;

// Swizzles of the bf16 32x32 tile (XAttn32), for rows of RB = 2 D bytes.
// K: a quarter wave reads 16 distinct rows at one 16-byte chunk, so the
// chunk is XORed with the row's position among the rows that share a
// 256-byte bank span.  V: a half wave reads 4 consecutive rows at two
// adjacent 32-byte pairs, so the pair is XORed with twice the row's
// position among 4 rows, counted in bank spans; both give 8 (V) or 16 (K)
// distinct bank groups per access.
template <int CPR>
__device__ __forceinline__ int k32_swz(int row) { return (row / (16 / CPR)) & (CPR - 1); }
template <int RB>
__device__ __forceinline__ int v32_swz(int row) {
  constexpr int PP = RB / 32;   // 32-byte pairs per row
  return 2 * ((row / (8 / PP)) & (PP / 2 - 1));
}

// Per-lane part of the DMA byte offsets (loop invariant); the tile's own
// offset is wave-uniform and goes into the instructions' SGPR offset.  M32
// selects the swizzles of the 32x32 tile (specialization below).
template <typename T, int D, bool M32 = false>
struct DmaLanes {
  using X = XTile<T, D>;
  int k[X::KBLK / kWaves];
  int v[X::KBLK / kWaves];
  __device__ __forceinline__ void init(int hkv, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < X::KBLK / kWaves; ++j) {
      const int byte = (wave * (X::KBLK / kWaves) + j) * 1024 + lane * 16;
      const int row = byte / X::RB, pc = (byte % X::RB) / 16;
      int sw;
      if constexpr (M32) sw = k32_swz<X::CPR>(row);
      else sw = k_swz<X::CPR>(row);
      k[j] = row * hkv * X::RB + (pc ^ sw) * 16;
    }
#pragma unroll
    for (int j = 0; j < X::KBLK / kWaves; ++j) {
      const int byte = (wave * (X::KBLK / kWaves) + j) * 1024 + lane * 16;
      const int row = byte / X::RB, pc = (byte % X::RB) / 16;
      int sw;
      if constexpr (M32) sw = v32_swz<X::RB>(row);
      else sw = vr_swz<X::RB>(row);
      v[j] = row * hkv * X::RB + ((pc ^ (2 * sw)) << 4);
    }
  }
};

// The 32x32 tile's swizzles repeat every 16 rows (K) and every 4 rows (V),
// so a wave's K blocks need only one per-lane offset per 16-row period and
// its V blocks one offset in all: the blocks further on differ by whole
// rows, a wave-uniform amount that goes into the SGPR offset.  At d = 128
// that is 5 registers where one per block takes 8.
template <typename T, int D>
struct DmaLanes<T, D, true> {
  using X = XTile<T, D>;
  static_assert(sizeof(T) == 2, "the 32x32 tile is bf16");
  static constexpr int NB = X::KBLK / kWaves;          // 1 KB blocks per wave and tensor
  static constexpr int RPB = 1024 / X::RB;             // rows per block
  static constexpr int KP = (16 / RPB) < NB ? 16 / RPB : NB;   // blocks per 16-row K period
  static_assert(NB % KP == 0 && RPB % 4 == 0, "swizzle periods align with the blocks");
  int k[KP];
  int v;
  __device__ __forceinline__ void init(int hkv, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const int byte = (wave * NB + j) * 1024 + lane * 16;
      const int row = byte / X::RB, pc = (byte % X::RB) / 16;
      k[j] = row * hkv * X::RB + (pc ^ k32_swz<X::CPR>(row)) * 16;
    }
    const int byte = wave * NB * 1024 + lane * 16;
    const int row = byte / X::RB, pc = (byte % X::RB) / 16;
    v = row * hkv * X::RB + ((pc ^ (2 * v32_swz<X::RB>(row))) << 4);
  }
};

template <typename T, int D, bool M32>
__device__ __forceinline__ void dma_tile(char* stage, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                         const DmaLanes<T, D, M32>& ln, int ksoff, int vsoff, int wave, int hkv) {
  using X = XTile<T, D>;
  if constexpr (M32) {
    using L = DmaLanes<T, D, true>;
    const int rowb = hkv * X::RB;
#pragma unroll
    for (int j = 0; j < L::NB; ++j) {
      const int b = wave * L::NB + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(stage + b * 1024), 16, ln.k[j % L::KP],
                                               ksoff + (j / L::KP) * 16 * rowb, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < L::NB; ++j) {
      const int b = wave * L::NB + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(stage + X::KBYTES + b * 1024), 16, ln.v,
                                               vsoff + j * L::RPB * rowb, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < X::KBLK / kWaves; ++j) {
      const int b = wave * (X::KBLK / kWaves) + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(stage + b * 1024), 16, ln.k[j], ksoff, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < X::KBLK / kWaves; ++j) {
      const int b = wave * (X::KBLK / kWaves) + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(stage + X::KBYTES + b * 1024), 16, ln.v[j], vsoff,
                                               0, 0);
    }
  }
}

template <typename T>
__device__ __forceinline__ typename ElemTraits<T>::v8 lds_v8(const char* base, int chunk0, int swz, int nchunks);
template <>
__device__ __forceinline__ bf16x8 lds_v8<bf16>(const char* base, int chunk0, int swz, int nchunks) {
  return *reinterpret_cast<const bf16x8*>(base + ((chunk0 ^ swz) & (nchunks - 1)) * 16);
}
template <>
__device__ __forceinline__ f32x8 lds_v8<float>(const char* base, int chunk0, int swz, int nchunks) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(base + ((chunk0 ^ swz) & (nchunks - 1)) * 16);
  const f32x4 b = *reinterpret_cast<const f32x4*>(base + (((chunk0 + 1) ^ swz) & (nchunks - 1)) * 16);
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[4 + e] = b[e]; }
  return r;
}

// Reference-max slack of the online softmax, in log2 units (see tile()).
constexpr float kLazyLog2 = 8.f;

template <typename T>
__device__ __forceinline__ typename ElemTraits<T>::v8 ones_v8() {
  typename ElemTraits<T>::v8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = from_f32<T>(1.f);
  return r;
}

// One wave's 32 query rows against one staged tile.
template <typename T, int D>
struct XAttn {
  using V8 = typename ElemTraits<T>::v8;
  using X = XTile<T, D>;
  static constexpr int KS = D / 32, DB = D / 16;
  static constexpr int CPE = 16 / (int)sizeof(T) == 8 ? 1 : 2;   // 16-byte chunks per 8 elements

  V8 qB[2][KS];
  f32x4 o[DB][2];
  f32x4 ls[2];        // running sums, from a ones row in the PV product
  float m[2];         // reference max of the raw scores

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db][0] = o[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[0] = m[1] = -INFINITY;
    ls[0] = ls[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  template <bool kMasked>
  __device__ __forceinline__ void tile(const char* stage, int lane, float sl2, const Pred& pred, int q0, int key0) {
    const int r16 = lane & 15, g = lane >> 4;
    const char* ks = stage;
    const char* vt = stage + X::KBYTES;
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int row = s_key_row(kb, r16);
        const V8 a = lds_v8<T>(ks + row * X::RB, (4 * k + g) * CPE, k_swz<X::CPR>(row), X::CPR);
        s[kb][0] = mma16(a, qB[0][k], s[kb][0]);
        s[kb][1] = mma16(a, qB[1][k], s[kb][1]);
      }
    }
    V8 pB[2][2];
    float alpha[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float x[4][4];
      float mx = -INFINITY;
      const int q = q0 + 16 * qb + r16;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = s[kb][qb][i];
          if constexpr (kMasked) {
            const int key = key0 + 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + i;
            v = pred(q, key) ? v : -INFINITY;
          }
          x[kb][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = wave_max_16_32(mx);
      // Lazy rescaling: the reference max moves only when the tile's max
      // exceeds it by more than kLazyLog2 (in log2 units), so most tiles
      // leave O untouched; probabilities stay below 2^kLazyLog2.
      const bool grow = (mx - m[qb]) * sl2 > kLazyLog2;
      const float mnew = grow ? mx : m[qb];
      const float mneg = mnew == -INFINITY ? 0.f : -mnew * sl2;
      alpha[qb] = grow ? __builtin_amdgcn_exp2f(__builtin_fmaf(m[qb], sl2, mneg)) : 1.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pB[kb >> 1][qb][4 * (kb & 1) + i] = from_f32<T>(__builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][i], sl2, mneg)));
      m[qb] = mnew;
    }
    // rescale O only when some lane's reference max moved (the empty asm
    // keeps the multiplies inside the rarely taken branch)
    if (__ballot(alpha[0] != 1.f || alpha[1] != 1.f)) {
      float a0 = alpha[0], a1 = alpha[1];
      asm volatile("" : "+v"(a0), "+v"(a1));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[db][0] *= a0;
        o[db][1] *= a1;
      }
      ls[0] *= a0;
      ls[1] *= a1;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const V8 a = vrow_operand<T, D>(vt, c, db, r16, g);
        o[db][0] = mma16(a, pB[c][0], o[db][0]);
        o[db][1] = mma16(a, pB[c][1], o[db][1]);
      }
      // row sums of the probabilities as the MFMAs see them: a ones row
      // as the A operand sums P^T over the half's 32 keys per column
      ls[0] = mma16(ones_v8<T>(), pB[c][0], ls[0]);
      ls[1] = mma16(ones_v8<T>(), pB[c][1], ls[1]);
    }
  }

  static constexpr bool kM32 = false;   // LDS swizzles of this tile (DmaLanes)

  // Queries of the wave's unit: lane (r16, g) loads dims 32 k + 8 g .. +7 of
  // each half of queries q0 + r16 and q0 + 16 + r16, rotates them at the
  // extraction positions and keeps them as the B operand.  Every query and
  // cos/sin load is issued before issue_first() (the first tile's DMA), and
  // unconditionally (a row outside the wave's range reads the wave's first
  // row, or the region's row 0, and is zeroed afterwards): the vector-memory
  // counter retires in order, so one wait then covers all of them while the
  // tile is still in flight.
  template <typename Issue>
  __device__ __forceinline__ void load_queries(const ExtractParams& p, const ExtractPlan& P, int lane, int hq,
                                               int64_t qrow_off, Issue&& issue_first) {
    constexpr int H = D / 2, QK = D / 64;
    const int r16 = lane & 15, g = lane >> 4;
    float lo[2][QK][8], hi[2][QK][8];
    f32x4 cs4[2][QK][4];
    bool ok[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int ql = P.q0 + 16 * qb + r16;
      ok[qb] = P.wvalid && ql < P.qend;
      const int qc = ok[qb] ? ql : P.q0;
      const int pos = P.slot_region ? min(qc * P.ratio_k + P.ratio_k - 1, P.n - 1) : qc;
      const T* qrow = reinterpret_cast<const T*>(p.q) + ((P.row0 + qrow_off + qc) * hq + P.head) * (int64_t)D;
      const f32x4* crow = reinterpret_cast<const f32x4*>(p.rope + (int64_t)pos * H);
#pragma unroll
      for (int k = 0; k < QK; ++k) {
        load8_f32<T>(qrow + 32 * k + 8 * g, lo[qb][k]);
        load8_f32<T>(qrow + H + 32 * k + 8 * g, hi[qb][k]);
#pragma unroll
        for (int j = 0; j < 4; ++j) cs4[qb][k][j] = crow[16 * k + 4 * g + j];
      }
    }
    issue_first();
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int k = 0; k < QK; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const f32x4 c = cs4[qb][k][e >> 1];
          const float cc = ok[qb] ? c[2 * (e & 1)] : 1.f, sn = ok[qb] ? c[2 * (e & 1) + 1] : 0.f;
          float y0, y1;
          rope_pair(ok[qb] ? lo[qb][k][e] : 0.f, ok[qb] ? hi[qb][k][e] : 0.f, cc, sn, y0, y1);
          qB[qb][k][e] = from_f32<T>(y0);
          qB[qb][k + QK][e] = from_f32<T>(y1);
        }
  }

  // Normalise and write the unit's rows (and their log-sum-exp).
  __device__ __forceinline__ void write_rows(const ExtractParams& p, const ExtractPlan& P, int lane, int hq,
                                             int64_t qrow_off) const {
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float lt = ls[qb][0];   // every lane of a column holds its sum
      const float inv = 1.f / lt;
      const int ql = P.q0 + 16 * qb + r16;
      if (ql < P.qend) {
        const int64_t prow = P.row0 + qrow_off + ql;
        T* orow = reinterpret_cast<T*>(p.o) + (prow * hq + P.head) * (int64_t)D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          typename ElemTraits<T>::v4 outv;
#pragma unroll
          for (int i = 0; i < 4; ++i) outv[i] = from_f32<T>(o[db][qb][i] * inv);
          *reinterpret_cast<typename ElemTraits<T>::v4*>(orow + 16 * db + 4 * g) = outv;
        }
        if (g == 0 && p.lse)
          p.lse[(int64_t)P.head * p.total_rows + prow] =
              (m[qb] * p.scale_log2 + __log2f(lt)) * 0.69314718055994531f;
      }
    }
  }
};

template <typename T, int D>
constexpr int kXMinWaves = (2 * XTile<T, D>::STAGE * 2 <= 160 * 1024) ? 2 : 1;

// --------------------------------------------- bf16 extraction, 32x32 tiles
// The bf16 extraction tile on v_mfma_f32_32x32x16_bf16.  S^T = K Q^T puts the
// wave's 32 queries on the N side: lane l holds query l%32 and, in its two
// 16-register accumulators, 32 of the tile's 64 keys, while lane l^32 holds
// the other 32 keys of the same query.  Row statistics take one lane swap,
// every per-row quantity (reference max, rescale factor, running sum) is one
// scalar per lane, and each MFMA carries twice the work of a 16x16x32 one
// for the same operand registers.
//
// Key order.  S^T block kb reads K row 32 kb + (m with bits 2 and 3
// swapped) as its row m.  Register i of lane half h then holds key
// 32 kb + 16 (i/8) + 8 h + i%8: registers 8c' .. 8c'+7 are 8 consecutive
// keys, which is the P^T operand of PV step c = 2 kb + c' (keys
// 16 c + 8 h + e), and the V^T operand reads 8 consecutive keys per dim.
// Running sums come from v_dot2_f32_bf16 over the bf16 probabilities the PV
// MFMAs use, one partial per lane half, added at the end.

// V^T operand of PV step c for dims 32 db .. +31: lane l gets dim
// 32 db + l%32 of keys 16 c + 8 (l/32) + e, e = 0..7.  ds_read_b64_tr_b16:
// within each 16 lanes, output lane j element a is element j%4 of the 4
// values addressed by source lane 4a + j/4, so source lane s addresses
// 4 dims (4 (s%4) ..) of key row (s/4) of a 4-key group.
template <int D>
__device__ __forceinline__ bf16x8 vrow32_operand(const char* vt, int c, int db, int lane) {
  constexpr int RB = 2 * D;
  const int grp = lane >> 4, h = grp >> 1, dh = grp & 1, sl = lane & 15;
  pf_s4 x[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 16 * c + 8 * h + 4 * t + (sl >> 2);
    const int off = row * RB + 32 * ((2 * db + dh) ^ v32_swz<RB>(row)) + 8 * (sl & 3);
    x[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) pf_s4*)(vt + off));
  }
  typedef short s8 __attribute__((ext_vector_type(8)));
  const s8 v = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int D>
struct XAttn32 {
  using X = XTile<bf16, D>;
  static constexpr int KS = D / 16, DB = D / 32;

  bf16x8 qB[KS];
  f32x16 o[DB];
  float ls;    // running sum of this lane half's probabilities
  float m;     // reference max of the raw scores

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    ls = 0.f;
    m = -INFINITY;
  }

  template <bool kMasked>
  __device__ __forceinline__ void tile(const char* stage, int lane, float sl2, const Pred& pred, int q0, int key0) {
    const int r = lane & 31, h = lane >> 5;
    const char* ks = stage;
    const char* vt = stage + X::KBYTES;
    const int krow = (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1);   // bits 2 and 3 swapped
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + krow;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(ks + row * X::RB + (((2 * k + h) ^ k32_swz<X::CPR>(row)) << 4));
        s[kb] = mma32(a, qB[k], s[kb]);
      }
    }
    float x[2][16];
    float mx = -INFINITY;
    const int q = q0 + r;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = s[kb][i];
        if constexpr (kMasked) {
          const int key = key0 + 32 * kb + 16 * (i >> 3) + 8 * h + (i & 7);
          v = pred(q, key) ? v : -INFINITY;
        }
        x[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = half_max_32(mx);
    // Lazy rescaling, as in the 16x16 tile: the reference max moves only
    // when the tile's max exceeds it by more than kLazyLog2 (log2 units).
    const bool grow = (mx - m) * sl2 > kLazyLog2;
    const float mnew = grow ? mx : m;
    const float mneg = mnew == -INFINITY ? 0.f : -mnew * sl2;
    float alpha = grow ? __builtin_amdgcn_exp2f(__builtin_fmaf(m, sl2, mneg)) : 1.f;
    bf16x8 pB[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pB[2 * kb + (i >> 3)][i & 7] = from_f32<bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][i], sl2, mneg)));
    m = mnew;
    if (__ballot(alpha != 1.f)) {
      asm volatile("" : "+v"(alpha));
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      ls *= alpha;
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one2 = {from_f32<bf16>(1.f), from_f32<bf16>(1.f)};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mma32(vrow32_operand<D>(vt, c, db, lane), pB[c], o[db]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {pB[c][2 * e], pB[c][2 * e + 1]};
        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls, false);
      }
    }
  }

  static constexpr bool kM32 = true;    // LDS swizzles of this tile (DmaLanes)

  // Queries of the wave's unit: lane (r, h) loads dims 16 kk + 8 h .. +7 of
  // each half of query q0 + r, rotates them at the extraction position and
  // keeps them as the B operand; every load goes out before issue_first()
  // (the first tile's DMA), and unconditionally (a row outside the wave's
  // range reads the wave's first row and is zeroed), so one wait covers them
  // while the tile is in flight.
  template <typename Issue>
  __device__ __forceinline__ void load_queries(const ExtractParams& p, const ExtractPlan& P, int lane, int hq,
                                               int64_t qrow_off, Issue&& issue_first) {
    using T = bf16;
    const int r = lane & 31, h = lane >> 5;
    constexpr int H = D / 2, QH = KS / 2;
    float lo[QH][8], hi[QH][8];
    f32x4 cs4[QH][4];
    const int ql = P.q0 + r;
    const bool ok = P.wvalid && ql < P.qend;
    const int qc = ok ? ql : P.q0;
    const int pos = P.slot_region ? min(qc * P.ratio_k + P.ratio_k - 1, P.n - 1) : qc;
    const T* qrow = reinterpret_cast<const T*>(p.q) + ((P.row0 + qrow_off + qc) * hq + P.head) * (int64_t)D;
    const f32x4* crow = reinterpret_cast<const f32x4*>(p.rope + (int64_t)pos * H);
#pragma unroll
    for (int kk = 0; kk < QH; ++kk) {
      load8_f32<T>(qrow + 16 * kk + 8 * h, lo[kk]);
      load8_f32<T>(qrow + H + 16 * kk + 8 * h, hi[kk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) cs4[kk][j] = crow[8 * kk + 4 * h + j];
    }
    issue_first();
#pragma unroll
    for (int kk = 0; kk < QH; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f32x4 c = cs4[kk][e >> 1];
        const float cc = ok ? c[2 * (e & 1)] : 1.f, sn = ok ? c[2 * (e & 1) + 1] : 0.f;
        float y0, y1;
        rope_pair(ok ? lo[kk][e] : 0.f, ok ? hi[kk][e] : 0.f, cc, sn, y0, y1);
        qB[kk][e] = from_f32<T>(y0);
        qB[kk + QH][e] = from_f32<T>(y1);
      }
  }

  // Normalise and write the unit's rows: register i of block db is dim
  // 32 db + 8 (i/4) + 4 h + i%4 of query q0 + r.
  __device__ __forceinline__ void write_rows(const ExtractParams& p, const ExtractPlan& P, int lane, int hq,
                                             int64_t qrow_off) const {
    using T = bf16;
    const int r = lane & 31, h = lane >> 5;
    const float lt = half_sum_32(ls);
    const float inv = 1.f / lt;
    const int ql = P.q0 + r;
    if (ql < P.qend) {
      const int64_t prow = P.row0 + qrow_off + ql;
      T* orow = reinterpret_cast<T*>(p.o) + (prow * hq + P.head) * (int64_t)D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 outv;
#pragma unroll
          for (int e = 0; e < 4; ++e) outv[e] = from_f32<T>(o[db][4 * g4 + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g4 + 4 * h) = outv;
        }
      if (h == 0 && p.lse)
        p.lse[(int64_t)P.head * p.total_rows + prow] = (m * p.scale_log2 + __log2f(lt)) * 0.69314718055994531f;
    }
  }
};

// Extraction attention.  The plan, tile enumeration, DMA schedule and tile
// loop are shared by both tiles; A (XAttn for fp32, XAttn32 for bf16)
// supplies the query operand layout, the tile and the output layout, and
// selects the LDS swizzles (A::kM32).
template <typename T, int D, typename A>
__global__ __launch_bounds__(kThreads, (kXMinWaves<T, D>)) void extract_attn_kernel(const ExtractParams p) {
  using X = XTile<T, D>;
  __shared__ __attribute__((aligned(1024))) char stage0[X::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[X::STAGE];
  // The stages are written only by buffer_load ... lds; escape them so the
  // compiler does not treat them as never-stored memory.
  asm volatile("" : : "r"(stage0), "r"(stage1) : "memory");
  const int L = xcd_logical(blockIdx.x, p.grid_wg);
  if (L >= p.total_wg) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const ExtractPlan P = extract_plan(p, L, wave);
  const int hq = p.hq, hkv = p.hkv;
  const int64_t qrow_off = P.slot_region ? P.n : 0;
  // buffer resources: this document's rotated keys and its values, KV head
  // kvh; reads past the document's rows return zeros
  const int64_t doc_rows = (int64_t)P.n + P.m;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const char*>(p.krot) + ((P.row0 * hkv + P.kvh) * (int64_t)X::RB)), 0,
      (int)(doc_rows * hkv * X::RB), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const char*>(p.v) + ((P.row0 * hkv + P.kvh) * (int64_t)X::RB)), 0,
      (int)(doc_rows * hkv * X::RB), 0x00020000);
  DmaLanes<T, D, A::kM32> lanes;
  lanes.init(hkv, wave, lane);
  auto issue = [&](int it, char* stage) {
    const TileSel ts = extract_tile(P, it);
    const int krow0 = (ts.is_slot ? P.n : 0) + ts.key0;
    dma_tile<T, D>(stage, krs, vrs, lanes, krow0 * hkv * X::RB, krow0 * hkv * X::RB, wave, hkv);
  };
  const int ntiles = (P.nA1 - P.nA0) + (P.nB1 - P.nB0) + P.nS;

  A W;
  W.init();
  // the first tile's DMA goes out between the query loads and their
  // rotation, unconditionally, so the wait below is not widened by a branch:
  // a launched workgroup always has a tile (its wave 0 owns rows), and a DMA
  // past the document's rows reads zeros through the buffer range check
  W.load_queries(p, P, lane, hq, qrow_off, [&] { issue(0, stage0); });

  auto compute = [&](int it, const char* stage) {
    const TileSel ts = extract_tile(P, it);
    if (!ts.active) return;
    if (ts.masked) W.template tile<true>(stage, lane, p.scale_log2, ts.pred, P.q0, ts.key0);
    else W.template tile<false>(stage, lane, p.scale_log2, ts.pred, P.q0, ts.key0);
  };
  for (int it = 0; it < ntiles; it += 2) {
    wait_vmem();
    __syncthreads();
    if (it + 1 < ntiles) issue(it + 1, stage1);
    compute(it, stage0);
    if (it + 1 >= ntiles) break;
    wait_vmem();
    __syncthreads();
    if (it + 2 < ntiles) issue(it + 2, stage0);
    compute(it + 1, stage1);
  }

  if (!P.wvalid) return;
  W.write_rows(p, P, lane, hq, qrow_off);
}


// Counting twin of the extraction kernel: the same plan, tile enumeration and
// predicate, but each active (wave, tile) pair counts its visible cells.
__global__ __launch_bounds__(kThreads) void mask_count_kernel(const ExtractParams p) {
  const int L = xcd_logical(blockIdx.x, p.grid_wg);
  if (L >= p.total_wg) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const ExtractPlan P = extract_plan(p, L, wave);
  const int ntiles = (P.nA1 - P.nA0) + (P.nB1 - P.nB0) + P.nS;
  unsigned long long c_dd = 0, c_sd = 0, c_ss = 0, c_empty = 0, c_tiles = 0;
  for (int it = 0; it < ntiles; ++it) {
    const TileSel ts = extract_tile(P, it);
    if (!ts.active) continue;
    // lane -> query row (lane % 32), keys [32*(lane/32), +32)
    const int q = P.q0 + (lane & 31);
    int cnt = 0;
    if (q < P.qend) {
      for (int kk = 0; kk < 32; ++kk) {
        const int c = ts.key0 + 32 * (lane >> 5) + kk;
        cnt += ts.pred(q, c) ? 1 : 0;
      }
    }
    int tot = cnt;
    for (int off = 1; off < 64; off <<= 1) tot += __shfl_xor(tot, off);
    c_tiles += 1;
    if (tot == 0) c_empty += 1;
    if (ts.is_slot) c_ss += tot;          // slot keys (only slot rows see them, except under the anchor ablation)
    else if (!P.slot_region) c_dd += tot;
    else c_sd += tot;
  }
  // one query head per KV group is counted (the mask does not depend on the head)
  if (lane == 0 && P.wvalid && (P.head % p.G) == 0) {
    atomicAdd(reinterpret_cast<unsigned long long*>(p.counts + 0), c_dd);
    atomicAdd(reinterpret_cast<unsigned long long*>(p.counts + 1), c_sd);
    atomicAdd(reinterpret_cast<unsigned long long*>(p.counts + 2), c_ss);
    atomicAdd(reinterpret_cast<unsigned long long*>(p.counts + 3), c_empty);
    atomicAdd(reinterpret_cast<unsigned long long*>(p.counts + 4), c_tiles);
  }
}

// Tile-schedule twin of the extraction kernel: the same plan and tile
// enumeration; every (unit, tile) pair a wave computes is written out.
__global__ __launch_bounds__(kThreads) void tile_dump_kernel(const ExtractParams p) {
  const int L = xcd_logical(blockIdx.x, p.grid_wg);
  if (L >= p.total_wg) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const ExtractPlan P = extract_plan(p, L, wave);
  if (!P.wvalid) return;
  const int ntiles = (P.nA1 - P.nA0) + (P.nB1 - P.nB0) + P.nS;
  int cnt = 0;
  for (int it = 0; it < ntiles; ++it) cnt += extract_tile(P, it).active ? 1 : 0;
  unsigned long long base = 0;
  if (lane == 0) base = atomicAdd(reinterpret_cast<unsigned long long*>(p.counts), (unsigned long long)cnt);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)base);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(base >> 32));
  long long idx = (long long)(((unsigned long long)hi << 32) | lo);
  for (int it = 0; it < ntiles; ++it) {
    const TileSel ts = extract_tile(P, it);
    if (!ts.active) continue;
    if (lane == 0 && idx < p.entry_cap) {
      c2kv_tile_entry e;
      e.doc = p.doc_base + P.doc;
      e.kv_head = P.kvh;
      e.q_head = P.head;
      e.q_slot = P.slot_region;
      e.q0 = P.q0;
      e.q1 = P.qend;
      e.k_slot = ts.is_slot;
      e.key0 = ts.key0;
      e.nkeys = ts.nvalid;
      e.masked = ts.masked ? 1 : 0;
      p.entries[idx] = e;
    }
    ++idx;
  }
}

// ============================================== attention over the cache
// LDS DMA of one K tile and one row-major V tile (KB bytes each) of cache
// rows; this wave fills 1 KB blocks wave*NDMA .. +NDMA-1 of each.
template <int NDMA, int KB>
__device__ __forceinline__ void kv_rows_dma(char* stage, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                            const int* koff, const int* voff, int soff, int wave) {
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int b = wave * NDMA + j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(stage + b * 1024), 16, koff[j], soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(stage + KB + b * 1024), 16, voff[j], soff, 0, 0);
  }
}

// Question prefill over a composed cache, split-K over the keys, with the
// question's RoPE and append fused in.  A workgroup owns (request, KV head,
// key chunk, group of 4 units); a unit is 32 question rows of one query head.
// The workgroup has two groups of 4 waves holding the same 4 units: group 0
// takes the chunk's even 64-key tiles and group 1 its odd ones, so each SIMD
// runs two waves (one wave's MFMAs overlap the other's softmax), and the two
// halves are combined in LDS at the end, without more split partials.
//   * Queries are loaded pre-RoPE and rotated in registers at q_pos0 + t,
//     then rounded to the storage type for the MFMAs.  The cos/sin of the
//     workgroup's question tokens are computed once per workgroup into a
//     table in the second stage, which the DMA fills only after the
//     rotation.
//   * The tile code picks its group's half of a stage with a wave-uniform
//     branch on constant offsets; the compiler then sees that the DMA into
//     one stage never aliases the LDS reads of the other and inserts no
//     vector-memory wait inside the tile.
//   * K and V tiles come from the cache by LDS DMA, a pair of tiles (one per
//     group) per stage, double buffered where two stages fit 128 KB.
//   * Rows at or past cache_len are the question's own keys and values.
//     Before its first DMA, every workgroup whose chunk holds such rows
//     rotates those keys at their positions, copies the values, and writes
//     both into the cache; the unit groups of a chunk write the same bytes.
//     A workgroup-scope fence and a barrier order these stores before the
//     workgroup's own DMA of the rows.
//   * The same tile code as extraction; V stays row-major and its transposed
//     operand is read with ds_read_b64_tr_b16.
constexpr int kPWaves = 2 * kWaves;        // waves per prefill workgroup: two groups
constexpr int kPThreads = 64 * kPWaves;

template <typename T, int D>
__global__ __launch_bounds__(kPThreads, 1) void prefill_attn_kernel(const CacheParams p) {
  using X = XTile<T, D>;
  using A = XAttn<T, D>;
  constexpr int RB = X::RB, CPR = X::CPR, KB = X::KBYTES;     // V tile is KB bytes too
  constexpr int NDMA = KB / 1024 / kWaves;                    // per wave, per tensor
  constexpr int PSTAGE = 2 * X::STAGE;                        // one tile per group
  constexpr int NPS = 2 * PSTAGE <= 128 * 1024 ? 2 : 1;       // pair stages
  constexpr int CE = Chunk<T>::CE, H = D / 2, HC = CPR / 2;   // elements per chunk, half row, chunks per half
  // two distinct arrays, so the compiler sees that the DMA into one stage
  // never aliases the LDS reads of the other (no vmcnt wait before them)
  __shared__ __attribute__((aligned(1024))) char ring0[PSTAGE];
  __shared__ __attribute__((aligned(1024))) char ring1[NPS == 2 ? PSTAGE : 16];
  asm volatile("" : : "r"(ring0), "r"(ring1) : "memory");
  // The kernel-argument fields of the prologue, with the first request's
  // entry (the only one of a one-request launch), loaded in one round of
  // scalar loads: the empty asm needs them all at once, so they complete at
  // one wait instead of one dependent round per use.
  const int grid_wg = p.grid_wg, total_wg = p.total_wg, num_reqs = p.num_reqs, req0 = p.req0, nug = p.nug;
  const int G = p.G, nblk_q = p.nblk_q, tq = p.tq, hq = p.hq, hkv = p.hkv, chunk = p.chunk;
  const int64_t cap = p.cap;
  const CacheReq rq0 = p.reqs[0];
  const void* const q_in = p.q;
  void* const kc = p.kc;
  void* const vc = p.vc;
  asm volatile("" : : "s"(grid_wg), "s"(total_wg), "s"(num_reqs), "s"(req0), "s"(nug), "s"(G), "s"(nblk_q), "s"(tq),
               "s"(hq), "s"(hkv), "s"(chunk), "s"(cap), "s"(rq0.wg0), "s"(rq0.cache_len), "s"(rq0.nsplit),
               "s"(rq0.pbase), "s"(rq0.pos0), "s"(q_in), "s"(kc), "s"(vc));
  const int L = xcd_logical(blockIdx.x, grid_wg);
  if (L >= total_wg) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = wave / kWaves, wq = wave % kWaves;
  const int r16 = lane & 15, g = lane >> 4;
  const int ri = request_of(p.reqs, num_reqs, L);
  CacheReq rq = rq0;
  if (num_reqs != 1) rq = p.reqs[ri];
  const int r = req0 + ri;
  const int per_kvh = rq.nsplit * nug;
  const int local = L - rq.wg0;
  const int kvh = local / per_kvh;
  const int rem = local % per_kvh;
  const int split = rem / nug, ug = rem % nug;
  const int u = ug * kWaves + wq;
  const int nunits = nblk_q * G;
  const bool wvalid = u < nunits;
  const int blk = u / G, head = kvh * G + (u % G);
  const int t0 = blk * kQW, t1 = wvalid ? min(tq, t0 + kQW) : 0;
  const int Lr = rq.cache_len + tq;
  const int ks0 = split * chunk, ks1 = min(Lr, ks0 + chunk);
  const int64_t head_base = ((int64_t)r * hkv + kvh) * cap;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const char*>(kc) + head_base * RB), 0, ks1 * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const char*>(vc) + head_base * RB), 0, ks1 * RB, 0x00020000);
  int koff[NDMA], voff[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int byte = (wq * NDMA + j) * 1024 + lane * 16;
    const int row = byte / RB, pc = (byte % RB) / 16;
    koff[j] = row * RB + ((pc ^ k_swz<CPR>(row)) << 4);
    voff[j] = row * RB + ((pc ^ (2 * vr_swz<RB>(row))) << 4);
  }
  const int ntiles = (ks1 - ks0 + kBN - 1) / kBN;
  const int npairs = (ntiles + 1) / 2;
  // this group's tile of pair j into pair stage `ps` (each group's 4 waves
  // fill their own tile; tiles past the chunk read as zeros)
  auto issue_pair = [&](int j, char* ps) {
    const int it = 2 * j + grp;
    // (the tile's byte offset is wave-uniform: keep it in an SGPR)
    kv_rows_dma<NDMA, KB>(ps + grp * X::STAGE, krs, vrs, koff, voff,
                          __builtin_amdgcn_readfirstlane((ks0 + it * kBN) * RB), wq);
  };
  // RoPE frequencies this thread uses, loaded first: a thread keeps one
  // chunk column of the new rows and one frequency of the cos/sin table
  // (kPThreads is a multiple of HC and of H)
  static_assert(kPThreads % HC == 0 && kPThreads % H == 0, "fixed columns per thread");
  float fq[CE];
#pragma unroll
  for (int e = 0; e < CE; ++e) fq[e] = p.freqs.f[(tid % HC) * CE + e];
  const float ftab = p.freqs.f[tid % H];

  // ---- the chunk's question rows (keys rotated at q_pos0 + (row -
  // cache_len), values copied) go to the cache before any DMA reads them
  if (max(ks0, rq.cache_len) < ks1) {
    for (int item = tid; item < (ks1 - max(ks0, rq.cache_len)) * HC; item += kPThreads) {
      const int row = max(ks0, rq.cache_len) + item / HC, c = item % HC;
      const int t = row - rq.cache_len;
      const int64_t src = (((int64_t)r * tq + t) * hkv + kvh) * D + c * CE;
      const T* ksrc = reinterpret_cast<const T*>(p.k_new) + src;
      const T* vsrc = reinterpret_cast<const T*>(p.v_new) + src;
      uint4 klo = *reinterpret_cast<const uint4*>(ksrc);
      uint4 khi = *reinterpret_cast<const uint4*>(ksrc + H);
      const uint4 vlo = *reinterpret_cast<const uint4*>(vsrc);
      const uint4 vhi = *reinterpret_cast<const uint4*>(vsrc + H);
      float cs[CE], sn[CE];
#pragma unroll
      for (int e = 0; e < CE; ++e) rope_cs(rq.pos0 + t, fq[e], cs[e], sn[e]);
      rotate_chunk<T>(klo, khi, cs, sn);
      T* kd = reinterpret_cast<T*>(kc) + (head_base + row) * D + c * CE;
      T* vd = reinterpret_cast<T*>(vc) + (head_base + row) * D + c * CE;
      *reinterpret_cast<uint4*>(kd) = klo;
      *reinterpret_cast<uint4*>(kd + H) = khi;
      *reinterpret_cast<uint4*>(vd) = vlo;
      *reinterpret_cast<uint4*>(vd + H) = vhi;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  // ---- the wave's raw queries (rows past the unit read row t0 and are
  // zeroed), issued before the first DMA so that the rotation waits for
  // them only; then the cos/sin of the workgroup's tokens [tlo, thi) (at
  // most 4 blocks of 32) into the stage that pair 1 (pair 0 with one stage)
  // fills
  using V8 = typename ElemTraits<T>::v8;
  V8 qlo[2][D / 64], qhi[2][D / 64];   // kept packed until the rotation
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = t0 + 16 * qb + r16;
    const int tt = (wvalid && t < t1) ? t : (wvalid ? t0 : 0);
    const T* qrow = reinterpret_cast<const T*>(q_in) + (((int64_t)r * tq + tt) * hq + head) * D;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      qlo[qb][k] = *reinterpret_cast<const V8*>(qrow + 32 * k + 8 * g);
      qhi[qb][k] = *reinterpret_cast<const V8*>(qrow + H + 32 * k + 8 * g);
    }
  }
  if constexpr (NPS == 2) issue_pair(0, ring0);
  const int ulo = ug * kWaves, uhi = min(nunits, ulo + kWaves) - 1;
  const int tlo = (ulo / G) * kQW, thi = min(tq, (uhi / G + 1) * kQW);
  float2* cs_tab = reinterpret_cast<float2*>(NPS == 2 ? ring1 : ring0);
  static_assert(4 * kQW * H * sizeof(float2) <= PSTAGE, "cos/sin table fits one stage");
  for (int i = tid; i < (thi - tlo) * H; i += kPThreads) {
    float c, sn;
    rope_cs(rq.pos0 + tlo + i / H, ftab, c, sn);
    cs_tab[i] = make_float2(c, sn);
  }
  lds_barrier();   // the table is complete (the DMA of pair 0 stays in flight)
  A W;
  W.init();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = t0 + 16 * qb + r16;
    const bool ok = wvalid && t < t1;
    const float2* cs_row = cs_tab + (ok ? t - tlo : 0) * H;
#pragma unroll
    for (int k = 0; k < D / 64; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = cs_row[32 * k + 8 * g + e];
        float y0, y1;
        rope_pair(static_cast<float>(qlo[qb][k][e]), static_cast<float>(qhi[qb][k][e]), cs.x, cs.y, y0, y1);
        W.qB[qb][k][e] = from_f32<T>(ok ? y0 : 0.f);
        W.qB[qb][k + D / 64][e] = from_f32<T>(ok ? y1 : 0.f);
      }
  }
  if constexpr (NPS == 1) {
    __syncthreads();   // every wave is done with the table
    issue_pair(0, ring0);
  }

  const Pred pred = pred_causal(ks1, rq.cache_len);
  auto run_pair = [&](int j, const char* cur, char* nxt) {
    wait_vmcnt<0>();   // this wave's share of pair j has landed
    __syncthreads();   // both tiles of pair j are in LDS; pair j - 1 (and the table) is no longer read
    if (NPS == 2 && j + 1 < npairs) issue_pair(j + 1, nxt);
    const int it = 2 * j + grp;
    const int key0 = ks0 + it * kBN;
    if (it < ntiles && wvalid && key0 < rq.cache_len + t1) {
      const bool masked = (key0 + kBN - 1 > rq.cache_len + t0) || (key0 + kBN > ks1);
      if (grp == 0) {
        if (masked) W.template tile<true>(cur, lane, p.scale_log2, pred, t0, key0);
        else W.template tile<false>(cur, lane, p.scale_log2, pred, t0, key0);
      } else {
        if (masked) W.template tile<true>(cur + X::STAGE, lane, p.scale_log2, pred, t0, key0);
        else W.template tile<false>(cur + X::STAGE, lane, p.scale_log2, pred, t0, key0);
      }
    }
    if (NPS == 1 && j + 1 < npairs) {
      __syncthreads();   // pair j is no longer read
      issue_pair(j + 1, nxt);
    }
  };
  if constexpr (NPS == 2) {
    for (int j = 0; j < npairs; j += 2) {
      run_pair(j, ring0, ring1);
      if (j + 1 >= npairs) break;
      run_pair(j + 1, ring1, ring0);
    }
  } else {
    for (int j = 0; j < npairs; ++j) run_pair(j, ring0, ring0);
  }

  // ---- combine the groups: group 1 leaves (o, m, l) in LDS, group 0 merges
  // them into its own (both hold the same rows in the same lanes)
  constexpr int NV = A::DB * 2 * 4 + 4;                       // floats per lane
  // (waves 0-1 of a group exchange through the first stage, 2-3 through the
  // second; with one stage, all through it)
  float* cmb = NPS == 2 ? reinterpret_cast<float*>(wq < 2 ? ring0 : ring1) + (wq & 1) * NV * 64 + lane
                        : reinterpret_cast<float*>(ring0) + wq * NV * 64 + lane;
  static_assert(kWaves / NPS * NV * 64 * sizeof(float) <= PSTAGE, "exchange fits the stages");
  __syncthreads();   // no wave reads a tile any more
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < A::DB; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) cmb[((db * 2 + qb) * 4 + i) * 64] = W.o[db][qb][i];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      cmb[(A::DB * 8 + qb) * 64] = W.m[qb];
      cmb[(A::DB * 8 + 2 + qb) * 64] = W.ls[qb][0];
    }
  }
  __syncthreads();
  if (grp == 1 || !wvalid) return;
  float lt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float m1 = cmb[(A::DB * 8 + qb) * 64], l1 = cmb[(A::DB * 8 + 2 + qb) * 64];
    const float m0 = W.m[qb], l0 = W.ls[qb][0];
    const float mm = fmaxf(m0, m1);
    const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m0 - mm) * p.scale_log2);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - mm) * p.scale_log2);
#pragma unroll
    for (int db = 0; db < A::DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        W.o[db][qb][i] = W.o[db][qb][i] * a0 + cmb[((db * 2 + qb) * 4 + i) * 64] * a1;
    lt[qb] = l0 * a0 + l1 * a1;
    W.m[qb] = mm;
  }

  // ---- final rows (one key chunk) or split partials, m in log2 units
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float m2 = W.m[qb] * p.scale_log2;
    const int t = t0 + 16 * qb + r16;
    if (t >= t1) continue;
    if (rq.nsplit == 1) {
      const float inv = 1.f / lt[qb];
      T* orow = reinterpret_cast<T*>(p.o) + (((int64_t)r * p.tq + t) * p.hq + head) * D;
#pragma unroll
      for (int db = 0; db < A::DB; ++db) {
        typename ElemTraits<T>::v4 outv;
#pragma unroll
        for (int i = 0; i < 4; ++i) outv[i] = from_f32<T>(W.o[db][qb][i] * inv);
        *reinterpret_cast<typename ElemTraits<T>::v4*>(orow + 16 * db + 4 * g) = outv;
      }
      if (g == 0 && p.lse)
        p.lse[((int64_t)r * p.hq + head) * p.tq + t] = (m2 + __log2f(lt[qb])) * 0.69314718055994531f;
    } else {
      const int64_t idx = (int64_t)rq.pbase + ((int64_t)head * p.tq + t) * rq.nsplit + split;
      float* prow = p.part_o + idx * D;
      if (g == 0) p.part_ml[idx] = make_float2(W.m[qb] == -INFINITY ? -INFINITY : m2, lt[qb]);
#pragma unroll
      for (int db = 0; db < A::DB; ++db)
        *reinterpret_cast<f32x4*>(prow + 16 * db + 4 * g) = W.o[db][qb];
    }
  }
}

// ------------------------------------------------------------ launchers
template <typename T, int D>
static hipError_t launch_extract_t(const ExtractParams& p, int mode, hipStream_t st) {
  if (mode == kExtractCount) {
    hipLaunchKernelGGL(mask_count_kernel, dim3(p.grid_wg), dim3(kThreads), 0, st, p);
  } else if (mode == kExtractDump) {
    hipLaunchKernelGGL(tile_dump_kernel, dim3(p.grid_wg), dim3(kThreads), 0, st, p);
  } else if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((extract_attn_kernel<bf16, D, XAttn32<D>>), dim3(p.grid_wg), dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL((extract_attn_kernel<T, D, XAttn<T, D>>), dim3(p.grid_wg), dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_extract_attn(const ExtractParams& p, int dtype, int head_dim, int mode, hipStream_t st) {
  if (dtype == C2KV_BF16) {
    return head_dim == 128 ? launch_extract_t<bf16, 128>(p, mode, st) : launch_extract_t<bf16, 64>(p, mode, st);
  }
  return head_dim == 128 ? launch_extract_t<float, 128>(p, mode, st) : launch_extract_t<float, 64>(p, mode, st);
}

template <typename T, int D>
static hipError_t launch_prefill_t(const CacheParams& p, hipStream_t st) {
  hipLaunchKernelGGL((prefill_attn_kernel<T, D>), dim3(p.grid_wg), dim3(kPThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const CacheParams& p, int dtype, int head_dim, hipStream_t st) {
  if (dtype == C2KV_BF16) {
    return head_dim == 128 ? launch_prefill_t<bf16, 128>(p, st) : launch_prefill_t<bf16, 64>(p, st);
  }
  return head_dim == 128 ? launch_prefill_t<float, 128>(p, st) : launch_prefill_t<float, 64>(p, st);
}

}  // namespace c2kv
