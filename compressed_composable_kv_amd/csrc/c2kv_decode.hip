// Decode over a composed cache, and the split-K merge shared with prefill.
//
// Decode (the C2KV explainer's experimental-results section: every
// generated token reads the whole compressed cache) is bound by reading the
// cache once.  A workgroup owns one (request, KV head, key chunk); ALL query
// heads of the group sit in the 16 columns of one wave's MFMA tiles, and the
// four waves stream disjoint 32-key steps of the chunk, so every K/V byte is
// read from HBM exactly once:
//   * K goes straight from global memory into MFMA A-operand registers
//     (S^T = K Q^T, keys on the M side, heads on N);
//   * V goes from global memory into a wave-private LDS tile by
//     buffer_load ... lds (row-major, 16-byte chunks XOR-swizzled), and the
//     V^T operand of O^T += V^T P^T is read back transposed with
//     ds_read_b64_tr_b16 (bf16) or element reads (fp32);
//   * the cache is read once per call, so K and V loads carry the
//     non-temporal hint (streamed past the caches; on MI355X this raised
//     long-context decode from 6.2 to 6.8 TB/s);
//   * the first step's loads are issued before the query prologue, so the
//     RoPE table and query rotation overlap the memory latency;
//   * the new token's key is rotated (RoPE at the decode position) in the
//     registers that would have loaded it, its value is patched into the LDS
//     tile, and both are written to the cache -- no separate append launch;
//   * the four waves' (max, sum, O) are combined in LDS; with one chunk per
//     (request, KV head) the workgroup writes the final output, otherwise a
//     partial row that merge_kernel combines by log-sum-exp.
#include "c2kv_device.hpp"
#include "c2kv_launch.hpp"

namespace c2kv {

// Order this wave's own LDS writes before its reads of other lanes' data
// (and the reads of one step before the next step's writes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait for this wave's outstanding vector-memory operations (incl. LDS DMA).
__device__ __forceinline__ void dec_wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N of them are outstanding (the counter retires in
// issue order, so every older operation has completed).  gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at
// their maxima.
template <int N>
__device__ __forceinline__ void dec_wait_vmem_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

typedef __attribute__((address_space(3))) void dec_lds_void;
typedef short dec_s4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ void v8_to_f32(const typename ElemTraits<T>::v8& v, float* f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = to_f32(v[e]);
}

// One wave's V tile: 32 keys x D, row-major, 16-byte chunks swizzled.
template <typename T, int D>
struct DecTile {
  static constexpr int ES = sizeof(T);
  static constexpr int RB = D * ES;              // bytes per key row
  static constexpr int CPR = RB / 16;            // chunks per row
  static constexpr int BYTES = 32 * RB;
  static constexpr int NDMA = BYTES / 1024;      // 1 KB DMA instructions per step
  static_assert(BYTES % 1024 == 0, "tile must be whole DMA blocks");
};

// Physical chunk of logical chunk c in tile row `row` is c ^ dv_swz(row).
// bf16: the transposed reads of a 32-lane half touch 8 rows x 32 bytes,
// spread over all 64 banks by XOR-ing the 32-byte pair index with the row.
// fp32: the element reads of the four lane groups hit 4 rows, offset by 4
// chunks each.
template <typename T, int D>
__device__ __forceinline__ int dv_swz(int row) {
  constexpr int CPR = DecTile<T, D>::CPR;
  if constexpr (sizeof(T) == 2) return CPR >= 16 ? 2 * (row & 7) : 2 * ((row >> 1) & 3);
  else return (4 * ((row >> 2) & 3)) & (CPR - 1);
}

// Cache-policy operand of the streaming loads: the non-temporal bit.
constexpr int kDecNT = 2;

// buffer_load ... lds of one V tile: instruction j fills LDS bytes
// [1024 j, 1024 j + 1024) of the tile, lane i taking 16 bytes from byte
// offset row_off + off[j] of the resource (zeros past its end).
template <int NDMA>
__device__ __forceinline__ void dma_v_tile(__amdgpu_buffer_rsrc_t rs, char* tile, const int* off, int row_off) {
#pragma unroll
  for (int j = 0; j < NDMA; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (dec_lds_void*)(tile + j * 1024), 16, row_off + off[j], 0, 0, kDecNT);
}

// K A-operand of one 32-key step through a buffer resource (rows past its
// end read as zeros): lane (r16, g) takes, for each 16-key block kb, the 8
// elements 32 ks + 8 g .. +7 of key key0 + 16 kb + r16.  It issues
// kDecKLoads<T, D> vector loads.
template <typename T, int D>
constexpr int kDecKLoads = 2 * (D / 32) * (sizeof(T) == 2 ? 1 : 2);

template <typename T, int D>
__device__ __forceinline__ void dec_load_k(typename ElemTraits<T>::v8 (&ka)[2][D / 32], __amdgpu_buffer_rsrc_t rs,
                                           int key0, int r16, int g) {
  using V8 = typename ElemTraits<T>::v8;
  constexpr int ES = sizeof(T), RB = D * ES;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = (key0 + 16 * kb + r16) * RB;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int off = row + (32 * ks + 8 * g) * ES;
      if constexpr (ES == 2) {
        const auto u = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kDecNT);
        ka[kb][ks] = __builtin_bit_cast(V8, u);
      } else {
        const auto u0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kDecNT);
        const auto u1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, kDecNT);
        typedef unsigned int u8v __attribute__((ext_vector_type(8)));
        const u8v w = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
        ka[kb][ks] = __builtin_bit_cast(V8, w);
      }
    }
  }
}

template <typename T, int D>
constexpr int kDecLdsBytes = (kWaves * DecTile<T, D>::BYTES > kWaves * 16 * (D + 2) * 4)
                                 ? kWaves * DecTile<T, D>::BYTES : kWaves * 16 * (D + 2) * 4;

template <typename T, int D>
constexpr int kDecMinWaves = (kDecLdsBytes<T, D> * 3 <= 160 * 1024) ? 3 : 1;

// V^T A operand for dims 16 db .. 16 db + 15: lane (r16, g) gets dim
// 16 db + r16 of keys 4g + a (elements a = 0..3) and 16 + 4g + a (4..7),
// the key order of the P^T operand built from the S^T accumulators.
template <typename T, int D>
__device__ __forceinline__ typename ElemTraits<T>::v8 vt_operand(const char* vt, int db, int r16, int g);

template <>
__device__ __forceinline__ bf16x8 vt_operand<bf16, 128>(const char* vt, int db, int r16, int g) {
  // ds_read_b64_tr_b16: within each 16 lanes, output lane j element a is
  // element (j % 4) of the 4 values addressed by source lane 4a + j / 4.
  // Source lane i therefore addresses row 16h + 4g + i/4, dims
  // 16 db + 4 (i % 4) .. +3.
  dec_s4 x[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * h + 4 * g + (r16 >> 2);
    const int off = row * 256 + 32 * (db ^ (row & 7)) + 8 * (r16 & 3);
    x[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) dec_s4*)(vt + off));
  }
  typedef short s8 __attribute__((ext_vector_type(8)));
  const s8 v = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}
template <>
__device__ __forceinline__ bf16x8 vt_operand<bf16, 64>(const char* vt, int db, int r16, int g) {
  dec_s4 x[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * h + 4 * g + (r16 >> 2);
    const int off = row * 128 + 32 * (db ^ ((row >> 1) & 3)) + 8 * (r16 & 3);
    x[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) dec_s4*)(vt + off));
  }
  typedef short s8 __attribute__((ext_vector_type(8)));
  const s8 v = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}
template <int D>
__device__ __forceinline__ f32x8 vt_operand_f32(const char* vt, int db, int r16, int g) {
  constexpr int RB = D * 4;
  f32x8 a;
  const int col = 16 * db + r16;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = 16 * (e >> 2) + 4 * g + (e & 3);
    const int off = row * RB + (((col >> 2) ^ dv_swz<float, D>(row)) << 4) + 4 * (col & 3);
    a[e] = *reinterpret_cast<const float*>(vt + off);
  }
  return a;
}
template <>
__device__ __forceinline__ f32x8 vt_operand<float, 128>(const char* vt, int db, int r16, int g) {
  return vt_operand_f32<128>(vt, db, r16, g);
}
template <>
__device__ __forceinline__ f32x8 vt_operand<float, 64>(const char* vt, int db, int r16, int g) {
  return vt_operand_f32<64>(vt, db, r16, g);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, (kDecMinWaves<T, D>)) void decode_attn_kernel(const DecodeParams p) {
  using V8 = typename ElemTraits<T>::v8;
  using Tile = DecTile<T, D>;
  constexpr int KS = D / 32, DB = D / 16, H = D / 2;
  constexpr int RB = Tile::RB, CPR = Tile::CPR, NDMA = Tile::NDMA;
  __shared__ float2 s_cs[kWaves * H];
  __shared__ __attribute__((aligned(1024))) char s_raw[kDecLdsBytes<T, D>];

  const int L = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // The kernel-argument fields of the prologue, with the first request's
  // entry (the only one of a one-request launch) and every request's entry
  // one per lane (the host zeroes the unused ones), loaded in one round: the
  // empty asm needs them all at once, so they complete at one wait instead
  // of one dependent round per use.
  static_assert(C2KV_MAX_BATCH == 64, "one lane per request of a launch");
  const DecodeReq e = p.reqs[lane];
  const int total_wg = p.total_wg, num_reqs = p.num_reqs, req0 = p.req0, hq = p.hq, hkv = p.hkv, G = p.G;
  const float sl2 = p.scale_log2;
  const int64_t cap = p.cap;
  const DecodeReq rq0 = p.reqs[0];
  const void* const q_in = p.q;
  const void* const kn_in = p.k_new;
  const void* const vn_in = p.v_new;
  void* const kc = p.kc;
  void* const vc = p.vc;
  asm volatile("" : : "s"(total_wg), "s"(num_reqs), "s"(req0), "s"(hq), "s"(hkv), "s"(G), "s"(sl2), "s"(cap), "s"(rq0.wg0),
               "s"(rq0.cache_len), "s"(rq0.pos), "s"(rq0.nsplit), "s"(rq0.chunk), "s"(rq0.pbase), "s"(q_in),
               "s"(kn_in), "s"(vn_in), "s"(kc), "s"(vc), "v"(e.wg0), "v"(e.cache_len), "v"(e.pos), "v"(e.nsplit),
               "v"(e.chunk), "v"(e.pbase));
  if (L >= total_wg) return;
  const int r16 = lane & 15, g = lane >> 4;
  int ri = 0;
  DecodeReq rq = rq0;
  if (num_reqs != 1) {
    // the ballot over the requests' first workgroups picks this
    // workgroup's request, and its fields come from that request's lane
    ri = __builtin_amdgcn_readfirstlane(__popcll(__ballot(lane < num_reqs && e.wg0 <= L)) - 1);
    rq.wg0 = __builtin_amdgcn_readlane(e.wg0, ri);
    rq.cache_len = __builtin_amdgcn_readlane(e.cache_len, ri);
    rq.pos = __builtin_amdgcn_readlane(e.pos, ri);
    rq.nsplit = __builtin_amdgcn_readlane(e.nsplit, ri);
    rq.chunk = __builtin_amdgcn_readlane(e.chunk, ri);
    rq.pbase = __builtin_amdgcn_readlane(e.pbase, ri);
  }
  const int r = req0 + ri;
  const int local = L - rq.wg0;
  const int kvh = local / rq.nsplit, split = local % rq.nsplit;
  const int newk = rq.cache_len;                       // row of the new token
  const int k0 = split * rq.chunk, k1 = min(newk + 1, k0 + rq.chunk);
  const int nsteps = (k1 - k0 + 31) / 32;

  const int64_t head_base = ((int64_t)r * hkv + kvh) * cap;
  const T* knew = reinterpret_cast<const T*>(kn_in) + ((int64_t)r * hkv + kvh) * D;
  const T* vnew = reinterpret_cast<const T*>(vn_in) + ((int64_t)r * hkv + kvh) * D;
  char* vt = s_raw + wave * Tile::BYTES;
  // K and V rows of this head: rows at or past min(k1, newk) read as zeros
  // (the new token's key is loaded from k_new, its value patched in LDS)
  const int nrec = min(k1, newk) * RB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const char*>(kc) + head_base * RB), 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const char*>(vc) + head_base * RB), 0, nrec, 0x00020000);
  int voff[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int byte = j * 1024 + lane * 16;
    const int row = byte / RB, pc = (byte % RB) / 16;
    voff[j] = row * RB + ((pc ^ dv_swz<T, D>(row)) << 4);
  }

  V8 ka[2][KS];

  // ---- loads in the order they are consumed (the vector-memory counter
  // retires in order): RoPE frequency, query, then the first step's K and V
  const float freq = p.freqs.f[lane];                 // 64 entries, zero past H
  V8 qraw[KS];
  {
    const bool ok = r16 < G;
    const T* qrow = reinterpret_cast<const T*>(q_in) + ((int64_t)r * hq + kvh * G + (ok ? r16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      qraw[ks] = *reinterpret_cast<const V8*>(qrow + 32 * ks + 8 * g);
      qraw[ks + KS / 2] = *reinterpret_cast<const V8*>(qrow + H + 32 * ks + 8 * g);
    }
  }
  // (unconditional: a wave without a step reads past the resource, i.e.
  // zeros, so the counter waits below stay exact)
  dec_load_k<T, D>(ka, krs, k0 + 32 * wave, r16, g);
  dma_v_tile<NDMA>(vrs, vt, voff, (k0 + 32 * wave) * RB);

  // cos/sin of the decode position (shared by the query and the new key),
  // one table per wave so no workgroup barrier waits on the loads above
  float2* cs_tab = s_cs + wave * H;
  if (lane < H) {
    float c, s;
    rope_cs(rq.pos, freq, c, s);
    cs_tab[lane] = make_float2(c, s);
  }
  wave_lds_sync();

  // ---- queries of the group's heads as the B operand (column = head);
  // heads past G give zero columns
  V8 qB[KS];
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks) {
    float lo[8], hi[8];
    v8_to_f32<T>(qraw[ks], lo);
    v8_to_f32<T>(qraw[ks + KS / 2], hi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = cs_tab[32 * ks + 8 * g + e];
      float y0, y1;
      rope_pair(lo[e], hi[e], cs.x, cs.y, y0, y1);
      qB[ks][e] = from_f32<T>(r16 < G ? y0 : 0.f);
      qB[ks + KS / 2][e] = from_f32<T>(r16 < G ? y1 : 0.f);
    }
  }

  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  for (int st = wave; st < nsteps; st += kWaves) {
    const int key0 = k0 + 32 * st;
    if (st != wave) {
      wave_lds_sync();   // previous step's V^T reads are done before the DMA refills the tile
      dma_v_tile<NDMA>(vrs, vt, voff, key0 * RB);
    }
    const bool has_new = newk >= key0 && newk < key0 + 32;   // wave-uniform
    // the new token: rotate its key in place and append key and value
    if (has_new) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = key0 + 16 * kb + r16;
        if (key == newk) {
          T* kdst = reinterpret_cast<T*>(p.kc) + (head_base + key) * D;
#pragma unroll
          for (int ks = 0; ks < KS / 2; ++ks) {
            float lo[8], hi[8];
            v8_to_f32<T>(*reinterpret_cast<const V8*>(knew + 32 * ks + 8 * g), lo);
            v8_to_f32<T>(*reinterpret_cast<const V8*>(knew + H + 32 * ks + 8 * g), hi);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float2 cs = cs_tab[32 * ks + 8 * g + e];
              float y0, y1;
              rope_pair(lo[e], hi[e], cs.x, cs.y, y0, y1);
              ka[kb][ks][e] = from_f32<T>(y0);
              ka[kb][ks + KS / 2][e] = from_f32<T>(y1);
            }
            *reinterpret_cast<V8*>(kdst + 32 * ks + 8 * g) = ka[kb][ks];
            *reinterpret_cast<V8*>(kdst + H + 32 * ks + 8 * g) = ka[kb][ks + KS / 2];
          }
        }
      }
    }
    // ---- S^T = K Q^T over the 32 keys of the step
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s[0] = mma16(ka[0][ks], qB[ks], s[0]);
      s[1] = mma16(ka[1][ks], qB[ks], s[1]);
    }
    // ---- the wave's next step's K, in flight during this step's softmax
    // and P V (unconditional: past the resource it reads zeros, and the
    // V wait below counts on these loads being the newest)
    V8 kn[2][KS];
    dec_load_k<T, D>(kn, krs, key0 + 32 * kWaves, r16, g);
    // ---- online softmax over the step (column = head, 8 keys per lane)
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 16 * kb + 4 * g + i;
        const float v = key < k1 ? s[kb][i] * sl2 : -INFINITY;
        x[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = wave_max_16_32(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    float rs = 0.f;
    V8 pB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(x[kb][i] - mnew);
        rs += pv;
        pB[4 * kb + i] = from_f32<T>(pv);
      }
    l = l * alpha + rs;
    m = mnew;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    dec_wait_vmem_upto<kDecKLoads<T, D>>();   // the V tile has landed in LDS (only the K prefetch may be in flight)
    if (has_new) {
      // patch the new token's value row (zeros from the DMA) and append it
      const int row = newk - key0;
      if (lane < CPR) {
        const uint4 vv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(vnew) + lane * 16);
        *reinterpret_cast<uint4*>(vt + row * RB + ((lane ^ dv_swz<T, D>(row)) << 4)) = vv;
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(p.vc) + (head_base + newk) * RB + lane * 16) = vv;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = mma16(vt_operand<T, D>(vt, db, r16, g), pB, o[db]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[kb][ks] = kn[kb][ks];
  }

  // ---- combine the four waves (LDS reused), then write output or partial
  const float lt = wave_sum_16_32(l);
  dec_wait_vmem();   // no DMA into the tiles is still in flight
  __syncthreads();
  float* cmb = reinterpret_cast<float*>(s_raw);          // [kWaves][16][D + 2]
  constexpr int CROW = D + 2;
  if (r16 < G) {
    float* row = cmb + (wave * 16 + r16) * CROW;
    if (g == 0) { row[D] = m; row[D + 1] = lt; }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) row[16 * db + 4 * g + i] = o[db][i];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int hg = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cmb[(w * 16 + hg) * CROW + D]);
    float acc = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* row = cmb + (w * 16 + hg) * CROW;
      const float wt = row[D] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(row[D] - M);
      acc += row[d] * wt;
      ls += row[D + 1] * wt;
    }
    const int head = kvh * G + hg;
    if (rq.nsplit == 1) {
      T* orow = reinterpret_cast<T*>(p.o) + ((int64_t)r * p.hq + head) * D;
      orow[d] = from_f32<T>(acc / ls);
      if (d == 0 && p.lse) p.lse[(int64_t)r * p.hq + head] = (M + __log2f(ls)) * 0.69314718055994531f;
    } else {
      const int64_t idx = (int64_t)rq.pbase + (int64_t)head * rq.nsplit + split;
      p.part_o[idx * D + d] = acc;
      if (d == 0) p.part_ml[idx] = make_float2(M, ls);
    }
  }
}

// ---------------------------------------------------------------- merge
// The split partials of each output row (request of the launch, head,
// token) are combined by log-sum-exp.  WPR waves take one row: many rows
// with few splits each (a decode batch, a prefill) take one wave per row,
// few rows with many splits (decode of one request) take the workgroup's
// four waves per row.  Lane s of every wave of the row holds the (m, l) of
// split s (splits past 64 in further rounds); the row's 2 * WPR half-waves
// take the splits in turn, each lane covering D/32 consecutive dims, with
// kMergeNB partial rows per half-wave in flight, the first batch loaded
// together with the (m, l) pairs before the maximum is known.  The
// half-waves are added with one lane swap and, with WPR = 4, through LDS.
// Rows of requests with a single key chunk already hold their output.
constexpr int kMergeNB = 8;
constexpr int kMergeRowsPerWave = 512;   // at least this many rows: one wave per row

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return wave_max_16_32(x);
}

template <int N> struct MergeVec;
template <> struct MergeVec<4> { using type = f32x4; };
template <> struct MergeVec<2> { using type = float2; };

template <typename T, int D, int WPR>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeParams p) {
  constexpr int DPL = D / 32, NB = kMergeNB, HW = 2 * WPR;   // dims per lane, half-waves per row
  static_assert(WPR == 1 || WPR == kWaves, "one wave or the whole workgroup per row");
  using VF = typename MergeVec<DPL>::type;
  __shared__ float s_red[WPR > 1 ? kWaves * (D + 1) : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the kernel-argument fields, with the first request's entries (the only
  // ones of a one-request launch), in one round of scalar loads
  const int num_rows = p.num_rows, hq = p.hq, tq = p.tq, req0 = p.req0, nsplit0 = p.nsplit[0], pbase0 = p.pbase[0];
  // (and every request's entries, one per lane, for launches of several)
  static_assert(C2KV_MAX_BATCH == 64, "one lane per request of a launch");
  const int nsplit_l = p.nsplit[lane], pbase_l = p.pbase[lane];
  const float* const part_o = p.part_o;
  const float2* const part_ml = p.part_ml;
  void* const out = p.o;
  float* const lse = p.lse;
  asm volatile("" : : "s"(num_rows), "s"(hq), "s"(tq), "s"(req0), "s"(nsplit0), "s"(pbase0), "s"(part_o),
               "s"(part_ml), "s"(out), "s"(lse), "v"(nsplit_l), "v"(pbase_l));
  const int row = WPR == 1 ? blockIdx.x * kWaves + wave : blockIdx.x;
  if (row >= num_rows) return;
  const int rows_per_req = hq * tq;
  const int ri = num_rows == rows_per_req ? 0 : row / rows_per_req;
  const int rem = row - ri * rows_per_req;      // head * tq + t
  int nsplit = nsplit0, pbase = pbase0;
  if (ri != 0) {
    nsplit = __shfl(nsplit_l, ri);
    pbase = __shfl(pbase_l, ri);
  }
  if (nsplit <= 1) return;        // single-chunk requests were written directly
  const int64_t idx0 = (int64_t)pbase + (int64_t)rem * nsplit;
  const float* base = part_o + idx0 * D;
  const float2* ml = part_ml + idx0;
  const int half = lane >> 5, col = (lane & 31) * DPL;
  const int hw = (WPR == 1 ? 0 : 2 * wave) + half;     // this half-wave's first split
  auto load_o = [&](int s) { return *reinterpret_cast<const VF*>(base + (int64_t)min(s, nsplit - 1) * D + col); };
  // (m, l) of the first 64 splits, and the first batch of partial rows
  const float2 ml0 = ml[min(lane, nsplit - 1)];
  VF os[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) os[i] = load_o(hw + HW * i);
  float M = lane < nsplit ? ml0.x : -INFINITY;
  for (int s = lane + 64; s < nsplit; s += 64) M = fmaxf(M, ml[s].x);
  M = wave_max64(M);
  auto split_ml = [&](int s) {
    // splits below 64 come from their lane, the rest from memory (selected
    // as values: a conditional between the shuffled value and the memory
    // operand as lvalues makes the compiler spill the former to scratch and
    // load either through a flat pointer)
    float2 v = make_float2(__shfl(ml0.x, s & 63), __shfl(ml0.y, s & 63));
    if (s >= 64) {
      const float2 g = ml[min(s, nsplit - 1)];
      v = g;
    }
    return v;
  };
  VF acc;
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float ls = 0.f;
  for (int s0 = hw;; s0 += HW * NB) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s = s0 + HW * i;
      const float2 sm = split_ml(s);
      const float w = (s < nsplit && sm.x != -INFINITY) ? __builtin_amdgcn_exp2f(sm.x - M) : 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += os[i][e] * w;
      ls += s < nsplit ? sm.y * w : 0.f;
    }
    if (s0 + HW * NB >= nsplit) break;
#pragma unroll
    for (int i = 0; i < NB; ++i) os[i] = load_o(s0 + HW * (NB + i));
  }
  // add the odd half-wave into the even one (lanes l and l ^ 32)
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] += __shfl_xor(acc[e], 32);
  ls += __shfl_xor(ls, 32);
  if constexpr (WPR > 1) {
    if (half == 0) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) s_red[wave * (D + 1) + col + e] = acc[e];
      if (lane == 0) s_red[wave * (D + 1) + D] = ls;
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < WPR; ++w) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += s_red[w * (D + 1) + col + e];
      ls += s_red[w * (D + 1) + D];
    }
  }
  if (half == 0) {
    const int head = rem / tq, t = rem % tq;
    const int r = req0 + ri;
    T* orow = reinterpret_cast<T*>(out) + (((int64_t)r * tq + t) * hq + head) * D + col;
    const float inv = 1.f / ls;
#pragma unroll
    for (int e = 0; e < DPL; ++e) orow[e] = from_f32<T>(acc[e] * inv);
    if (lane == 0 && lse)
      lse[((int64_t)r * hq + head) * tq + t] = (M + __log2f(ls)) * 0.69314718055994531f;
  }
}

// ------------------------------------------------------------ launchers
template <typename T, int D>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_attn_kernel<T, D>), dim3(p.total_wg), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const DecodeParams& p, int dtype, int head_dim, hipStream_t st) {
  if (dtype == C2KV_BF16) return head_dim == 128 ? launch_decode_t<bf16, 128>(p, st) : launch_decode_t<bf16, 64>(p, st);
  return head_dim == 128 ? launch_decode_t<float, 128>(p, st) : launch_decode_t<float, 64>(p, st);
}

template <typename T, int D>
static hipError_t launch_merge_t(const MergeParams& p, hipStream_t st) {
  if (p.num_rows >= kMergeRowsPerWave)
    hipLaunchKernelGGL((merge_kernel<T, D, 1>), dim3((p.num_rows + kWaves - 1) / kWaves), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((merge_kernel<T, D, kWaves>), dim3(p.num_rows), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t st) {
  if (dtype == C2KV_BF16) return head_dim == 128 ? launch_merge_t<bf16, 128>(p, st) : launch_merge_t<bf16, 64>(p, st);
  return head_dim == 128 ? launch_merge_t<float, 128>(p, st) : launch_merge_t<float, 64>(p, st);
}

}  // namespace c2kv
