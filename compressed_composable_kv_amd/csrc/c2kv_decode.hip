// Decode over a composed cache, and the split-K merge shared with prefill.
//
// Decode (the C2KV explainer's experimental-results section: every
// generated token reads the whole compressed cache) is bound by reading the
// cache once.  A workgroup owns one (request, KV head, key chunk); ALL query
// heads of the group sit in the 16 columns of one wave's MFMA tiles, and the
// four waves stream disjoint 32-key steps of the chunk, so every K/V byte is
// read from HBM exactly once and never shared through LDS:
//   * K goes straight from global memory into MFMA A-operand registers
//     (S^T = K Q^T, keys on the M side, heads on N);
//   * V is transposed through a small wave-private LDS tile for the
//     O^T += V^T P^T product;
//   * the new token's key is rotated (RoPE at the decode position) in the
//     registers that would have loaded it, used as is, and written to the
//     cache together with its value -- no separate append launch;
//   * the four waves' (max, sum, O) are combined in LDS; with one chunk per
//     (request, KV head) the workgroup writes the final output, otherwise a
//     partial row that merge_kernel combines by log-sum-exp.
#include "c2kv_device.hpp"
#include "c2kv_launch.hpp"

namespace c2kv {

constexpr int kDecVPad = 8;                    // elements of padding per V^T row
constexpr int kDecVRow = 32 + kDecVPad;

// 4-key group swizzle of the 32-key V^T rows (conflict-free operand reads).
__device__ __forceinline__ int dvt_group(int d, int kg) { return kg ^ ((d >> 3) & 7); }

// Order this wave's own LDS writes before its reads of other lanes' data
// (and the reads of one step before the next step's writes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T> __device__ __forceinline__ uint32_t elem_bits(const uint4& x, int e);
template <> __device__ __forceinline__ uint32_t elem_bits<bf16>(const uint4& x, int e) {
  const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
template <> __device__ __forceinline__ uint32_t elem_bits<float>(const uint4& x, int e) {
  return e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w;
}

template <typename T> __device__ __forceinline__ void v8_to_f32(const typename ElemTraits<T>::v8& v, float* f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = to_f32(v[e]);
}

template <typename T, int D>
constexpr int kDecMinWaves = (kWaves * D * kDecVRow * (int)sizeof(T) * 2 <= 160 * 1024) ? 2 : 1;

template <typename T, int D>
__global__ __launch_bounds__(kThreads, (kDecMinWaves<T, D>)) void decode_attn_kernel(const DecodeParams p) {
  using V8 = typename ElemTraits<T>::v8;
  using V4 = typename ElemTraits<T>::v4;
  constexpr int KS = D / 32, DB = D / 16, H = D / 2;
  constexpr int CE = ElemTraits<T>::kChunk, CPR = D / CE;
  constexpr int VTASK = 8 * CPR;                       // (4 keys x 1 chunk) tasks per step
  constexpr int VPT = (VTASK + 63) / 64;
  constexpr int kVtElems = D * kDecVRow;
  __shared__ float2 s_cs[H];
  __shared__ __attribute__((aligned(16))) T s_vt[kWaves * kVtElems];
  static_assert(kWaves * 16 * (D + 2) * sizeof(float) <= sizeof(T) * kWaves * kVtElems,
                "wave-combine scratch must fit in the V^T tiles");

  const int L = blockIdx.x;
  if (L >= p.total_wg) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  int ri = 0;
  while (ri + 1 < p.num_reqs && p.reqs[ri + 1].wg0 <= L) ++ri;
  const DecodeReq rq = p.reqs[ri];
  const int r = p.req0 + ri;
  const int local = L - rq.wg0;
  const int kvh = local / rq.nsplit, split = local % rq.nsplit;
  const int G = p.G;
  const int newk = rq.cache_len;                       // row of the new token
  const int k0 = split * p.chunk, k1 = min(newk + 1, k0 + p.chunk);

  // cos/sin of the decode position, shared by the query and the new key
  if (tid < H) {
    float c, s;
    rope_cs(rq.pos, p.freqs.f[tid], c, s);
    s_cs[tid] = make_float2(c, s);
  }
  __syncthreads();

  // ---- queries of the group's heads as the B operand (column = head)
  V8 qB[KS];
  {
    const bool ok = r16 < G;
    const T* qrow = reinterpret_cast<const T*>(p.q) + ((int64_t)r * p.hq + kvh * G + (ok ? r16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      float lo[8], hi[8];
      if (ok) {
        v8_to_f32<T>(*reinterpret_cast<const V8*>(qrow + 32 * ks + 8 * g), lo);
        v8_to_f32<T>(*reinterpret_cast<const V8*>(qrow + H + 32 * ks + 8 * g), hi);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = hi[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = s_cs[32 * ks + 8 * g + e];
        float y0, y1;
        rope_pair(lo[e], hi[e], cs.x, cs.y, y0, y1);
        qB[ks][e] = from_f32<T>(y0);
        qB[ks + KS / 2][e] = from_f32<T>(y1);
      }
    }
  }

  const int64_t head_base = ((int64_t)r * p.hkv + kvh) * p.cap;
  const T* kc = reinterpret_cast<const T*>(p.kc) + head_base * D;
  const T* vc = reinterpret_cast<const T*>(p.vc) + head_base * D;
  const T* knew = reinterpret_cast<const T*>(p.k_new) + ((int64_t)r * p.hkv + kvh) * D;
  const T* vnew = reinterpret_cast<const T*>(p.v_new) + ((int64_t)r * p.hkv + kvh) * D;
  T* vt = s_vt + wave * kVtElems;

  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const int nsteps = (k1 - k0 + 31) / 32;

  for (int st = wave; st < nsteps; st += kWaves) {
    const int key0 = k0 + 32 * st;
    // ---- K: A operand rows key0 + 16 kb + r16, k-group g
    V8 ka[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = key0 + 16 * kb + r16;
      if (key < k1 && key != newk) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[kb][ks] = *reinterpret_cast<const V8*>(kc + (int64_t)key * D + 32 * ks + 8 * g);
      } else if (key == newk && key < k1) {
        // the new token: rotate its key here and append key and value
        T* kdst = reinterpret_cast<T*>(p.kc) + (head_base + key) * D;
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) {
          float lo[8], hi[8];
          v8_to_f32<T>(*reinterpret_cast<const V8*>(knew + 32 * ks + 8 * g), lo);
          v8_to_f32<T>(*reinterpret_cast<const V8*>(knew + H + 32 * ks + 8 * g), hi);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float2 cs = s_cs[32 * ks + 8 * g + e];
            float y0, y1;
            rope_pair(lo[e], hi[e], cs.x, cs.y, y0, y1);
            ka[kb][ks][e] = from_f32<T>(y0);
            ka[kb][ks + KS / 2][e] = from_f32<T>(y1);
          }
          *reinterpret_cast<V8*>(kdst + 32 * ks + 8 * g) = ka[kb][ks];
          *reinterpret_cast<V8*>(kdst + H + 32 * ks + 8 * g) = ka[kb][ks + KS / 2];
        }
        T* vdst = reinterpret_cast<T*>(p.vc) + (head_base + key) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          *reinterpret_cast<V8*>(vdst + 32 * ks + 8 * g) = *reinterpret_cast<const V8*>(vnew + 32 * ks + 8 * g);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) ka[kb][ks][e] = from_f32<T>(0.f);
      }
    }
    // ---- V: 4 keys x one 16-byte chunk per task, transposed into LDS
    uint4 vr[VPT][4];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int t = lane + 64 * i;
      const int kg = t / CPR, dc = t % CPR;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = key0 + 4 * kg + rr;
        const T* src = key == newk ? vnew + dc * CE : vc + (int64_t)key * D + dc * CE;
        vr[i][rr] = (t < VTASK && key < k1) ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
      }
    }
    // ---- S^T = K Q^T over the 32 keys of the step
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s[0] = mma16(ka[0][ks], qB[ks], s[0]);
      s[1] = mma16(ka[1][ks], qB[ks], s[1]);
    }
    wave_lds_sync();   // previous step's V^T reads are done
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int t = lane + 64 * i;
      if (t >= VTASK) break;
      const int kg = t / CPR, dc = t % CPR;
#pragma unroll
      for (int e = 0; e < CE; ++e) {
        const int d = dc * CE + e;
        T* dst = vt + d * kDecVRow + dvt_group(d, kg) * 4;
        if constexpr (sizeof(T) == 2) {
          const uint32_t h0 = elem_bits<T>(vr[i][0], e), h1 = elem_bits<T>(vr[i][1], e);
          const uint32_t h2 = elem_bits<T>(vr[i][2], e), h3 = elem_bits<T>(vr[i][3], e);
          *reinterpret_cast<uint2*>(dst) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(elem_bits<T>(vr[i][0], e), elem_bits<T>(vr[i][1], e),
                                                      elem_bits<T>(vr[i][2], e), elem_bits<T>(vr[i][3], e));
        }
      }
    }
    // ---- online softmax over the step (column = head, 8 keys per lane)
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 16 * kb + 4 * g + i;
        const float v = key < k1 ? s[kb][i] * p.scale_log2 : -INFINITY;
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
    wave_lds_sync();   // this step's V^T writes are visible to the wave
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 16 * db + r16;
      const T* row = vt + d * kDecVRow;
      const V4 lo = *reinterpret_cast<const V4*>(row + dvt_group(d, g) * 4);
      const V4 hi = *reinterpret_cast<const V4*>(row + dvt_group(d, 4 + g) * 4);
      V8 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = lo[i]; a[4 + i] = hi[i]; }
      o[db] = mma16(a, pB, o[db]);
    }
  }

  // ---- combine the four waves (LDS reused), then write output or partial
  const float lt = wave_sum_16_32(l);
  __syncthreads();
  float* cmb = reinterpret_cast<float*>(s_vt);          // [kWaves][16][D + 2]
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
      float* prow = p.part + (((int64_t)ri * p.hq + head) * p.nsplit_stride + split) * (D + 4);
      prow[d] = acc;
      if (d == 0) { prow[D] = M; prow[D + 1] = ls; }
    }
  }
}

// ---------------------------------------------------------------- merge
// One workgroup per output row (request of the launch, head, token): the
// split partials [o(D) | m | l] of that row are combined by log-sum-exp.
// Rows of requests with a single key chunk already hold their output.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeParams p) {
  constexpr int C4 = D / 4, SG = kThreads / C4;        // split groups
  __shared__ float s_red[kThreads];
  __shared__ __attribute__((aligned(16))) float s_acc[SG][D];
  __shared__ float s_l[SG];
  const int row = blockIdx.x;
  if (row >= p.num_rows) return;
  const int tid = threadIdx.x;
  const int ri = row / (p.hq * p.tq);
  const int nsplit = p.nsplit[ri];
  if (nsplit <= 1) return;        // single-chunk requests were written directly
  const float* base = p.part + (int64_t)row * p.nsplit_stride * (D + 4);
  // max over splits
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += kThreads) M = fmaxf(M, base[(int64_t)s * (D + 4) + D]);
  s_red[tid] = M;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
    __syncthreads();
  }
  M = s_red[0];
  // weighted sums: thread (split group sg, 4-wide chunk d4)
  const int sg = tid / C4, d4 = tid % C4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float ls = 0.f;
#pragma unroll 4
  for (int s = sg; s < nsplit; s += SG) {
    const float* pr = base + (int64_t)s * (D + 4);
    const float ms = pr[D];
    const float wt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    acc += *reinterpret_cast<const f32x4*>(pr + 4 * d4) * wt;
    ls += pr[D + 1] * wt;
  }
  *reinterpret_cast<f32x4*>(&s_acc[sg][4 * d4]) = acc;
  if (d4 == 0) s_l[sg] = ls;
  __syncthreads();
  if (tid < D) {
    float a = 0.f, lsum = 0.f;
#pragma unroll
    for (int j = 0; j < SG; ++j) { a += s_acc[j][tid]; lsum += s_l[j]; }
    const int rem = row % (p.hq * p.tq);
    const int head = rem / p.tq, t = rem % p.tq;
    const int r = p.req0 + ri;
    T* orow = reinterpret_cast<T*>(p.o) + (((int64_t)r * p.tq + t) * p.hq + head) * D;
    orow[tid] = from_f32<T>(a / lsum);
    if (tid == 0 && p.lse) p.lse[((int64_t)r * p.hq + head) * p.tq + t] = (M + __log2f(lsum)) * 0.69314718055994531f;
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
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3(p.num_rows), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t st) {
  if (dtype == C2KV_BF16) return head_dim == 128 ? launch_merge_t<bf16, 128>(p, st) : launch_merge_t<bf16, 64>(p, st);
  return head_dim == 128 ? launch_merge_t<float, 128>(p, st) : launch_merge_t<float, 64>(p, st);
}

}  // namespace c2kv
