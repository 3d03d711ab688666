// Host side of the prefill and decode entry points: argument validation
// (always before the first HIP call), the split-K plan, workspace layout and
// the kernel-argument tables of the cache attention, decode and merge
// launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "c2kv.h"
#include "c2kv_host.hpp"
#include "c2kv_launch.hpp"

using namespace c2kv;
using namespace c2kv::host;

namespace {

// ------------------------------------------------------ prefill / decode
// Split plan shared by the size query and the call.  Keys of a request are
// cut into pieces processed by separate workgroups, at most C2KV_MAX_SPLITS
// per request.
//  * prefill: one `chunk` for all requests, a multiple of the kernel's key
//    tile, sized so that a launch has about one workgroup per CU;
//  * decode: the launch is sized to one round of the workgroups the chip
//    holds at once (kDecodeSlots), and each request's keys are cut into
//    pieces of nearly equal length (chunk_r, a multiple of one wave's 32-key
//    step), so every workgroup streams about the same number of bytes and
//    no second, partly filled round trails the first.
constexpr int64_t kDecodeSlots = 3 * 256;   // decode workgroups resident at once on a 256-CU MI355X
// Minimum keys per decode piece (a multiple of one wave's 32-key step).
// Measured on the Llama layer's batch-1 decode (8 KV heads x 8193 keys) on
// one MI355X, per step: 12.1 us at 288 keys (232 workgroups), 12.2 at 320,
// 12.3 at 352, 12.6 at 384, 13.3 at 416, and 15.1 at 256 (264 workgroups,
// more than the CUs); the Qwen2.5 pool (pieces of about 1100 keys) is
// unaffected.
constexpr int64_t kDecodeMinKeys = 288;
constexpr int64_t kPrefillSlots = 256;      // prefill workgroups per launch: one per CU (two measured slower)
struct CachePlan {
  bool decode = false;
  int32_t nug = 0, nblk_q = 0, chunk = 0;
  std::vector<int32_t> nsplit, chunk_r, pbase;   // pbase: first partial of the request within its launch
  size_t part_off = 0, ml_off = 0, total = 0;
};

c2kv_status cache_plan(const int32_t* cache_len, int32_t num_reqs, int32_t tq, int32_t hq, int32_t hkv,
                       int32_t head_dim, c2kv_dtype dt, int64_t cap_or_neg, bool decode, CachePlan& P) {
  if (!cache_len) return fail(C2KV_ERR_INVALID_ARG, "cache_len is NULL");
  if (num_reqs < 1) return fail(C2KV_ERR_INVALID_ARG, "num_reqs=%d must be >= 1", num_reqs);
  if (tq < 1) return fail(C2KV_ERR_INVALID_ARG, "tq=%d must be >= 1", tq);
  const int32_t G = hq / hkv;
  P.decode = decode;
  P.nblk_q = (int32_t)ceil_div(tq, kQW);
  P.nug = decode ? 1 : (int32_t)ceil_div((int64_t)P.nblk_q * G, kWaves);
  int64_t total_keys = 0, max_len = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    const int64_t c = cache_len[r];
    if (c < 0) return fail(C2KV_ERR_INVALID_ARG, "cache_len[%d]=%lld is negative", r, (long long)c);
    if (cap_or_neg >= 0 && c + tq > cap_or_neg)
      return fail(C2KV_ERR_CAPACITY, "cache_len[%d]=%lld + %d new rows exceed cap=%lld", r, (long long)c, tq,
                  (long long)cap_or_neg);
    if (c + tq >= ((int64_t)1 << 30)) return fail(C2KV_ERR_CAPACITY, "request %d has too many rows", r);
    total_keys += c + tq;
    max_len = std::max(max_len, c + tq);
  }
  // keys per unit of the chunk search: one wave's step for decode, a
  // workgroup's step (a tile per wave group) for prefill
  const int64_t step = decode ? 32 : 2 * kBN;
  P.nsplit.resize(num_reqs);
  P.chunk_r.resize(num_reqs);
  if (!decode) {
    int64_t chunk = ceil_div(total_keys * hkv * P.nug, kPrefillSlots);
    chunk = std::max<int64_t>(step, ceil_div(chunk, step) * step);
    chunk = std::max<int64_t>(chunk, ceil_div(ceil_div(max_len, C2KV_MAX_SPLITS), step) * step);
    P.chunk = (int32_t)chunk;
    for (int32_t r = 0; r < num_reqs; ++r) {
      P.nsplit[r] = (int32_t)ceil_div(cache_len[r] + tq, chunk);
      P.chunk_r[r] = (int32_t)chunk;
    }
  } else {
    // per-workgroup key budget w: the smallest multiple of the step whose
    // pieces fit the resident slots of every launch of C2KV_MAX_BATCH
    // requests (or one piece per request and head, if even that does not fit)
    // (the workgroup count only falls as w grows: binary search over
    // multiples of the step)
    auto fits = [&](int64_t w) {
      for (int32_t r0 = 0; r0 < num_reqs; r0 += C2KV_MAX_BATCH) {
        int64_t wgs = 0;
        for (int32_t r = r0; r < std::min(num_reqs, r0 + C2KV_MAX_BATCH); ++r)
          wgs += ceil_div(cache_len[r] + tq, w) * hkv;
        if (wgs > kDecodeSlots) return false;
      }
      return true;
    };
    // (at least kDecodeMinKeys per piece: shorter pieces leave the first
    // loads' latency and the partial write unamortised)
    int64_t lo = std::max<int64_t>(kDecodeMinKeys / step, ceil_div(ceil_div(total_keys * hkv, kDecodeSlots), step));
    lo = std::max<int64_t>(lo, ceil_div(ceil_div(max_len, C2KV_MAX_SPLITS), step));
    int64_t hi = std::max<int64_t>(lo, ceil_div(max_len, step));   // one piece per request: the fallback
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (fits(mid * step)) hi = mid;
      else lo = mid + 1;
    }
    const int64_t w = lo * step;
    P.chunk = (int32_t)w;
    for (int32_t r = 0; r < num_reqs; ++r) {
      const int64_t len = cache_len[r] + tq;
      const int64_t n = ceil_div(len, w);
      const int64_t c = ceil_div(ceil_div(len, n), 32) * 32;   // equal pieces, whole 32-key steps
      P.chunk_r[r] = (int32_t)c;
      P.nsplit[r] = (int32_t)ceil_div(len, c);
    }
  }
  // compact split partials: requests with more than one piece, in launch
  // order, hq * tq * nsplit partials each
  size_t max_part = 0;
  P.pbase.assign(num_reqs, 0);
  for (int32_t r0 = 0; r0 < num_reqs; r0 += C2KV_MAX_BATCH) {
    const int32_t r1 = std::min(num_reqs, r0 + C2KV_MAX_BATCH);
    size_t cnt = 0;
    for (int32_t r = r0; r < r1; ++r) {
      P.pbase[r] = (int32_t)cnt;
      if (P.nsplit[r] > 1) cnt += (size_t)hq * tq * P.nsplit[r];
    }
    if (cnt >= ((size_t)1 << 31)) return fail(C2KV_ERR_CAPACITY, "%zu split partials in one launch", cnt);
    max_part = std::max(max_part, cnt);
  }
  P.part_off = 0;
  P.ml_off = P.part_off + align_up(max_part * head_dim * sizeof(float));
  P.total = P.ml_off + align_up(max_part * sizeof(float2));
  return C2KV_OK;
}

// Validation of a prefill / decode call (no HIP call); fills the plan.
c2kv_status cache_validate(const void* q, const void* k_new, const void* v_new, void* cache_k, void* cache_v,
                           int64_t cap, const int32_t* cache_len, const int32_t* q_pos0, int32_t num_reqs,
                           int32_t tq, bool decode, int32_t hq, int32_t hkv, int32_t head_dim, float rope_theta,
                           void* o, float* lse, c2kv_dtype dt, CachePlan& P) {
  c2kv_status s;
  if ((s = check_heads(hq, hkv, head_dim, dt))) return s;
  if ((s = check_theta(rope_theta))) return s;
  if ((s = check_dev(q, "q")) || (s = check_dev(k_new, "k_new")) || (s = check_dev(v_new, "v_new")) ||
      (s = check_dev(cache_k, "cache_k")) || (s = check_dev(cache_v, "cache_v")) || (s = check_dev(o, "o")))
    return s;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(C2KV_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (!q_pos0) return fail(C2KV_ERR_INVALID_ARG, "q_pos is NULL");
  if (cap < 1) return fail(C2KV_ERR_INVALID_ARG, "cap=%lld must be >= 1", (long long)cap);
  // per-head byte offsets are 32-bit in the kernels, including the decode
  // wave's prefetch of its next step (up to 128 + 31 rows past a chunk)
  if ((cap + 256) * head_dim * elem_bytes(dt) >= ((int64_t)1 << 31))
    return fail(C2KV_ERR_CAPACITY, "cap=%lld rows of one head exceed 2 GiB", (long long)cap);
  if ((s = cache_plan(cache_len, num_reqs, tq, hq, hkv, head_dim, dt, cap, decode, P))) return s;
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (q_pos0[r] < 0 || (int64_t)q_pos0[r] + tq > (1 << 24))
      return fail(C2KV_ERR_CAPACITY, "q_pos[%d]=%d + %d tokens outside [0, 2^24]", r, q_pos0[r], tq);
  }
  return C2KV_OK;
}

c2kv_status cache_attention(const void* q, const void* k_new, const void* v_new, void* cache_k, void* cache_v,
                            int64_t cap, const int32_t* cache_len, const int32_t* q_pos0, int32_t num_reqs,
                            int32_t tq, bool decode, int32_t hq, int32_t hkv, int32_t head_dim, float rope_theta,
                            void* o, float* lse, c2kv_dtype dt, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
  c2kv_status s;
  CachePlan P;
  if ((s = cache_validate(q, k_new, v_new, cache_k, cache_v, cap, cache_len, q_pos0, num_reqs, tq, decode, hq, hkv,
                          head_dim, rope_theta, o, lse, dt, P)))
    return s;
  if ((s = check_ws(workspace, ws_bytes, P.total))) return s;

  char* ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws + P.part_off);
  float2* part_ml = reinterpret_cast<float2*>(ws + P.ml_off);
  const RopeFreqs freqs = make_freqs(head_dim, rope_theta);
  const int32_t G = hq / hkv;
  for (int32_t r0 = 0; r0 < num_reqs; r0 += C2KV_MAX_BATCH) {
    const int32_t cnt = std::min<int32_t>(C2KV_MAX_BATCH, num_reqs - r0);
    int32_t stride = 0;
    for (int32_t i = 0; i < cnt; ++i) stride = std::max(stride, P.nsplit[r0 + i]);
    hipError_t e;
    if (decode) {
      DecodeParams dp;
      std::memset(&dp, 0, sizeof(dp));
      dp.q = q; dp.k_new = k_new; dp.v_new = v_new; dp.kc = cache_k; dp.vc = cache_v; dp.o = o; dp.lse = lse;
      dp.part_o = part_o; dp.part_ml = part_ml;
      dp.cap = cap; dp.req0 = r0; dp.num_reqs = cnt; dp.hq = hq; dp.hkv = hkv; dp.G = G;
      dp.scale_log2 = scale_log2(head_dim); dp.freqs = freqs;
      int64_t wg = 0;
      for (int32_t i = 0; i < cnt; ++i) {
        dp.reqs[i].wg0 = (int32_t)wg;
        dp.reqs[i].cache_len = cache_len[r0 + i];
        dp.reqs[i].pos = q_pos0[r0 + i];
        dp.reqs[i].nsplit = P.nsplit[r0 + i];
        dp.reqs[i].chunk = P.chunk_r[r0 + i];
        dp.reqs[i].pbase = P.pbase[r0 + i];
        wg += (int64_t)hkv * P.nsplit[r0 + i];
      }
      dp.total_wg = (int32_t)wg;
      e = launch_decode_attn(dp, dt, head_dim, stream);
      if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    } else {
      CacheParams cp;
      std::memset(&cp, 0, sizeof(cp));
      cp.q = q; cp.k_new = k_new; cp.v_new = v_new;
      cp.kc = cache_k; cp.vc = cache_v; cp.o = o; cp.lse = lse; cp.part_o = part_o; cp.part_ml = part_ml;
      cp.cap = cap; cp.req0 = r0; cp.num_reqs = cnt; cp.tq = tq; cp.hq = hq; cp.hkv = hkv; cp.G = G;
      cp.nblk_q = P.nblk_q; cp.nug = P.nug; cp.chunk = P.chunk;
      cp.scale_log2 = scale_log2(head_dim);
      cp.freqs = freqs;
      int64_t wg = 0;
      for (int32_t i = 0; i < cnt; ++i) {
        cp.reqs[i].wg0 = (int32_t)wg;
        cp.reqs[i].cache_len = cache_len[r0 + i];
        cp.reqs[i].nsplit = P.nsplit[r0 + i];
        cp.reqs[i].pbase = P.pbase[r0 + i];
        cp.reqs[i].pos0 = q_pos0[r0 + i];
        wg += (int64_t)hkv * P.nsplit[r0 + i] * P.nug;
      }
      cp.total_wg = (int32_t)wg;
      cp.grid_wg = (int32_t)((wg + 7) / 8 * 8);
      e = launch_prefill_attn(cp, dt, head_dim, stream);
      if (e != hipSuccess) return hip_fail(e, "prefill attention kernel launch");
    }
    if (stride > 1) {
      MergeParams mp;
      std::memset(&mp, 0, sizeof(mp));
      mp.part_o = part_o; mp.part_ml = part_ml;
      mp.o = o; mp.lse = lse; mp.req0 = r0; mp.num_rows = cnt * hq * tq; mp.hq = hq; mp.tq = tq;
      for (int32_t i = 0; i < cnt; ++i) { mp.nsplit[i] = P.nsplit[r0 + i]; mp.pbase[i] = P.pbase[r0 + i]; }
      e = launch_merge(mp, dt, head_dim, stream);
      if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    }
  }
  return ok();
}

}  // namespace

extern "C" {

size_t c2kv_workspace_size_prefill(const int32_t* cache_len, int32_t num_reqs, int32_t tq, int32_t hq, int32_t hkv,
                                   int32_t head_dim, c2kv_dtype dt) {
  if (hq < 1 || hkv < 1 || hq % hkv) return 0;
  CachePlan P;
  if (cache_plan(cache_len, num_reqs, tq, hq, hkv, head_dim, dt, -1, false, P)) return 0;
  return std::max<size_t>(P.total, kAlign);
}

size_t c2kv_workspace_size_decode(const int32_t* cache_len, int32_t num_reqs, int32_t hq, int32_t hkv,
                                  int32_t head_dim, c2kv_dtype dt) {
  if (hq < 1 || hkv < 1 || hq % hkv) return 0;
  CachePlan P;
  if (cache_plan(cache_len, num_reqs, 1, hq, hkv, head_dim, dt, -1, true, P)) return 0;
  return std::max<size_t>(P.total, kAlign);
}

c2kv_status c2kv_attn_prefill(const void* q, const void* k_new, const void* v_new, void* cache_k, void* cache_v,
                              int64_t cap, const int32_t* cache_len, const int32_t* q_pos0, int32_t num_reqs,
                              int32_t tq, int32_t hq, int32_t hkv, int32_t head_dim, float rope_theta, void* o,
                              float* lse, c2kv_dtype dt, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return cache_attention(q, k_new, v_new, cache_k, cache_v, cap, cache_len, q_pos0, num_reqs, tq, false, hq, hkv,
                         head_dim, rope_theta, o, lse, dt, workspace, ws_bytes, stream);
}

c2kv_status c2kv_attn_decode(const void* q, const void* k_new, const void* v_new, void* cache_k, void* cache_v,
                             int64_t cap, const int32_t* cache_len, const int32_t* q_pos, int32_t num_reqs,
                             int32_t hq, int32_t hkv, int32_t head_dim, float rope_theta, void* o, float* lse,
                             c2kv_dtype dt, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return cache_attention(q, k_new, v_new, cache_k, cache_v, cap, cache_len, q_pos, num_reqs, 1, true, hq, hkv,
                         head_dim, rope_theta, o, lse, dt, workspace, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Split-K partials of c2kv_attn_decode_noalloc: one array per GPU, never
// freed.  Host code uses only the per-device addresses from
// hipGetSymbolAddress, never the array's name.
__device__ __align__(256) char scratch[C2KV_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the stream's device, looked up once per device
// with that device current.
c2kv_status scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(C2KV_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (e2 != hipSuccess) return hip_fail(e2, "hipSetDevice");
    if (!p || !aligned256(p)) return fail(C2KV_ERR_HIP, "scratch address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return C2KV_OK;
}

}  // namespace

extern "C" c2kv_status c2kv_attn_decode_noalloc(const void* q, const void* k_new, const void* v_new, void* cache_k,
                                                void* cache_v, int64_t cap, const int32_t* cache_len,
                                                const int32_t* q_pos, int32_t num_reqs, int32_t hq, int32_t hkv,
                                                int32_t head_dim, float rope_theta, void* o, float* lse,
                                                c2kv_dtype dt, hipStream_t stream) {
  c2kv_status s;
  // the same validation as c2kv_attn_decode, before any HIP call
  CachePlan P;
  if ((s = cache_validate(q, k_new, v_new, cache_k, cache_v, cap, cache_len, q_pos, num_reqs, 1, true, hq, hkv,
                          head_dim, rope_theta, o, lse, dt, P)))
    return s;
  if (P.total > C2KV_NOALLOC_SCRATCH_BYTES)
    return fail(C2KV_ERR_WORKSPACE, "the step needs %zu bytes of split scratch; the static scratch holds %u", P.total,
                (unsigned)C2KV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_for_stream(stream, &ws))) return s;
  return cache_attention(q, k_new, v_new, cache_k, cache_v, cap, cache_len, q_pos, num_reqs, 1, true, hq, hkv,
                         head_dim, rope_theta, o, lse, dt, ws, C2KV_NOALLOC_SCRATCH_BYTES, stream);
}
