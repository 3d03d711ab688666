// Host side of the C2KV C ABI: argument validation (always before the first
// HIP call), workspace planning, kernel-argument tables and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "c2kv.h"
#include "c2kv_host.hpp"
#include "c2kv_launch.hpp"

using namespace c2kv;

namespace c2kv {
namespace host {

thread_local std::string g_err;

c2kv_status fail(c2kv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

c2kv_status ok() {
  g_err.clear();
  return C2KV_OK;
}

c2kv_status hip_fail(hipError_t e, const char* what) {
  return fail(C2KV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}


c2kv_status check_heads(int32_t hq, int32_t hkv, int32_t head_dim, c2kv_dtype dt) {
  if (dt != C2KV_BF16 && dt != C2KV_F32) return fail(C2KV_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (hq < 1 || hkv < 1) return fail(C2KV_ERR_INVALID_ARG, "hq=%d hkv=%d must be >= 1", hq, hkv);
  if (hq % hkv != 0) return fail(C2KV_ERR_INVALID_ARG, "hq=%d is not a multiple of hkv=%d", hq, hkv);
  if (hq / hkv > 16) return fail(C2KV_ERR_UNSUPPORTED, "hq/hkv=%d exceeds 16", hq / hkv);
  if (head_dim != 64 && head_dim != 128) return fail(C2KV_ERR_UNSUPPORTED, "head_dim=%d (64 or 128 supported)", head_dim);
  return C2KV_OK;
}

c2kv_status check_theta(float theta) {
  if (!(theta > 1.0f) || !std::isfinite(theta)) return fail(C2KV_ERR_INVALID_ARG, "rope_theta=%g must be finite and > 1", (double)theta);
  return C2KV_OK;
}

RopeFreqs make_freqs(int head_dim, float theta) {
  RopeFreqs f;
  std::memset(&f, 0, sizeof(f));
  for (int i = 0; i < head_dim / 2; ++i)
    f.f[i] = (float)std::pow((double)theta, -2.0 * (double)i / (double)head_dim);
  return f;
}

float scale_log2(int head_dim) {
  return (float)(1.4426950408889634 / std::sqrt((double)head_dim));
}

c2kv_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return C2KV_OK;
  if (!ws) return fail(C2KV_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned256(ws)) return fail(C2KV_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need) return fail(C2KV_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return C2KV_OK;
}

c2kv_status check_dev(const void* p, const char* name) {
  if (!p) return fail(C2KV_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(C2KV_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return C2KV_OK;
}

const char* last_error() { return g_err.c_str(); }

}  // namespace host
}  // namespace c2kv

using namespace c2kv::host;

namespace {

// ------------------------------------------------------------- extraction
// Workspace: rotated keys [rows][hkv][D] and the RoPE cos/sin table
// [max_n][D/2].  Values are read in place.
struct ExtractLayout {
  int64_t rows = 0;
  int32_t max_n = 0;
  size_t krot_off = 0, table_off = 0, total = 0;
};

c2kv_status extract_layout(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t hkv,
                           int32_t head_dim, c2kv_dtype dt, ExtractLayout& L) {
  if (!doc_lens) return fail(C2KV_ERR_INVALID_ARG, "doc_lens is NULL");
  if (num_docs < 1) return fail(C2KV_ERR_INVALID_ARG, "num_docs=%d must be >= 1", num_docs);
  if (ratio_k < 1) return fail(C2KV_ERR_INVALID_ARG, "ratio_k=%d must be >= 1", ratio_k);
  const int64_t rb = (int64_t)head_dim * elem_bytes(dt);
  L.rows = 0;
  L.max_n = 0;
  for (int32_t b = 0; b < num_docs; ++b) {
    const int32_t n = doc_lens[b];
    if (n < 1) return fail(C2KV_ERR_INVALID_ARG, "doc_lens[%d]=%d must be >= 1", b, n);
    if (n > (1 << 24)) return fail(C2KV_ERR_CAPACITY, "doc_lens[%d]=%d exceeds 2^24 positions", b, n);
    const int64_t m = num_slots_i(n, ratio_k);
    // a document's rows (plus one 64-key tile) are addressed with 32-bit offsets
    if ((n + m + 64) * hkv * rb >= ((int64_t)1 << 31))
      return fail(C2KV_ERR_CAPACITY, "document %d: %lld rows x %d KV heads exceed the 2 GiB tile window", b,
                  (long long)(n + m), hkv);
    L.rows += n + m;
    L.max_n = std::max(L.max_n, n);
  }
  if (L.rows >= ((int64_t)1 << 31)) return fail(C2KV_ERR_CAPACITY, "%lld packed rows exceed 2^31-1", (long long)L.rows);
  L.krot_off = 0;
  L.table_off = align_up((size_t)L.rows * hkv * head_dim * elem_bytes(dt));
  L.total = L.table_off + align_up((size_t)L.max_n * (head_dim / 2) * sizeof(float2));
  return C2KV_OK;
}

// Fill the per-launch document tables; returns the number of docs consumed.
int fill_extract_chunk(const int32_t* doc_lens, int32_t first, int32_t num_docs, int32_t ratio_k,
                       int32_t G, int32_t hkv, int64_t row0, ExtractParams& p, RotateParams& rp) {
  const int cnt = std::min<int>(C2KV_MAX_BATCH, num_docs - first);
  int64_t wg = 0, row = row0;
  for (int i = 0; i < cnt; ++i) {
    const int32_t n = doc_lens[first + i];
    const int32_t m = num_slots_i(n, ratio_k);
    ExtractDoc& d = p.docs[i];
    d.row0 = row;
    d.n = n;
    d.m = m;
    d.wg0 = (int32_t)wg;
    d.nwg_doc = (int32_t)ceil_div(ceil_div(n, kQW) * G, kWaves);
    d.nwg_slot = (int32_t)ceil_div(ceil_div(m, kQW) * G, kWaves);
    d.pad = 0;
    wg += (int64_t)hkv * (d.nwg_doc + d.nwg_slot);
    rp.docs[i].row0 = row;
    rp.docs[i].n = n;
    rp.docs[i].m = m;
    row += n + m;
  }
  p.num_docs = cnt;
  p.total_wg = (int32_t)wg;
  p.grid_wg = (int32_t)((wg + 7) / 8 * 8);
  rp.num_docs = cnt;
  rp.row_begin = row0;
  rp.row_end = row;
  return cnt;
}

}  // namespace

// ========================================================================
extern "C" {

const char* c2kv_version(void) { return "c2kv-mi355x 0.1.0 (gfx950)"; }

const char* c2kv_status_string(c2kv_status s) {
  // C callers may pass any int; read it as one (a C++ enum load of a value
  // outside the enumerators' range is undefined)
  int v;
  static_assert(sizeof(v) == sizeof(s), "c2kv_status is an int");
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case C2KV_OK: return "ok";
    case C2KV_ERR_INVALID_ARG: return "invalid argument";
    case C2KV_ERR_UNSUPPORTED: return "unsupported";
    case C2KV_ERR_WORKSPACE: return "workspace too small or misaligned";
    case C2KV_ERR_CAPACITY: return "capacity exceeded";
    case C2KV_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* c2kv_last_error(void) { return last_error(); }

int32_t c2kv_num_slots(int32_t n, int32_t k) {
  if (n < 0 || k < 1) return -1;
  return (int32_t)(((int64_t)n + k - 1) / k);
}

int32_t c2kv_slot_position(int32_t n, int32_t k, int32_t j) {
  const int32_t m = c2kv_num_slots(n, k);
  if (m < 0 || j < 0 || j >= m) return -1;
  return (int32_t)std::min<int64_t>((int64_t)j * k + k - 1, (int64_t)n - 1);
}

c2kv_status c2kv_rope_inv_freq(int32_t head_dim, float rope_theta, float* out) {
  if (!out) return fail(C2KV_ERR_INVALID_ARG, "out is NULL");
  if (head_dim < 2 || head_dim % 2 || head_dim > 2 * kMaxHalfDim)
    return fail(C2KV_ERR_INVALID_ARG, "head_dim=%d must be even and <= %d", head_dim, 2 * kMaxHalfDim);
  c2kv_status s;
  if ((s = check_theta(rope_theta))) return s;
  const RopeFreqs f = make_freqs(head_dim, rope_theta);
  std::memcpy(out, f.f, sizeof(float) * (head_dim / 2));
  return ok();
}

// ------------------------------------------------------------- extraction
size_t c2kv_workspace_size_extract(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t hkv,
                                   int32_t head_dim, c2kv_dtype dt) {
  ExtractLayout L;
  if (hkv < 1 || (head_dim != 64 && head_dim != 128)) return 0;
  if (extract_layout(doc_lens, num_docs, ratio_k, hkv, head_dim, dt, L)) return 0;
  return L.total;
}

c2kv_status c2kv_extract_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t sink_len,
                              int32_t hq, int32_t hkv, int32_t head_dim, float rope_theta, c2kv_dtype dt,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  return c2kv_extract_attn_ex(q, k, v, o, lse, doc_lens, num_docs, ratio_k, sink_len, hq, hkv, head_dim, rope_theta,
                              dt, 0u, workspace, ws_bytes, stream);
}

c2kv_status c2kv_extract_attn_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t sink_len,
                                 int32_t hq, int32_t hkv, int32_t head_dim, float rope_theta, c2kv_dtype dt,
                                 uint32_t flags, void* workspace, size_t ws_bytes, hipStream_t stream) {
  c2kv_status s;
  if (flags & ~C2KV_EXTRACT_ANCHOR) return fail(C2KV_ERR_INVALID_ARG, "flags=%u has unknown bits", flags);
  if ((s = check_heads(hq, hkv, head_dim, dt))) return s;
  if ((s = check_theta(rope_theta))) return s;
  if ((s = check_dev(q, "q")) || (s = check_dev(k, "k")) || (s = check_dev(v, "v")) || (s = check_dev(o, "o")))
    return s;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(C2KV_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (sink_len < 0) return fail(C2KV_ERR_INVALID_ARG, "sink_len=%d must be >= 0", sink_len);
  ExtractLayout L;
  if ((s = extract_layout(doc_lens, num_docs, ratio_k, hkv, head_dim, dt, L))) return s;
  if ((s = check_ws(workspace, ws_bytes, L.total))) return s;

  char* ws = static_cast<char*>(workspace);
  float2* table = reinterpret_cast<float2*>(ws + L.table_off);
  const RopeFreqs freqs = make_freqs(head_dim, rope_theta);
  hipError_t e = launch_rope_table(table, L.max_n, head_dim, freqs, stream);
  if (e != hipSuccess) return hip_fail(e, "rope table kernel launch");

  ExtractParams p;
  RotateParams rp;
  std::memset(&p, 0, sizeof(p));
  std::memset(&rp, 0, sizeof(rp));
  p.q = q; p.krot = ws + L.krot_off; p.v = v; p.o = o; p.lse = lse; p.rope = table;
  p.total_rows = L.rows;
  p.hq = hq; p.hkv = hkv; p.G = hq / hkv; p.ratio_k = ratio_k; p.sink_len = sink_len;
  p.scale_log2 = scale_log2(head_dim);
  p.anchor = (flags & C2KV_EXTRACT_ANCHOR) ? 1 : 0;
  rp.k = k; rp.krot = ws + L.krot_off; rp.rope = table;
  rp.hkv = hkv; rp.ratio_k = ratio_k;
  int64_t row = 0;
  for (int32_t b = 0; b < num_docs;) {
    const int cnt = fill_extract_chunk(doc_lens, b, num_docs, ratio_k, p.G, hkv, row, p, rp);
    e = launch_rotate_k(rp, dt, head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "key rotation kernel launch");
    e = launch_extract_attn(p, dt, head_dim, kExtractAttn, stream);
    if (e != hipSuccess) return hip_fail(e, "extraction attention kernel launch");
    row = rp.row_end;
    b += cnt;
  }
  return ok();
}

// ---------------------------------------------------------- extractor layer
}  // extern "C"

namespace {

struct LayerLayout {
  ExtractLayout ex;
  size_t h_off = 0, q_off = 0, o_off = 0, act_off = 0, ex_off = 0, ex_bytes = 0, total = 0;
};

c2kv_status layer_layout(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t dm, int32_t hq,
                         int32_t hkv, int32_t head_dim, int32_t ffn, c2kv_dtype dt, LayerLayout& L) {
  c2kv_status s;
  if ((s = check_heads(hq, hkv, head_dim, dt))) return s;
  if (dt != C2KV_BF16) return fail(C2KV_ERR_UNSUPPORTED, "the extractor layer runs in bf16 only");
  if (dm < 128 || dm % 128 || dm > 32768) return fail(C2KV_ERR_UNSUPPORTED, "dm=%d must be a multiple of 128 up to 32768", dm);
  if (ffn < 64 || ffn % 64 || ffn > (1 << 20)) return fail(C2KV_ERR_UNSUPPORTED, "ffn=%d must be a positive multiple of 64", ffn);
  if ((hq * head_dim) % 128 || (hkv * head_dim) % 128)
    return fail(C2KV_ERR_UNSUPPORTED, "hq*head_dim and hkv*head_dim must be multiples of 128");
  if ((s = extract_layout(doc_lens, num_docs, ratio_k, hkv, head_dim, dt, L.ex))) return s;
  const size_t T = (size_t)L.ex.rows, es = 2;
  if ((int64_t)T * std::max(dm, 2 * ffn) >= ((int64_t)1 << 40)) return fail(C2KV_ERR_CAPACITY, "layer buffers too large");
  size_t off = 0;
  L.h_off = off;   off += align_up(T * dm * es);
  L.q_off = off;   off += align_up(T * hq * head_dim * es);
  L.o_off = off;   off += align_up(T * hq * head_dim * es);
  L.act_off = off; off += align_up(T * ffn * es);
  L.ex_off = off;
  L.ex_bytes = c2kv_workspace_size_extract(doc_lens, num_docs, ratio_k, hkv, head_dim, dt);
  off += align_up(L.ex_bytes);
  L.total = off;
  return C2KV_OK;
}

// C = A * B^T over all rows [0, rows) with one weight matrix; epilogue epi
// (kEpiResidual adds `resid`, kEpiSwiglu writes silu(gate) * up).
hipError_t gemm_all_rows(const void* a, int64_t lda, const void* b, int K, int N, void* c, int64_t ldc,
                         const void* resid, int64_t rows, int epi, hipStream_t st) {
  GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.a = static_cast<const bf16*>(a);
  p.b0 = p.b1 = static_cast<const bf16*>(b);
  p.c0 = p.c1 = p.c2 = static_cast<bf16*>(c);
  p.r = static_cast<const bf16*>(resid);
  p.lda = lda; p.ldc0 = p.ldc1 = p.ldc2 = ldc; p.ldr = ldc;
  p.K = K; p.N = N; p.n1 = p.n2 = N;
  p.num_ranges = 1;
  p.ranges[0] = GemmRange{0, (int32_t)rows, 0, 0};
  p.m_tiles = (int32_t)ceil_div(rows, 128);
  p.n_tiles = N / 128;
  return launch_gemm(p, epi, st);
}

}  // namespace

extern "C" {

size_t c2kv_workspace_size_extract_layer(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t dm,
                                         int32_t hq, int32_t hkv, int32_t head_dim, int32_t ffn, c2kv_dtype dt) {
  LayerLayout L;
  if (layer_layout(doc_lens, num_docs, ratio_k, dm, hq, hkv, head_dim, ffn, dt, L)) return 0;
  return L.total;
}

c2kv_status c2kv_extract_layer(void* x, const void* slot_embed, const c2kv_layer_weights* w, void* k_out,
                               void* v_out, const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k,
                               int32_t sink_len, int32_t dm, int32_t hq, int32_t hkv, int32_t head_dim,
                               int32_t ffn, float rope_theta, float rms_eps, c2kv_dtype dt, void* workspace,
                               size_t ws_bytes, hipStream_t stream) {
  c2kv_status s;
  LayerLayout L;
  if ((s = layer_layout(doc_lens, num_docs, ratio_k, dm, hq, hkv, head_dim, ffn, dt, L))) return s;
  if ((s = check_theta(rope_theta))) return s;
  if (!(rms_eps >= 0.0f) || !std::isfinite(rms_eps)) return fail(C2KV_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (sink_len < 0) return fail(C2KV_ERR_INVALID_ARG, "sink_len=%d must be >= 0", sink_len);
  if (!w) return fail(C2KV_ERR_INVALID_ARG, "weights is NULL");
  if ((s = check_dev(x, "x")) || (s = check_dev(k_out, "k_out")) || (s = check_dev(v_out, "v_out")) ||
      (s = check_dev(w->attn_norm, "attn_norm")) || (s = check_dev(w->wqkv, "wqkv")) ||
      (s = check_dev(w->wqkv_c2, "wqkv_c2")) || (s = check_dev(w->wo, "wo")) ||
      (s = check_dev(w->ffn_norm, "ffn_norm")) || (s = check_dev(w->w_gate_up, "w_gate_up")) ||
      (s = check_dev(w->w_down, "w_down")))
    return s;
  if (slot_embed && (s = check_dev(slot_embed, "slot_embed"))) return s;
  if ((s = check_ws(workspace, ws_bytes, L.total))) return s;
  char* ws = static_cast<char*>(workspace);
  void* h = ws + L.h_off;
  void* q = ws + L.q_off;
  void* o = ws + L.o_off;
  void* act = ws + L.act_off;
  const int64_t T = L.ex.rows;
  const int qd = hq * head_dim, kd = hkv * head_dim, nqkv = qd + 2 * kd;
  hipError_t e;

  // slot rows take the shared vector (first layer)
  if (slot_embed) {
    int64_t row = 0;
    for (int32_t b0 = 0; b0 < num_docs; b0 += C2KV_MAX_BATCH) {
      SlotFillParams fp;
      std::memset(&fp, 0, sizeof(fp));
      fp.x = x; fp.embed = slot_embed; fp.dm = dm;
      int slots = 0;
      const int cnt = std::min<int>(C2KV_MAX_BATCH, num_docs - b0);
      for (int i = 0; i < cnt; ++i) {
        const int32_t n = doc_lens[b0 + i], m = num_slots_i(n, ratio_k);
        fp.docs[i] = SlotFillDoc{row + n, slots, 0};
        slots += m;
        row += n + m;
      }
      fp.num_docs = cnt;
      if ((e = launch_slot_fill(fp, slots, stream)) != hipSuccess) return hip_fail(e, "slot fill launch");
    }
  }
  if ((e = launch_rms_norm(x, w->attn_norm, h, T, dm, rms_eps, stream)) != hipSuccess) return hip_fail(e, "rms norm launch");

  // q | k | v: frozen weights on document rows, C2 weights on slot rows
  {
    int64_t row = 0;
    for (int32_t b0 = 0; b0 < num_docs; b0 += C2KV_MAX_BATCH) {
      GemmParams p;
      std::memset(&p, 0, sizeof(p));
      p.a = static_cast<const bf16*>(h);
      p.b0 = static_cast<const bf16*>(w->wqkv);
      p.b1 = static_cast<const bf16*>(w->wqkv_c2);
      p.c0 = static_cast<bf16*>(q);
      p.c1 = static_cast<bf16*>(k_out);
      p.c2 = static_cast<bf16*>(v_out);
      p.lda = dm; p.ldc0 = qd; p.ldc1 = kd; p.ldc2 = kd;
      p.K = dm; p.N = nqkv; p.n1 = qd; p.n2 = qd + kd;
      p.n_tiles = nqkv / 128;
      int tiles = 0, nr = 0;
      const int cnt = std::min<int>(C2KV_MAX_BATCH, num_docs - b0);
      for (int i = 0; i < cnt; ++i) {
        const int32_t n = doc_lens[b0 + i], m = num_slots_i(n, ratio_k);
        p.ranges[nr++] = GemmRange{(int32_t)row, n, 0, tiles};
        tiles += (int)ceil_div(n, 128);
        p.ranges[nr++] = GemmRange{(int32_t)(row + n), m, 1, tiles};
        tiles += (int)ceil_div(m, 128);
        row += n + m;
      }
      p.num_ranges = nr;
      p.m_tiles = tiles;
      if ((e = launch_gemm(p, kEpiStore, stream)) != hipSuccess) return hip_fail(e, "qkv projection launch");
    }
  }
  if ((s = c2kv_extract_attn(q, k_out, v_out, o, nullptr, doc_lens, num_docs, ratio_k, sink_len, hq, hkv, head_dim,
                             rope_theta, dt, ws + L.ex_off, L.ex_bytes, stream)))
    return s;
  if ((e = gemm_all_rows(o, qd, w->wo, qd, dm, x, dm, x, T, kEpiResidual, stream)) != hipSuccess)
    return hip_fail(e, "output projection launch");
  if ((e = launch_rms_norm(x, w->ffn_norm, h, T, dm, rms_eps, stream)) != hipSuccess) return hip_fail(e, "rms norm launch");
  if ((e = gemm_all_rows(h, dm, w->w_gate_up, dm, 2 * ffn, act, ffn, nullptr, T, kEpiSwiglu, stream)) != hipSuccess)
    return hip_fail(e, "gate/up projection launch");
  if ((e = gemm_all_rows(act, ffn, w->w_down, ffn, dm, x, dm, x, T, kEpiResidual, stream)) != hipSuccess)
    return hip_fail(e, "down projection launch");
  return ok();
}

// ------------------------------------------------------------ composition
size_t c2kv_workspace_size_compose(int32_t num_segs) {
  (void)num_segs;
  return 0;
}

}  // extern "C"

namespace {

// Validation shared by both compose entry points (no HIP call): geometry of
// every segment, request table, capacity and positions.  Fills the rows and
// the next position of each request.
c2kv_status compose_plan(const c2kv_segment* segs, int32_t num_segs, const int32_t* req_seg_ptr, int32_t num_reqs,
                         const int32_t* pos_base, int32_t ratio_k, int32_t hkv, int32_t head_dim, float rope_theta,
                         const void* cache_k, const void* cache_v, int64_t cap, const int32_t* pos_out,
                         const int32_t* cache_len_out, c2kv_dtype dt, std::vector<int32_t>& lens,
                         std::vector<int32_t>& nexts) {
  c2kv_status s;
  if ((s = check_heads(hkv, hkv, head_dim, dt))) return s;
  if ((s = check_theta(rope_theta))) return s;
  if (ratio_k < 1) return fail(C2KV_ERR_INVALID_ARG, "ratio_k=%d must be >= 1", ratio_k);
  if (!segs || num_segs < 1) return fail(C2KV_ERR_INVALID_ARG, "segs is NULL or num_segs=%d < 1", num_segs);
  if (!req_seg_ptr || num_reqs < 1) return fail(C2KV_ERR_INVALID_ARG, "req_seg_ptr is NULL or num_reqs < 1");
  if (!cache_len_out) return fail(C2KV_ERR_INVALID_ARG, "cache_len_out is NULL");
  if ((s = check_dev(cache_k, "cache_k")) || (s = check_dev(cache_v, "cache_v"))) return s;
  if (pos_out && (reinterpret_cast<uintptr_t>(pos_out) & 3u)) return fail(C2KV_ERR_INVALID_ARG, "pos_out misaligned");
  if (cap < 1) return fail(C2KV_ERR_INVALID_ARG, "cap=%lld must be >= 1", (long long)cap);
  if (req_seg_ptr[0] != 0 || req_seg_ptr[num_reqs] != num_segs)
    return fail(C2KV_ERR_INVALID_ARG, "req_seg_ptr must start at 0 and end at num_segs");
  const int64_t row_elems = (int64_t)hkv * head_dim;
  lens.assign(num_reqs, 0);
  nexts.assign(num_reqs, 0);
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (req_seg_ptr[r + 1] < req_seg_ptr[r]) return fail(C2KV_ERR_INVALID_ARG, "req_seg_ptr is not monotone at %d", r);
    int64_t rows = 0, pos = pos_base ? pos_base[r] : 0;
    if (pos < 0) return fail(C2KV_ERR_INVALID_ARG, "pos_base[%d] is negative", r);
    for (int32_t t = req_seg_ptr[r]; t < req_seg_ptr[r + 1]; ++t) {
      const c2kv_segment& g = segs[t];
      if ((s = check_dev(g.k, "segs[].k")) || (s = check_dev(g.v, "segs[].v"))) return s;
      if (g.doc_len < 1) return fail(C2KV_ERR_INVALID_ARG, "segs[%d].doc_len=%d must be >= 1", t, g.doc_len);
      if (g.flags & ~(C2KV_SEGMENT_HOST | C2KV_SEGMENT_NO_REALIGN))
        return fail(C2KV_ERR_INVALID_ARG, "segs[%d].flags=%d has unknown bits", t, g.flags);
      if (g.row_stride < row_elems || g.row_stride >= ((int64_t)1 << 31) || (g.row_stride * (int64_t)elem_bytes(dt)) % 16)
        return fail(C2KV_ERR_INVALID_ARG, "segs[%d].row_stride=%lld invalid (>= hkv*head_dim, 16-byte multiple)", t,
                    (long long)g.row_stride);
      rows += num_slots_i(g.doc_len, ratio_k);
      pos += g.doc_len;
    }
    if (rows > cap) return fail(C2KV_ERR_CAPACITY, "request %d composes %lld rows > cap=%lld", r, (long long)rows, (long long)cap);
    if (pos > (1 << 24)) return fail(C2KV_ERR_CAPACITY, "request %d reaches position %lld > 2^24", r, (long long)pos);
    lens[r] = (int32_t)rows;
    nexts[r] = (int32_t)pos;
  }

  return C2KV_OK;
}

// Page-locked host range check; returns the device-side address of `first`.
c2kv_status map_host_range(const void* host_ptr, size_t bytes, const void** dev_ptr) {
  if (!host_ptr || !dev_ptr) return fail(C2KV_ERR_INVALID_ARG, "host_ptr or dev_ptr is NULL");
  if (bytes == 0) return fail(C2KV_ERR_INVALID_ARG, "bytes must be >= 1");
  // address arithmetic in integers: a range that wraps is rejected before
  // any pointer is formed from it
  const uintptr_t first = reinterpret_cast<uintptr_t>(host_ptr);
  if (bytes - 1 > UINTPTR_MAX - first) return fail(C2KV_ERR_INVALID_ARG, "host range wraps the address space");
  const uintptr_t last = first + (bytes - 1);
  hipPointerAttribute_t a0, a1;
  std::memset(&a0, 0, sizeof(a0));
  std::memset(&a1, 0, sizeof(a1));
  hipError_t e0 = hipPointerGetAttributes(&a0, reinterpret_cast<const void*>(first));
  hipError_t e1 = e0 == hipSuccess ? hipPointerGetAttributes(&a1, reinterpret_cast<const void*>(last)) : hipSuccess;
  if (e0 != hipSuccess || e1 != hipSuccess) {
    (void)hipGetLastError();   // the query's own failure is not a launch error
    return fail(C2KV_ERR_INVALID_ARG, "host range [%p, +%zu) is not page-locked host memory (%s)", host_ptr, bytes,
                hipGetErrorString(e0 != hipSuccess ? e0 : e1));
  }
  if (a0.type != hipMemoryTypeHost || a1.type != hipMemoryTypeHost || !a0.devicePointer || !a1.devicePointer ||
      !a0.hostPointer || !a1.hostPointer)
    return fail(C2KV_ERR_INVALID_ARG, "host range [%p, +%zu) is not page-locked host memory mapped for the device",
                host_ptr, bytes);
  // the attributes may describe the queried address or its allocation's
  // base; the host-side distance to the reported host address maps either
  const uintptr_t d0 = reinterpret_cast<uintptr_t>(a0.devicePointer) + (first - reinterpret_cast<uintptr_t>(a0.hostPointer));
  const uintptr_t d1 = reinterpret_cast<uintptr_t>(a1.devicePointer) + (last - reinterpret_cast<uintptr_t>(a1.hostPointer));
  if (d1 - d0 != last - first)
    return fail(C2KV_ERR_INVALID_ARG, "host range [%p, +%zu) spans more than one page-locked allocation", host_ptr,
                bytes);
  *dev_ptr = reinterpret_cast<const void*>(d0);
  return C2KV_OK;
}

}  // namespace

extern "C" {

c2kv_status c2kv_compose(const c2kv_segment* segs, int32_t num_segs, const int32_t* req_seg_ptr, int32_t num_reqs,
                         const int32_t* pos_base, int32_t ratio_k, int32_t hkv, int32_t head_dim, float rope_theta,
                         void* cache_k, void* cache_v, int64_t cap, int32_t* pos_out, int32_t* cache_len_out,
                         int32_t* next_pos_out, c2kv_dtype dt, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  (void)workspace;
  (void)ws_bytes;
  c2kv_status s;
  std::vector<int32_t> lens, nexts;
  if ((s = compose_plan(segs, num_segs, req_seg_ptr, num_reqs, pos_base, ratio_k, hkv, head_dim, rope_theta, cache_k,
                        cache_v, cap, pos_out, cache_len_out, dt, lens, nexts)))
    return s;

  ComposeParams p;
  std::memset(&p, 0, sizeof(p));
  p.cache_k = cache_k; p.cache_v = cache_v; p.pos_out = pos_out; p.cap = cap;
  p.hkv = hkv; p.ratio_k = ratio_k; p.freqs = make_freqs(head_dim, rope_theta);
  const ComposeTiling tl = compose_tiling((int)elem_bytes(dt), head_dim, hkv);
  const int rpt = tl.rpt;
  p.rpt = tl.rpt; p.gpb = tl.gpb; p.nblk = tl.nblk;
  int ndocs = 0, nocc = 0, nruns = 0;
  int32_t tiles = 0;
  int32_t open_req = -1;      // request of the run being filled (-1: none)
  bool host_pass = false;
  std::vector<int32_t> doc_cnt(kComposeDocs, 0);
  auto flush = [&]() -> hipError_t {
    if (nocc == 0) return hipSuccess;
    p.num_docs = ndocs;
    p.num_occ = nocc;
    p.num_runs = nruns;
    p.run_occ0[nruns] = (uint16_t)nocc;
    // units: row tiles x head blocks x occurrence groups of each document
    int64_t units = 0;
    for (int d = 0; d < ndocs; ++d)
      units += ceil_div(num_slots_i(p.docs[d].n, ratio_k), rpt) * tl.nblk * ceil_div(doc_cnt[d], kComposeGroup);
    p.total_units = (int32_t)units;
    hipError_t e = launch_compose(p, dt, head_dim, host_pass, stream);
    ndocs = nocc = nruns = 0;
    tiles = 0;
    open_req = -1;
    std::fill(doc_cnt.begin(), doc_cnt.end(), 0);
    return e;
  };
  auto doc_index = [&](const c2kv_segment& g) -> int {
    for (int i = 0; i < ndocs; ++i) {
      const ComposeDoc& d = p.docs[i];
      if (d.k == g.k && d.v == g.v && d.stride == (int32_t)g.row_stride && d.n == g.doc_len) return i;
    }
    return -1;
  };
  // device segments first, then host-resident ones in launches of their own;
  // a run is broken wherever a segment of the other kind (or of another
  // launch) intervenes, so rows and positions advance only inside a run
  for (int pass = 0; pass < 2; ++pass) {
    host_pass = pass == 1;
    for (int32_t r = 0; r < num_reqs; ++r) {
      int32_t out_row = 0;
      int64_t pos = pos_base ? pos_base[r] : 0;
      open_req = -1;
      for (int32_t t = req_seg_ptr[r]; t < req_seg_ptr[r + 1]; ++t) {
        const c2kv_segment& g = segs[t];
        const int32_t m = num_slots_i(g.doc_len, ratio_k);
        const int32_t mt = (m + rpt - 1) / rpt;
        if (((g.flags & C2KV_SEGMENT_HOST) != 0) != host_pass) {
          open_req = -1;
        } else {
          int di = doc_index(g);
          if (nocc == kComposeOcc || (di < 0 && ndocs == kComposeDocs) ||
              (open_req != r && nruns == kComposeRuns) || (int64_t)tiles + mt >= ((int64_t)1 << 24)) {
            hipError_t e = flush();
            if (e != hipSuccess) return hip_fail(e, "compose kernel launch");
            di = -1;
          }
          if (di < 0) {
            di = ndocs++;
            p.docs[di] = ComposeDoc{g.k, g.v, (int32_t)g.row_stride, g.doc_len};
          }
          if (open_req != r) {
            p.run_req[nruns] = r;
            p.run_row0[nruns] = out_row;
            p.run_pos0[nruns] = (int32_t)pos;
            p.run_base[nruns] = pos_base ? pos_base[r] : 0;
            p.run_occ0[nruns] = (uint16_t)nocc;
            ++nruns;
            open_req = r;
          }
          p.occ_doc[nocc++] = (uint8_t)(di | ((g.flags & C2KV_SEGMENT_NO_REALIGN) ? kComposeNoRealign : 0));
          ++doc_cnt[di];
          tiles += mt;
        }
        out_row += m;
        pos += g.doc_len;
      }
    }
    hipError_t e = flush();
    if (e != hipSuccess) return hip_fail(e, "compose kernel launch");
  }
  for (int32_t r = 0; r < num_reqs; ++r) {
    cache_len_out[r] = lens[r];
    if (next_pos_out) next_pos_out[r] = nexts[r];
  }
  return ok();
}

size_t c2kv_workspace_size_compose_staged(const c2kv_segment* segs, int32_t num_segs, int32_t ratio_k, int32_t hkv,
                                          int32_t head_dim, c2kv_dtype dt) {
  if (!segs || num_segs < 1 || ratio_k < 1 || hkv < 1 || (head_dim != 64 && head_dim != 128) ||
      (dt != C2KV_BF16 && dt != C2KV_F32))
    return 0;
  size_t total = 0;
  for (int32_t t = 0; t < num_segs; ++t) {
    if (segs[t].doc_len < 1) return 0;
    total += 2 * align_up((size_t)num_slots_i(segs[t].doc_len, ratio_k) * hkv * head_dim * elem_bytes(dt));
  }
  return total;
}

c2kv_status c2kv_compose_staged(const c2kv_segment* segs, int32_t num_segs, const int32_t* req_seg_ptr,
                                int32_t num_reqs, const int32_t* pos_base, int32_t ratio_k, int32_t hkv,
                                int32_t head_dim, float rope_theta, void* cache_k, void* cache_v, int64_t cap,
                                int32_t* pos_out, int32_t* cache_len_out, int32_t* next_pos_out, c2kv_dtype dt,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
  c2kv_status s;
  std::vector<int32_t> lens, nexts;
  if ((s = compose_plan(segs, num_segs, req_seg_ptr, num_reqs, pos_base, ratio_k, hkv, head_dim, rope_theta, cache_k,
                        cache_v, cap, pos_out, cache_len_out, dt, lens, nexts)))
    return s;
  if ((s = check_ws(workspace, ws_bytes, c2kv_workspace_size_compose_staged(segs, num_segs, ratio_k, hkv, head_dim, dt))))
    return s;
  const size_t es = elem_bytes(dt), row_bytes = (size_t)hkv * head_dim * es;
  // every source range must be page-locked, so that the copies below are
  // asynchronous DMA on `stream` (checked for all segments before the first)
  for (int32_t t = 0; t < num_segs; ++t) {
    const size_t m = (size_t)num_slots_i(segs[t].doc_len, ratio_k);
    const size_t span = ((m - 1) * (size_t)segs[t].row_stride) * es + row_bytes;
    const void* unused;
    if ((s = map_host_range(segs[t].k, span, &unused)) || (s = map_host_range(segs[t].v, span, &unused))) return s;
  }
  std::vector<c2kv_segment> staged(num_segs);
  char* base = static_cast<char*>(workspace);
  size_t off = 0;
  for (int32_t t = 0; t < num_segs; ++t) {
    const c2kv_segment& g = segs[t];
    const size_t m = (size_t)num_slots_i(g.doc_len, ratio_k);
    const size_t pitch = (size_t)g.row_stride * es;
    void* dk = base + off;
    off += align_up(m * row_bytes);
    void* dv = base + off;
    off += align_up(m * row_bytes);
    hipError_t e;
    if (pitch == row_bytes) {
      e = hipMemcpyAsync(dk, g.k, m * row_bytes, hipMemcpyHostToDevice, stream);
      if (e == hipSuccess) e = hipMemcpyAsync(dv, g.v, m * row_bytes, hipMemcpyHostToDevice, stream);
    } else {
      e = hipMemcpy2DAsync(dk, row_bytes, g.k, pitch, row_bytes, m, hipMemcpyHostToDevice, stream);
      if (e == hipSuccess) e = hipMemcpy2DAsync(dv, row_bytes, g.v, pitch, row_bytes, m, hipMemcpyHostToDevice, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "host-to-device copy of a slot cache");
    staged[t] = c2kv_segment{dk, dv, (int64_t)hkv * head_dim, g.doc_len, g.flags & C2KV_SEGMENT_NO_REALIGN};
  }
  return c2kv_compose(staged.data(), num_segs, req_seg_ptr, num_reqs, pos_base, ratio_k, hkv, head_dim, rope_theta,
                      cache_k, cache_v, cap, pos_out, cache_len_out, next_pos_out, dt, nullptr, 0, stream);
}

c2kv_status c2kv_workspace_init(void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (ws_bytes == 0) return ok();
  if (!workspace || !aligned256(workspace)) return fail(C2KV_ERR_INVALID_ARG, "workspace NULL or not 256-byte aligned");
  if (ws_bytes % 4) return fail(C2KV_ERR_INVALID_ARG, "ws_bytes=%zu is not a multiple of 4", ws_bytes);
  hipError_t e = launch_fill_zero(workspace, ws_bytes, stream);
  if (e != hipSuccess) return hip_fail(e, "fill kernel launch");
  return ok();
}

// ------------------------------------------------- host-resident slot caches
c2kv_status c2kv_host_device_ptr(const void* host_ptr, size_t bytes, const void** dev_ptr) {
  c2kv_status s = map_host_range(host_ptr, bytes, dev_ptr);
  return s ? s : ok();
}

// ---------------------------------------------------------------- testing
size_t c2kv_workspace_size_mask_cells(void) { return 256; }

c2kv_status c2kv_mask_cells(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t sink_len,
                            uint64_t* counts_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return c2kv_mask_cells_ex(doc_lens, num_docs, ratio_k, sink_len, 0u, counts_out, workspace, ws_bytes, stream);
}

c2kv_status c2kv_mask_cells_ex(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t sink_len,
                               uint32_t flags, uint64_t* counts_out, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  c2kv_status s;
  if (flags & ~C2KV_EXTRACT_ANCHOR) return fail(C2KV_ERR_INVALID_ARG, "flags=%u has unknown bits", flags);
  if (!counts_out) return fail(C2KV_ERR_INVALID_ARG, "counts_out is NULL");
  if (sink_len < 0) return fail(C2KV_ERR_INVALID_ARG, "sink_len=%d must be >= 0", sink_len);
  ExtractLayout L;
  if ((s = extract_layout(doc_lens, num_docs, ratio_k, 1, 64, C2KV_F32, L))) return s;
  if ((s = check_ws(workspace, ws_bytes, c2kv_workspace_size_mask_cells()))) return s;
  uint64_t* counts = static_cast<uint64_t*>(workspace);
  hipError_t e = launch_fill_zero(counts, 64, stream);
  if (e != hipSuccess) return hip_fail(e, "fill kernel launch");
  ExtractParams p;
  RotateParams rp;
  std::memset(&p, 0, sizeof(p));
  std::memset(&rp, 0, sizeof(rp));
  p.hq = 1; p.hkv = 1; p.G = 1; p.ratio_k = ratio_k; p.sink_len = sink_len; p.counts = counts;
  p.anchor = (flags & C2KV_EXTRACT_ANCHOR) ? 1 : 0;
  p.total_rows = L.rows;
  int64_t row = 0;
  for (int32_t b = 0; b < num_docs;) {
    const int cnt = fill_extract_chunk(doc_lens, b, num_docs, ratio_k, 1, 1, row, p, rp);
    e = launch_extract_attn(p, C2KV_F32, 64, kExtractCount, stream);
    if (e != hipSuccess) return hip_fail(e, "mask count kernel launch");
    row = rp.row_end;
    b += cnt;
  }
  uint64_t host[5];
  e = hipMemcpyAsync(host, counts, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  std::memcpy(counts_out, host, sizeof(host));
  return ok();
}

size_t c2kv_workspace_size_tile_schedule(void) { return 256; }

c2kv_status c2kv_tile_schedule(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t sink_len,
                               int32_t hq, int32_t hkv, uint32_t flags, c2kv_tile_entry* entries,
                               int64_t capacity, int64_t* count_out, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  c2kv_status s;
  if (flags & ~C2KV_EXTRACT_ANCHOR) return fail(C2KV_ERR_INVALID_ARG, "flags=%u has unknown bits", flags);
  if (!count_out) return fail(C2KV_ERR_INVALID_ARG, "count_out is NULL");
  if (sink_len < 0) return fail(C2KV_ERR_INVALID_ARG, "sink_len=%d must be >= 0", sink_len);
  if ((s = check_heads(hq, hkv, 64, C2KV_F32))) return s;
  if (capacity < 0) return fail(C2KV_ERR_INVALID_ARG, "capacity=%lld must be >= 0", (long long)capacity);
  if (capacity > 0 && (s = check_dev(entries, "entries"))) return s;
  ExtractLayout L;
  if ((s = extract_layout(doc_lens, num_docs, ratio_k, hkv, 64, C2KV_F32, L))) return s;
  if ((s = check_ws(workspace, ws_bytes, c2kv_workspace_size_tile_schedule()))) return s;
  uint64_t* counter = static_cast<uint64_t*>(workspace);
  hipError_t e = launch_fill_zero(counter, 64, stream);
  if (e != hipSuccess) return hip_fail(e, "fill kernel launch");
  ExtractParams p;
  RotateParams rp;
  std::memset(&p, 0, sizeof(p));
  std::memset(&rp, 0, sizeof(rp));
  p.hq = hq; p.hkv = hkv; p.G = hq / hkv; p.ratio_k = ratio_k; p.sink_len = sink_len;
  p.counts = counter; p.entries = entries; p.entry_cap = capacity;
  p.anchor = (flags & C2KV_EXTRACT_ANCHOR) ? 1 : 0;
  p.total_rows = L.rows;
  int64_t row = 0;
  for (int32_t b = 0; b < num_docs;) {
    const int cnt = fill_extract_chunk(doc_lens, b, num_docs, ratio_k, p.G, hkv, row, p, rp);
    p.doc_base = b;
    e = launch_extract_attn(p, C2KV_F32, 64, kExtractDump, stream);
    if (e != hipSuccess) return hip_fail(e, "tile dump kernel launch");
    row = rp.row_end;
    b += cnt;
  }
  uint64_t total = 0;
  e = hipMemcpyAsync(&total, counter, sizeof(total), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  *count_out = (int64_t)total;
  if ((int64_t)total > capacity && (entries || capacity > 0))
    return fail(C2KV_ERR_CAPACITY, "the schedule has %llu entries, capacity is %lld", (unsigned long long)total,
                (long long)capacity);
  return ok();
}

}  // extern "C"
