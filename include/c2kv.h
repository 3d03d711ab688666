/*
 * c2kv.h -- C ABI of the C2KV hot path on AMD Instinct MI355X (gfx950).
 *
 * C2KV (compressed, composable KV-cache reuse) has three data-parallel steps
 * on its hot path, each exported here:
 *
 *   c2kv_extract_attn   structured-flow attention of the extractor over one
 *                       batch of documents (doc tokens + C2 slot tokens)
 *   c2kv_extract_layer  that attention inside a whole extractor layer
 *                       (norms, frozen / C2 projections, FFN)
 *   c2kv_compose        RoPE-realigned concatenation of pre-RoPE slot K/V of
 *                       several documents into one contiguous cache
 *   c2kv_attn_prefill   question prefill over a composed cache (GQA)
 *   c2kv_attn_decode    one decode step over a composed cache (GQA, split-K)
 *
 * Stored slot caches may stay in page-locked host memory: compose reads them
 * in place (c2kv_host_device_ptr) or copies them in first
 * (c2kv_compose_staged).
 *
 * Sources, cited by page and section:
 *   [Explainer] "C2KV: Compressed and Composable KV Cache Reuse for Efficient
 *               LLM Inference", paper-daily.com explainer page.
 *   [Abstract]  arXiv 2607.17715 abstract page (arxivdaily.com).
 *   [KV-size]   "LLM inference optimisation: KV cache compression schemes"
 *               (feinterview.poetries.top), Llama 3 / GQA paragraph.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns c2kv_status.  On failure c2kv_last_error()
 *   returns a thread-local message describing the first problem found.
 * - All arguments are validated on the host BEFORE any HIP call, so a bad
 *   argument never reaches the GPU (and can be tested on a machine without
 *   one).  Device pointers are checked for NULL and 16-byte alignment only.
 *   Host-memory ranges (the two host-pool functions) are additionally
 *   checked with HIP pointer queries before any copy or launch.
 * - Device tensors are dense, row-major, in the element type `dt`
 *   (C2KV_BF16 or C2KV_F32).  head_dim must be 64 or 128; hq % hkv == 0;
 *   hq / hkv <= 16.
 * - Ownership: the caller owns every buffer (tensors, caches, workspace).
 *   The library allocates no memory and keeps no state between calls beyond
 *   the thread-local error string.  Host arrays are read during the call
 *   and may be released when it returns.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *   the legacy default stream).  Results are valid once the stream has
 *   reached the work.  Calls are reentrant; two calls that are in flight at
 *   the same time must not share a workspace.
 * - workspace: device memory, 256-byte aligned, of at least the size the
 *   matching c2kv_workspace_size_* function returns for the same arguments.
 *   Its contents on entry are ignored and are undefined on return.
 * - Per-call tables (documents, requests) are passed to the GPU as kernel
 *   arguments in chunks of at most C2KV_MAX_BATCH entries per launch, so
 *   extract/prefill/decode perform no host-to-device copies and may be
 *   captured in a HIP graph.  Compose passes its table the same way (the
 *   distinct documents, one byte per occurrence and the requests' runs of
 *   occurrences: up to 64 documents, 1024 occurrences and 64 runs per
 *   launch) and needs no workspace.
 */
#ifndef C2KV_H_
#define C2KV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum c2kv_status {
  C2KV_OK = 0,
  C2KV_ERR_INVALID_ARG = 1,   /* NULL pointer, bad shape, dtype, k < 1, ... */
  C2KV_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. head_dim 96) */
  C2KV_ERR_WORKSPACE = 3,     /* workspace too small or misaligned */
  C2KV_ERR_CAPACITY = 4,      /* cache rows would exceed `cap`, or an index overflows */
  C2KV_ERR_HIP = 5            /* a HIP launch or runtime call failed */
} c2kv_status;

typedef enum c2kv_dtype {
  C2KV_BF16 = 0,              /* bfloat16 storage, fp32 accumulation */
  C2KV_F32 = 1                /* fp32 storage and accumulation */
} c2kv_dtype;

#define C2KV_MAX_BATCH 64     /* documents / requests per kernel launch */
#define C2KV_MAX_SPLITS 512   /* split-K chunks per (request, KV head) */

/* ---- library information ------------------------------------------------ */

const char* c2kv_version(void);
const char* c2kv_status_string(c2kv_status s);
/* Message of the last failure on the calling thread ("" if none). */
const char* c2kv_last_error(void);

/* ---- closed forms (host only, no GPU) ----------------------------------- */

/* Number of C2 slots of an n-token document at compression ratio k:
 * ceil(n / k).  [Explainer] "C2 token" section: one slot per k document
 * tokens; a trailing partial block also gets a slot.  Returns -1 when
 * n < 0 or k < 1. */
int32_t c2kv_num_slots(int32_t n, int32_t k);

/* Extraction-time position of slot j: the position of the last token of
 * the block it summarises, min(j*k + k - 1, n - 1).  [Explainer] section on
 * positions at concatenation (3, 7, ... at k = 4).  Returns -1 for
 * arguments outside 0 <= j < c2kv_num_slots(n, k). */
int32_t c2kv_slot_position(int32_t n, int32_t k, int32_t j);

/* RoPE inverse frequencies theta^(-2i/d), i < head_dim/2, computed in
 * double and rounded once to float, written to out[head_dim/2] (host).
 * Every kernel rotates with exactly these values: angle = fp32(pos * f_i),
 * x'_i = x_i c - x_{i+d/2} s, x'_{i+d/2} = x_{i+d/2} c + x_i s with each
 * product and sum rounded to fp32 (no fused multiply-add). */
c2kv_status c2kv_rope_inv_freq(int32_t head_dim, float rope_theta, float* out);

/* ---- extraction: structured-flow attention ------------------------------- */

/* Workspace bytes for c2kv_extract_attn with the same arguments. */
size_t c2kv_workspace_size_extract(const int32_t* doc_lens, int32_t num_docs,
                                   int32_t ratio_k, int32_t hkv, int32_t head_dim,
                                   c2kv_dtype dt);

/* Attention of the C2 extractor over a batch of independently extracted
 * documents.  [Explainer] "structured information flow" section and its mask
 * figure; "C2 token" section; positions section.  [Abstract]: structured
 * attention flow of the sidecar extractor.
 *
 * Rows of document b are packed as [n_b document tokens | m_b slots],
 * m_b = c2kv_num_slots(n_b, ratio_k), documents back to back.
 *   q      device [sum_T][hq][head_dim]   pre-RoPE queries
 *   k, v   device [sum_T][hkv][head_dim]  pre-RoPE keys, values
 *   o      device [sum_T][hq][head_dim]   output (may not alias q/k/v)
 *   lse    device [hq][sum_T] float or NULL: natural-log sum-exp of the
 *          scaled scores of each row
 *   doc_lens  host [num_docs], each >= 1; num_docs >= 1
 * Queries and keys are rotated at the extraction positions (document token
 * i at i, slot j at c2kv_slot_position(n, k, j)); V is not rotated.  Row
 * visibility (rows = queries, columns = keys):
 *   doc i  -> doc c  iff c <= i;  doc -> slot never;
 *   slot j -> doc c  iff c < min(sink_len, n) or c / k == j;
 *   slot j -> slot j' iff j' <= j.
 * The sink is the document's first min(sink_len, n) tokens; the pages fix
 * sink_len = ratio_k.  Query head h reads KV head h / (hq / hkv).  Scale is
 * 1/sqrt(head_dim).  Key/value tiles with no visible cell are never loaded.
 * The workspace holds the rotated keys and the cos/sin table; q, k and v
 * are read in place.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, CAPACITY (sum_T >= 2^31
 * rows, or one document's rows of all KV heads reach 2 GiB), HIP. */
c2kv_status c2kv_extract_attn(const void* q, const void* k, const void* v,
                              void* o, float* lse,
                              const int32_t* doc_lens, int32_t num_docs,
                              int32_t ratio_k, int32_t sink_len,
                              int32_t hq, int32_t hkv, int32_t head_dim,
                              float rope_theta, c2kv_dtype dt,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/* Extraction with options.  flags = 0 is c2kv_extract_attn.
 * C2KV_EXTRACT_ANCHOR: the anchor-token ablation of [Explainer]
 * experimental-results section (the extra tokens and the document tokens
 * see each other both ways, which entangles the cache with its context).
 * Slot rows act as the anchors: a document row sees the document rows up to
 * itself and every slot row of its document; a slot row sees every row of
 * its document.  Positions, RoPE, GQA and outputs as for c2kv_extract_attn;
 * same workspace.  Errors: as c2kv_extract_attn, INVALID_ARG for unknown
 * flag bits. */
#define C2KV_EXTRACT_ANCHOR 1u
c2kv_status c2kv_extract_attn_ex(const void* q, const void* k, const void* v,
                                 void* o, float* lse,
                                 const int32_t* doc_lens, int32_t num_docs,
                                 int32_t ratio_k, int32_t sink_len,
                                 int32_t hq, int32_t hkv, int32_t head_dim,
                                 float rope_theta, c2kv_dtype dt, uint32_t flags,
                                 void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- extraction: one extractor layer around the attention ---------------- */

/* Weights of one layer (device pointers, bf16, row-major).  [Explainer]
 * "C2 token" section: document tokens keep the frozen Q/K/V projections,
 * slot tokens use their own per-layer C2 projections, and everything else
 * (output projection, FFN) is the frozen model's.  The norm and FFN form
 * the pre-norm decoder layer of the base models the pages evaluate
 * (Llama3.1-8B, Qwen2.5, Qwen3). */
typedef struct c2kv_layer_weights {
  const void* attn_norm;   /* [dm]  RMSNorm gain before attention */
  const void* wqkv;        /* [(hq+2*hkv)*head_dim][dm] frozen Q/K/V (rows: q heads, k heads, v heads) */
  const void* wqkv_c2;     /* same shape: the C2 projections, used for slot rows */
  const void* wo;          /* [dm][hq*head_dim] output projection */
  const void* ffn_norm;    /* [dm]  RMSNorm gain before the FFN */
  const void* w_gate_up;   /* [2*ffn][dm]: blocks of 16 gate rows, each followed by the 16 up rows of the
                              same FFN columns (rows 32b..32b+15: gate 16b..16b+15; 32b+16..32b+31: up) */
  const void* w_down;      /* [dm][ffn] */
} c2kv_layer_weights;

size_t c2kv_workspace_size_extract_layer(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k,
                                         int32_t dm, int32_t hq, int32_t hkv, int32_t head_dim,
                                         int32_t ffn, c2kv_dtype dt);

/* One layer of the frozen model with the C2 extractor attached, over a batch
 * of independently extracted documents packed as for c2kv_extract_attn.
 *   x           device [sum_T][dm] hidden states, updated in place:
 *               x += attn(...) W_o^T, then x += FFN(RMSNorm(x))
 *   slot_embed  device [dm] or NULL: when given, every slot row of x is set
 *               to this shared vector first (the first layer: all C2 tokens
 *               share one learnable embedding, [Explainer] "C2 token")
 *   k_out,v_out device [sum_T][hkv][head_dim]: this layer's pre-RoPE keys
 *               and values; their slot rows are the stored C2KV of the layer
 * Steps: h = RMSNorm(x) * attn_norm; [q|k|v] = h W^T with W = wqkv for
 * document rows and wqkv_c2 for slot rows; o = c2kv_extract_attn(q, k, v)
 * (structured mask, RoPE at extraction positions, sink_len, rope_theta);
 * x += o W_o^T; h = RMSNorm(x) * ffn_norm; x += (silu(h Wg^T) * (h Wu^T)) Wd^T.
 * RMSNorm(x) = x / sqrt(mean(x^2) + rms_eps).  Matrix products accumulate
 * in fp32; h, q, the attention output and the SwiGLU product (formed from
 * the fp32 gate and up sums) are rounded to bf16, and each residual add is
 * done in fp32 and rounded once.
 * bf16 only.  Requires dm % 128 == 0, ffn % 64 == 0, and hq*head_dim and
 * hkv*head_dim multiples of 128.
 * Errors: INVALID_ARG, UNSUPPORTED (fp32, shapes off the tile grid),
 * WORKSPACE, CAPACITY, HIP. */
c2kv_status c2kv_extract_layer(void* x, const void* slot_embed, const c2kv_layer_weights* w,
                               void* k_out, void* v_out,
                               const int32_t* doc_lens, int32_t num_docs,
                               int32_t ratio_k, int32_t sink_len,
                               int32_t dm, int32_t hq, int32_t hkv, int32_t head_dim, int32_t ffn,
                               float rope_theta, float rms_eps, c2kv_dtype dt,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- composition --------------------------------------------------------- */

/* One document's stored slot cache: `doc_len` is the document's ORIGINAL
 * token count n (its slots number c2kv_num_slots(n, ratio_k)).  k and v
 * point at slot 0's row; row j of head h is at element offset
 * j*row_stride + h*head_dim.  Pre-RoPE keys. */
typedef struct c2kv_segment {
  const void* k;
  const void* v;
  int64_t row_stride;   /* elements between consecutive slot rows (>= hkv*head_dim) */
  int32_t doc_len;      /* original document length n >= 1 */
  int32_t flags;        /* 0, or C2KV_SEGMENT_HOST and/or C2KV_SEGMENT_NO_REALIGN */
} c2kv_segment;

/* Segment flag: k and v are device addresses of page-locked host memory
 * (from c2kv_host_device_ptr).  c2kv_compose composes such segments in
 * launches of their own with a small grid (16 workgroups): the host link,
 * not the GPU, bounds them, and few concurrent readers keep its transfers
 * efficient.  Device segments keep the full grid. */
#define C2KV_SEGMENT_HOST 1

/* Segment flag for the ablation without positional realignment
 * ([Explainer] experimental-results section: removing the realignment
 * lowers quality): the segment's slots are rotated at their extraction
 * positions plus pos_base only, not shifted by the original lengths of the
 * documents before it.  Rows, lengths and next_pos_out are unchanged. */
#define C2KV_SEGMENT_NO_REALIGN 2

size_t c2kv_workspace_size_compose(int32_t num_segs);

/* Compose the slot caches of several documents, per request, in the given
 * order.  [Explainer] "overall flow" section (fetch the stored caches,
 * re-apply positions, concatenate, no patching) and the positions section
 * (each document keeps its original length in positions: document t starts
 * at pos_base + sum of the earlier documents' lengths; its slot j sits at
 * that offset + c2kv_slot_position(n_t, k, j)).
 *   segs          host [num_segs], grouped per request in composition order
 *   req_seg_ptr   host [num_reqs+1], CSR: request r owns segs[ptr[r]..ptr[r+1])
 *   pos_base      host [num_reqs] or NULL (all 0)
 *   cache_k/v     device [num_reqs][hkv][cap][head_dim]: row i of request r
 *                 receives composed slot i; K rotated (fp32, rounded once to
 *                 dt), V copied bit for bit.  Rows >= cache_len are untouched.
 *   pos_out       device [num_reqs][cap] int32 or NULL: composed positions
 *   cache_len_out host [num_reqs]: number of composed rows per request
 *   next_pos_out  host [num_reqs] or NULL: pos_base + sum of the request's
 *                 document lengths (where the question starts)
 * Asynchronous on `stream`: the segments' memory (device or host) must stay
 * allocated and unwritten until `stream` has passed the call, and for as
 * long as a graph that captured the call may be replayed.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, CAPACITY (a request needs more
 * than cap rows, or a position exceeds 2^24), HIP. */
c2kv_status c2kv_compose(const c2kv_segment* segs, int32_t num_segs,
                         const int32_t* req_seg_ptr, int32_t num_reqs,
                         const int32_t* pos_base,
                         int32_t ratio_k, int32_t hkv, int32_t head_dim, float rope_theta,
                         void* cache_k, void* cache_v, int64_t cap,
                         int32_t* pos_out, int32_t* cache_len_out, int32_t* next_pos_out,
                         c2kv_dtype dt, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- host-resident slot caches ------------------------------------------ */

/* Device address of page-locked host memory, so that c2kv_compose can read
 * stored slot caches where they live.  [Explainer] problem section (Fig. 1):
 * stored caches sit in host memory and are moved to the GPU when a request
 * uses them, and that move, not recomputation, dominates time to first
 * token.  A c2kv_segment whose k/v are addresses returned here makes compose
 * fetch only the compressed slot rows across the host link and rotate them
 * on arrival; no staging copy in device memory is made.  Such segments
 * should carry flags = C2KV_SEGMENT_HOST (correct either way; the flag
 * selects the launch shape that reads host memory fastest).
 *   host_ptr  host address inside one allocation made page-locked by
 *             hipHostMalloc / hipHostAlloc (a pinned PyTorch CPU tensor is one)
 *   bytes     number of bytes from host_ptr the device may read, >= 1
 *   dev_ptr   out: the address kernels use for host_ptr; valid while the
 *             allocation lives.  Host reads and writes stay valid; writes the
 *             host makes while a kernel reads the memory are a race.
 * Both host_ptr and host_ptr + bytes - 1 must be page-locked host memory
 * mapped for the current device, at the same offset from each other on the
 * device side; pageable memory is rejected, never touched by a kernel.
 * Synchronous, no device work.  Clears any HIP error state its own queries
 * raise.
 * Errors: INVALID_ARG (NULL, bytes == 0, not mapped page-locked memory). */
c2kv_status c2kv_host_device_ptr(const void* host_ptr, size_t bytes, const void** dev_ptr);

/* Compose from stored slot caches in page-locked host memory by copying
 * them to the device first.  Same source as c2kv_host_device_ptr ([Explainer]
 * problem section, Fig. 1: the caches move from host memory to the GPU when
 * a request uses them).  Each segment's m slot rows of K and V are copied
 * (async DMA on `stream`) into the workspace, packed [m][hkv][head_dim],
 * and c2kv_compose then runs on the staged copies.  Only compressed rows
 * cross the host link.  Where HIP executes host-to-device copies as kernels
 * (blit kernels, as on MI355X systems), composing the host segments in
 * place with C2KV_SEGMENT_HOST is the faster load; this entry point is for
 * callers that want the rows staged in device memory.
 *   segs        host [num_segs]: k/v are HOST addresses in page-locked
 *               memory (every byte of [k, k + ((m-1)*row_stride +
 *               hkv*head_dim) elements) is checked before the first copy)
 *   workspace   device, >= c2kv_workspace_size_compose_staged(...) bytes;
 *               holds the staged rows until the compose kernel has read them
 *   all other arguments and outputs exactly as c2kv_compose.
 * The host memory must stay allocated and unwritten until `stream` has
 * passed the call.
 * Errors: as c2kv_compose, plus INVALID_ARG for memory that is not
 * page-locked and WORKSPACE.  The size query returns 0 for invalid input. */
size_t c2kv_workspace_size_compose_staged(const c2kv_segment* segs, int32_t num_segs, int32_t ratio_k,
                                          int32_t hkv, int32_t head_dim, c2kv_dtype dt);
c2kv_status c2kv_compose_staged(const c2kv_segment* segs, int32_t num_segs,
                                const int32_t* req_seg_ptr, int32_t num_reqs,
                                const int32_t* pos_base,
                                int32_t ratio_k, int32_t hkv, int32_t head_dim, float rope_theta,
                                void* cache_k, void* cache_v, int64_t cap,
                                int32_t* pos_out, int32_t* cache_len_out, int32_t* next_pos_out,
                                c2kv_dtype dt, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- attention over the composed cache ----------------------------------- */

size_t c2kv_workspace_size_prefill(const int32_t* cache_len, int32_t num_reqs, int32_t tq,
                                   int32_t hq, int32_t hkv, int32_t head_dim, c2kv_dtype dt);

/* Question prefill over composed caches.  [Explainer] "overall flow" section:
 * after concatenation the question is appended and generation starts, with
 * nothing in the reused cache patched; positions section for where the
 * question starts.
 *   q             device [num_reqs][tq][hq][head_dim]  pre-RoPE
 *   k_new, v_new  device [num_reqs][tq][hkv][head_dim] pre-RoPE
 *   cache_k/v     device [num_reqs][hkv][cap][head_dim]
 *   cache_len     host [num_reqs]: rows already in each cache
 *   q_pos0        host [num_reqs]: position of the first question token
 *   o             device [num_reqs][tq][hq][head_dim]
 *   lse           device [num_reqs][hq][tq] float or NULL
 * Token t of request r is rotated at q_pos0[r] + t; its key (rounded to dt)
 * and value are written to row cache_len[r] + t.  Token t attends to every
 * row < cache_len[r] and to question rows <= t.  GQA as for extraction.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, CAPACITY (cache_len + tq > cap,
 * or (cap + 256) rows of one KV head reach 2 GiB), HIP. */
c2kv_status c2kv_attn_prefill(const void* q, const void* k_new, const void* v_new,
                              void* cache_k, void* cache_v, int64_t cap,
                              const int32_t* cache_len, const int32_t* q_pos0,
                              int32_t num_reqs, int32_t tq, int32_t hq, int32_t hkv,
                              int32_t head_dim, float rope_theta,
                              void* o, float* lse, c2kv_dtype dt,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

size_t c2kv_workspace_size_decode(const int32_t* cache_len, int32_t num_reqs,
                                  int32_t hq, int32_t hkv, int32_t head_dim, c2kv_dtype dt);

/* One decode step over composed caches ([Explainer] experimental-results
 * section: every generated token reads the whole compressed cache).  Same
 * contract as c2kv_attn_prefill with tq = 1:
 *   q [num_reqs][hq][head_dim], k_new/v_new [num_reqs][hkv][head_dim],
 *   o [num_reqs][hq][head_dim], lse [num_reqs][hq] or NULL,
 *   cache_len[r] rows before the append; the new token goes to that row and
 *   is rotated at q_pos[r].
 * The sequence is split into chunks processed in parallel and merged by
 * log-sum-exp; the result does not depend on the number of chunks beyond
 * fp32 rounding. */
c2kv_status c2kv_attn_decode(const void* q, const void* k_new, const void* v_new,
                             void* cache_k, void* cache_v, int64_t cap,
                             const int32_t* cache_len, const int32_t* q_pos,
                             int32_t num_reqs, int32_t hq, int32_t hkv,
                             int32_t head_dim, float rope_theta,
                             void* o, float* lse, c2kv_dtype dt,
                             void* workspace, size_t ws_bytes, hipStream_t stream);

/* One decode step exactly as c2kv_attn_decode, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid allocation): the split-K partials live in a static
 * device array of C2KV_NOALLOC_SCRATCH_BYTES bytes per GPU, held until the
 * process ends, instead of a caller workspace.  Arguments, layouts, results
 * and errors as c2kv_attn_decode without workspace / ws_bytes.  The array's
 * address is looked up once per device, on the first call there.  Every call
 * on one GPU shares that GPU's array, which keeps the last call's partials:
 * calls that overlap in time on one GPU (on different streams, or from
 * several threads without ordering) race, and the caller must order them.
 * Nothing in the array needs clearing between calls.  Allocates nothing.
 * Errors: as c2kv_attn_decode, plus WORKSPACE when the step's split
 * partials (c2kv_workspace_size_decode) exceed the array. */
#define C2KV_NOALLOC_SCRATCH_BYTES (8u << 20)
c2kv_status c2kv_attn_decode_noalloc(const void* q, const void* k_new, const void* v_new,
                                     void* cache_k, void* cache_v, int64_t cap,
                                     const int32_t* cache_len, const int32_t* q_pos,
                                     int32_t num_reqs, int32_t hq, int32_t hkv,
                                     int32_t head_dim, float rope_theta,
                                     void* o, float* lse, c2kv_dtype dt, hipStream_t stream);

/* Zero `ws_bytes` (a multiple of 4) bytes of device memory with a fill
 * kernel on `stream` (no hipMemset, so it may be captured in a graph).  No
 * entry point requires a zeroed workspace; this is a convenience. */
c2kv_status c2kv_workspace_init(void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- test support ------------------------------------------------------- */

/* Count visible cells of the extraction mask ON THE GPU with the same tile
 * enumeration and visibility predicate the extraction kernel uses, for
 * doc_lens[num_docs] at ratio k and sink length.  counts_out (host) receives
 * [0] doc->doc, [1] slot->doc, [2] slot->slot visible cells, [3] tiles that
 * were enumerated for a wave but hold no visible cell for it (0 when the
 * enumeration is tight), [4] tiles enumerated in total.  Counts are summed
 * over documents (one query head).  Synchronises `stream`.
 * [Explainer] mask figure: 4 + 8 + 8 = 20 slot->doc cells for a 12-token
 * document at k = 4. */
size_t c2kv_workspace_size_mask_cells(void);
c2kv_status c2kv_mask_cells(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k,
                            int32_t sink_len, uint64_t* counts_out,
                            void* workspace, size_t ws_bytes, hipStream_t stream);
/* The same count for c2kv_extract_attn_ex's flags.  [2] counts every
 * visible cell whose key is a slot: slot->slot, plus document->slot under
 * C2KV_EXTRACT_ANCHOR. */
c2kv_status c2kv_mask_cells_ex(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k,
                               int32_t sink_len, uint32_t flags, uint64_t* counts_out,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/* Tile schedule of c2kv_extract_attn_ex, dumped for coverage tests.  The
 * extraction kernel gives each wave a unit of C2KV_EXTRACT_UNIT_ROWS query
 * rows of one query head (document rows or slot rows of one document) and
 * walks key tiles of C2KV_EXTRACT_TILE_KEYS keys; tiles in which no cell is
 * visible under the mask are never enumerated, and the visibility predicate
 * is applied only on tiles the entry marks `masked`.  [Explainer]
 * "structured information flow" section, its mask figure and three rules
 * (document rows causal and blind to slots; slot j sees the sink block and
 * its own block; slots causal among themselves).  One entry per (unit, key
 * tile) pair the kernel computes, exactly as the attention launch with the
 * same arguments enumerates them. */
#define C2KV_EXTRACT_TILE_KEYS 64
#define C2KV_EXTRACT_UNIT_ROWS 32
typedef struct c2kv_tile_entry {
  int32_t doc;       /* document index into doc_lens */
  int32_t kv_head;   /* KV head of the key tile */
  int32_t q_head;    /* query head of the unit */
  int32_t q_slot;    /* 1: the unit's query rows are slots, 0: document tokens */
  int32_t q0, q1;    /* query rows [q0, q1) of the unit, counted within its region */
  int32_t k_slot;    /* 1: the tile's keys are slots, 0: document tokens */
  int32_t key0;      /* first key of the tile, counted within its region */
  int32_t nkeys;     /* keys of the tile inside the region (<= C2KV_EXTRACT_TILE_KEYS) */
  int32_t masked;    /* 1: some cell of the tile is hidden from some row of the unit
                        (the kernel applies the predicate); 0: every cell is visible */
} c2kv_tile_entry;

size_t c2kv_workspace_size_tile_schedule(void);
/* Enumerate the tile schedule for doc_lens[num_docs] at ratio k, sink
 * length, hq query heads over hkv KV heads and extraction flags (0 or
 * C2KV_EXTRACT_ANCHOR).
 *   entries    device [capacity] c2kv_tile_entry, or NULL with capacity 0
 *              to count only; entry order is unspecified
 *   count_out  host: number of entries of the schedule
 * Synchronises `stream`.  Errors: INVALID_ARG, UNSUPPORTED (hq/hkv > 16),
 * WORKSPACE, CAPACITY (count_out > capacity: the first `capacity` entries
 * written are an arbitrary subset), HIP. */
c2kv_status c2kv_tile_schedule(const int32_t* doc_lens, int32_t num_docs, int32_t ratio_k, int32_t sink_len,
                               int32_t hq, int32_t hkv, uint32_t flags, c2kv_tile_entry* entries,
                               int64_t capacity, int64_t* count_out, void* workspace, size_t ws_bytes,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* C2KV_H_ */
