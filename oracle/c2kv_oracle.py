"""C2KV CPU oracle.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
module imports nothing from the product.

It is a plain, slow, obviously-correct numpy implementation of what the C2KV
hot path computes: explicit dense boolean masks, RoPE in fp32 with every
product and sum rounded separately, attention accumulated in fp64.

Sources (cited by page title and section throughout):

* [Explainer] "C2KV: Compressed and Composable KV Cache Reuse for Efficient
  LLM Inference", paper-daily.com explainer.  Sections used:
  - "C2 token" section (memory slots: one slot per k document tokens,
    appended after the document; only slot K/V are kept),
  - "structured information flow" section, with its interactive mask figure
    and the three mask rules listed under it,
  - "how positions are handled at concatenation" section,
  - "overall flow: extraction, storage, concatenation" section,
  - "experimental results" section (decode reads 3/4 less at k=4).
* [Abstract] arXiv 2607.17715 abstract page (arxivdaily.com): sidecar
  extractor, compression tokens, structured attention flow.
* [KV-size] "LLM inference optimisation: KV cache compression schemes"
  (feinterview.poetries.top), the Llama 3 paragraph defining grouped-query
  attention and its 128 KB-per-token cache.

Readings taken where the pages are silent (each listed again in the design doc):

R1  slot count m = ceil(n / k); the last slot's block may be partial.
R2  a partial block's slot sits at n - 1 (the last token of its block).
R3  the sink is the first min(sink_len, n) tokens, sink_len = k by default.
R4  packed layout per document: [n document rows | m slot rows].
R5  RoPE with half-split pairing (i, i + d/2), inv_freq_i = theta^(-2i/d),
    no frequency scaling.
R6  RoPE numerics: inv_freq computed in fp64 and rounded once to fp32;
    angle = fp32(fp32(p) * inv_freq); cos/sin = fp32(cos/sin(fp64(angle)));
    each rotation product and the sum rounded to fp32, no fused multiply-add.
R7  V is never rotated.
R8  the first composed document starts at position base 0 unless given.
R9  question and generated tokens continue at pos_base + sum of the
    composed documents' original lengths.
R10 question/decode tokens see every composed slot, and each other causally.
R11 GQA: query head h reads KV head floor(h / (Hq / Hkv)).
R12 softmax scale 1/sqrt(d), no capping; no row is ever fully masked.
R13 an appended key is stored in the cache dtype; attention reads the
    stored (rounded) value.  Rotated queries stay fp32 in the oracle.
R24 the anchor-token ablation: anchors (the slot rows) and document tokens
    see each other both ways; documents stay causal among themselves and
    anchors see every anchor; positions as for C2 slots.
R23 the ablation without positional realignment gives every composed
    document the offset pos_base (its extraction positions), instead of the
    cumulative original length of the documents before it.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Set, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Slot arithmetic
# ---------------------------------------------------------------------------


def num_slots(n: int, k: int) -> int:
    """Number of C2 slots for an n-token document at ratio k.

    [Explainer] "C2 token" section: one slot is appended per k document
    tokens (a 4000-token document keeps 1000 slots at k = 4).  Reading R1:
    a trailing partial block also gets a slot, so m = ceil(n / k).
    """
    if n < 0 or k < 1:
        raise ValueError("n >= 0 and k >= 1 required")
    return (n + k - 1) // k


def slot_position(n: int, k: int, j: int) -> int:
    """Extraction-time RoPE position of slot j.

    [Explainer] positions section: slot j takes the position of the last
    token of the block it summarises (3, 7, ... at k = 4, counting from 0).
    Reading R2: a partial last block ends at token n - 1.
    """
    return min(j * k + k - 1, n - 1)


def extraction_positions(n: int, k: int) -> np.ndarray:
    """Positions of the packed rows [doc 0..n-1 | slot 0..m-1] (reading R4)."""
    m = num_slots(n, k)
    doc = list(range(n))
    slots = [slot_position(n, k, j) for j in range(m)]
    return np.array(doc + slots, dtype=np.int64)


# ---------------------------------------------------------------------------
# Structured-flow mask
# ---------------------------------------------------------------------------


def structured_mask(n: int, k: int, sink_len: Optional[int] = None, anchor: bool = False) -> np.ndarray:
    """Dense T x T visibility matrix, rows = queries, columns = keys.

    [Explainer] structured-information-flow section and its mask figure:
      rule 1  document tokens attend causally to document tokens and never
              to a slot (so document outputs equal the frozen model's);
      rule 2  slot j attends to the sink block B(0) -- the first k document
              tokens -- plus its own k-token block; slot 0's own block is
              the sink itself;
      rule 3  slots attend causally to slots, themselves included.
    Reading R3 for the sink size.

    anchor=True is the experimental-results section's anchor-token ablation
    (reading R24): the extra tokens and the document tokens see each other
    both ways.  Document rows keep their causal mask over documents and see
    every anchor; anchor rows see every document token and every anchor.
    """
    if sink_len is None:
        sink_len = k
    m = num_slots(n, k)
    T = n + m
    s = min(sink_len, n)
    M = np.zeros((T, T), dtype=bool)
    r = np.arange(n)
    # rule 1: doc -> doc causal, doc -> slot never
    M[:n, :n] = r[None, :] <= r[:, None]
    # rule 2: slot -> doc: sink block plus own block
    c = np.arange(n)
    for j in range(m):
        M[n + j, :n] = (c < s) | (c // k == j)
    # rule 3: slot -> slot causal, including itself
    jj = np.arange(m)
    M[n:, n:] = jj[None, :] <= jj[:, None]
    if anchor:
        M[:n, n:] = True
        M[n:, :] = True
    return M


def visible_set(n: int, k: int, sink_len: Optional[int], row: int, anchor: bool = False) -> Set[int]:
    """Visible key indices of one packed row, built directly from the rule
    statements (not from the matrix) for brute-force checks.  anchor=True:
    the anchor-token ablation (see structured_mask)."""
    if sink_len is None:
        sink_len = k
    m = num_slots(n, k)
    s = min(sink_len, n)
    if anchor:
        anchors = set(range(n, n + m))
        return (set(range(row + 1)) | anchors) if row < n else (set(range(n)) | anchors)
    if row < n:
        return set(range(row + 1))
    j = row - n
    assert 0 <= j < m
    sink = set(range(s))
    own = set(range(j * k, min(n, j * k + k)))
    earlier_slots = {n + jj for jj in range(j + 1)}
    return sink | own | earlier_slots


def mask_cell_counts(n: int, k: int, sink_len: Optional[int] = None) -> Tuple[int, int, int]:
    """(doc->doc, slot->doc, slot->slot) visible cell counts of one document,
    counted on the dense matrix."""
    M = structured_mask(n, k, sink_len)
    return (int(M[:n, :n].sum()), int(M[n:, :n].sum()), int(M[n:, n:].sum()))


# ---------------------------------------------------------------------------
# Storage rounding
# ---------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); the result is
    returned as fp32 values that are exactly representable in bf16.  Inputs
    are finite (no NaN handling needed on this path)."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def storage_round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# RoPE (fp32, reading R5/R6)
# ---------------------------------------------------------------------------


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """inv_freq_i = theta^(-2i/d) for i < d/2, computed in fp64 and rounded
    once to fp32.  The pages only name RoPE ([Explainer] positions section);
    the standard frequency ladder is reading R5."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d).astype(np.float32)


def rope_cos_sin(pos: np.ndarray, d: int, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos/sin tables [len(pos)][d/2] in fp32 (reading R6)."""
    inv = rope_inv_freq(d, theta)
    p32 = np.asarray(pos, dtype=np.int64).astype(np.float32)
    ang = (p32[:, None] * inv[None, :]).astype(np.float32)   # one fp32 multiply
    a64 = ang.astype(np.float64)
    return np.cos(a64).astype(np.float32), np.sin(a64).astype(np.float32)


def rope_rotate(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate x[T][H][d] (fp32 values) at positions pos[T].

    Half-split pairing (x_i, x_{i+d/2}):
        x'_i       = x_i c - x_{i+d/2} s
        x'_{i+d/2} = x_{i+d/2} c + x_i s
    every product and the sum rounded to fp32 separately (reading R6).
    """
    x = np.asarray(x, dtype=np.float32)
    T, H, d = x.shape
    h = d // 2
    c, s = rope_cos_sin(pos, d, theta)
    c = c[:, None, :]
    s = s[:, None, :]
    lo = x[..., :h]
    hi = x[..., h:]
    # numpy float32 arithmetic rounds every operation to fp32 and never fuses
    out_lo = (lo * c).astype(np.float32) - (hi * s).astype(np.float32)
    out_hi = (hi * c).astype(np.float32) + (lo * s).astype(np.float32)
    return np.concatenate([out_lo.astype(np.float32), out_hi.astype(np.float32)], axis=-1)


# ---------------------------------------------------------------------------
# Attention (fp64, explicit mask, GQA)
# ---------------------------------------------------------------------------


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
              row_chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """Masked softmax attention with grouped-query heads.

    q [T][Hq][d], k/v [S][Hkv][d] (any float dtype, used in fp64),
    mask [T][S] bool (True = visible).  Returns o [T][Hq][d] and the natural
    log-sum-exp of the scaled scores lse [Hq][T], both fp64.

    Standard attention ([Explainer] "C2 token" section: projected slot and
    document tokens enter one ordinary attention); scale 1/sqrt(d) and no
    capping (reading R12); query head h uses KV head h // (Hq/Hkv)
    ([KV-size] Llama 3 paragraph for GQA; reading R11 for the mapping).
    """
    T, Hq, d = q.shape
    S, Hkv, _ = k.shape
    assert Hq % Hkv == 0 and mask.shape == (T, S)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    o = np.zeros((T, Hq, d), dtype=np.float64)
    lse = np.zeros((Hq, T), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        kh = np.asarray(k[:, g, :], dtype=np.float64)
        vh = np.asarray(v[:, g, :], dtype=np.float64)
        for r0 in range(0, T, row_chunk):
            r1 = min(T, r0 + row_chunk)
            qh = np.asarray(q[r0:r1, h, :], dtype=np.float64)
            sc = (qh @ kh.T) * scale
            mk = mask[r0:r1]
            sc = np.where(mk, sc, -np.inf)
            mx = sc.max(axis=1, keepdims=True)
            p = np.exp(sc - mx)
            den = p.sum(axis=1, keepdims=True)
            o[r0:r1, h, :] = (p @ vh) / den
            lse[h, r0:r1] = (mx + np.log(den))[:, 0]
    return o, lse


def attention_brute(q, k, v, visible: Sequence[Set[int]]) -> Tuple[np.ndarray, np.ndarray]:
    """Scalar-loop attention over explicit visibility sets (tiny inputs only):
    for every query row and head, sum exp over the visible keys with
    ``math.exp`` in Python floats."""
    T, Hq, d = q.shape
    S, Hkv, _ = k.shape
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    o = np.zeros((T, Hq, d), dtype=np.float64)
    lse = np.zeros((Hq, T), dtype=np.float64)
    for r in range(T):
        keys = sorted(visible[r])
        for h in range(Hq):
            g = h // G
            scores = []
            for c in keys:
                acc = 0.0
                for e in range(d):
                    acc += float(q[r, h, e]) * float(k[c, g, e])
                scores.append(acc * scale)
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            den = sum(ws)
            for e in range(d):
                o[r, h, e] = sum(w * float(v[c, g, e]) for w, c in zip(ws, keys)) / den
            lse[h, r] = mx + math.log(den)
    return o, lse


# ---------------------------------------------------------------------------
# Hot-path steps
# ---------------------------------------------------------------------------


def doc_row_offsets(doc_lens: Sequence[int], k: int) -> List[int]:
    """Start row of each document in the packed [doc | slots] layout."""
    offs, acc = [], 0
    for n in doc_lens:
        offs.append(acc)
        acc += n + num_slots(n, k)
    offs.append(acc)
    return offs


def extract_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, doc_lens: Sequence[int],
                 ratio_k: int, sink_len: Optional[int], theta: float,
                 docs: Optional[Sequence[int]] = None,
                 anchor: bool = False) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
    """Extraction attention of each document, run alone (offline extraction
    in the [Explainer] overall-flow section; each document is processed by
    itself).

    q [sumT][Hq][d], k/v [sumT][Hkv][d] hold pre-RoPE values packed per
    document as [n doc rows | m slot rows].  Q and K are rotated at the
    extraction positions (doc token i at i, slot j at its block's last
    token), V is not (reading R7); then masked attention under the
    structured mask (the anchor-token ablation's mask with anchor=True).
    Returns {doc: (o [T][Hq][d], lse [Hq][T])}.
    """
    offs = doc_row_offsets(doc_lens, ratio_k)
    out = {}
    for b in (range(len(doc_lens)) if docs is None else docs):
        n = doc_lens[b]
        r0, r1 = offs[b], offs[b + 1]
        pos = extraction_positions(n, ratio_k)
        qr = rope_rotate(np.asarray(q[r0:r1], dtype=np.float32), pos, theta)
        kr = rope_rotate(np.asarray(k[r0:r1], dtype=np.float32), pos, theta)
        M = structured_mask(n, ratio_k, sink_len, anchor)
        out[b] = attention(qr, kr, np.asarray(v[r0:r1], dtype=np.float64), M)
    return out


def compose_positions(doc_lens_in_order: Sequence[int], ratio_k: int,
                      pos_base: int = 0, realign: bool = True) -> Tuple[np.ndarray, List[int], int]:
    """Realigned slot positions of a composition.

    [Explainer] positions section: each compressed document occupies as
    many positions as its original length; later documents are shifted by
    the cumulative original length of the earlier ones (a 400-token document
    gives slots 3, 7, ..., 399 and the next document's first slot is 403).
    With realign=False (the experimental-results section's ablation without
    positional realignment, reading R23) every document keeps its
    extraction positions: its offset is pos_base, not shifted by the
    earlier documents.  Returns (positions of every composed row,
    per-document offsets, the position just after the last document; the
    latter is pos_base + the sum of the lengths either way).
    """
    pos, offsets = [], []
    off = pos_base
    for n in doc_lens_in_order:
        doc_off = off if realign else pos_base
        offsets.append(doc_off)
        pos.extend(doc_off + slot_position(n, ratio_k, j) for j in range(num_slots(n, ratio_k)))
        off += n
    return np.array(pos, dtype=np.int64), offsets, off


def compose(slot_k: Sequence[np.ndarray], slot_v: Sequence[np.ndarray],
            doc_lens_in_order: Sequence[int], ratio_k: int, theta: float,
            dtype: str, pos_base: int = 0, realign: bool = True):
    """Compose pre-RoPE slot caches into one contiguous cache.

    [Explainer] overall-flow and positions sections: the stored slot K/V
    are pre-RoPE; at composition each document's slots are rotated at their
    realigned positions and the caches are concatenated in request order with
    no recomputation.  K rows are rotated in fp32 and rounded to the storage
    dtype; V rows are copied unchanged (reading R7).

    slot_k[t], slot_v[t]: [m_t][Hkv][d].  realign=False composes without
    positional realignment (see compose_positions).  Returns (cache_k
    [M][Hkv][d] fp32 values, cache_v, positions [M] int64, next position).
    """
    pos, _, nxt = compose_positions(doc_lens_in_order, ratio_k, pos_base, realign)
    ks = np.concatenate([np.asarray(x, dtype=np.float32) for x in slot_k], axis=0)
    vs = np.concatenate([np.asarray(x, dtype=np.float32) for x in slot_v], axis=0)
    assert ks.shape[0] == pos.shape[0]
    ck = storage_round(rope_rotate(ks, pos, theta), dtype)
    return ck, vs.copy(), pos, nxt


def append_and_attend(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                      cache_k: np.ndarray, cache_v: np.ndarray, q_pos0: int,
                      theta: float, dtype: str):
    """Question prefill (or one decode step when Tq = 1) over a composed cache.

    [Explainer] overall-flow section: after concatenation the question is
    appended and generation starts; nothing in the reused cache is patched.
    Question token t sits at position q_pos0 + t (reading R9); its key is
    rotated, stored in the cache dtype and appended (reading R13); each
    question token sees every cache row and the question tokens up to and
    including itself (reading R10).

    q [Tq][Hq][d], k_new/v_new [Tq][Hkv][d] pre-RoPE; cache_k/v [M][Hkv][d].
    Returns (o [Tq][Hq][d], lse [Hq][Tq], new cache_k, new cache_v).
    """
    Tq = q.shape[0]
    M = cache_k.shape[0]
    pos = q_pos0 + np.arange(Tq, dtype=np.int64)
    qr = rope_rotate(np.asarray(q, dtype=np.float32), pos, theta)
    kr = storage_round(rope_rotate(np.asarray(k_new, dtype=np.float32), pos, theta), dtype)
    ck = np.concatenate([np.asarray(cache_k, dtype=np.float32), kr], axis=0)
    cv = np.concatenate([np.asarray(cache_v, dtype=np.float32),
                         np.asarray(v_new, dtype=np.float32)], axis=0)
    mask = np.zeros((Tq, M + Tq), dtype=bool)
    mask[:, :M] = True
    t = np.arange(Tq)
    mask[:, M:] = t[None, :] <= t[:, None]
    o, lse = attention(qr, ck, cv, mask)
    return o, lse, ck, cv


def decode_step(q, k_new, v_new, cache_k, cache_v, q_pos: int, theta: float, dtype: str):
    """One decode step: q [Hq][d], k_new/v_new [Hkv][d].  [Explainer] results
    section: each generated token reads the whole (compressed) cache."""
    o, lse, ck, cv = append_and_attend(q[None], k_new[None], v_new[None],
                                       cache_k, cache_v, q_pos, theta, dtype)
    return o[0], lse[:, 0], ck, cv


# ---------------------------------------------------------------------------
# Byte accounting
# ---------------------------------------------------------------------------


def kv_bytes_per_token(layers: int, hkv: int, d: int, elem_bytes: int) -> int:
    """K and V bytes cached per token ([KV-size] Llama 3 paragraph)."""
    return layers * hkv * d * 2 * elem_bytes


def decode_kv_bytes(rows: int, hkv: int, d: int, elem_bytes: int) -> int:
    """K and V bytes one decode step must read for one layer and request."""
    return rows * hkv * d * 2 * elem_bytes


# ---------------------------------------------------------------------------
# The extractor layer around the structured attention
# ---------------------------------------------------------------------------
#
# Readings (listed again in the design doc):
# R19 the frozen base layer is the pre-norm decoder layer of the base models
#     the pages evaluate (Llama3.1-8B, Qwen2.5, Qwen3): RMSNorm with a learned
#     gain, attention, output projection and residual add, RMSNorm, SwiGLU
#     FFN (silu(gate) * up, then down) and residual add.
# R20 the C2 projections replace only Q/K/V for slot rows; the attention
#     norm's gain, the output projection and the FFN are the frozen ones for
#     every row ([Explainer] "C2 token" section).
# R21 at the first layer every slot row's input is the one shared learnable
#     vector ([Explainer] "C2 token" section).


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x [T][D] -> x / sqrt(mean(x^2) + eps) * gamma, in fp64 (reading R19)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(gamma, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def slot_row_mask(doc_lens: Sequence[int], k: int) -> np.ndarray:
    """Boolean [sumT]: True on the slot rows of the packed layout (R4)."""
    out = []
    for n in doc_lens:
        out += [False] * n + [True] * num_slots(n, k)
    return np.array(out, dtype=bool)


def extractor_layer(x: np.ndarray, w: Dict[str, np.ndarray], doc_lens: Sequence[int], ratio_k: int,
                    sink_len: Optional[int], hq: int, hkv: int, d: int, theta: float, eps: float,
                    slot_embed: Optional[np.ndarray] = None
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One layer of the frozen model with the C2 extractor attached, over a
    batch of documents that are extracted independently.

    [Explainer] "C2 token" section: document tokens keep the frozen Q/K/V
    projections and slot tokens use their own per-layer C2 Q/K/V
    projections; both then enter one standard attention (the structured mask
    of the structured-flow section, with RoPE at the extraction positions);
    the output projection, the FFN and everything else stay the frozen
    model's.  Readings R19-R21.

    x [sumT][Dm] packed per document as [n doc rows | m slot rows].
    w: attn_norm [Dm], wqkv [(hq+2hkv)d][Dm] (frozen; rows: q heads, k
    heads, v heads), wqkv_c2 (same shape, C2), wo [Dm][hq d], ffn_norm [Dm],
    w_gate [F][Dm], w_up [F][Dm], w_down [Dm][F].
    slot_embed [Dm] or None: when given, every slot row's input is set to
    it first (the first layer, R21).
    Returns x_out [sumT][Dm] (fp64) and this layer's stored C2KV: the slot
    rows' pre-RoPE keys and values [sum m][hkv][d] (fp64).
    """
    x = np.array(x, dtype=np.float64)
    slot = slot_row_mask(doc_lens, ratio_k)
    assert x.shape[0] == slot.shape[0]
    if slot_embed is not None:
        x[slot] = np.asarray(slot_embed, dtype=np.float64)
    T = x.shape[0]
    h = rms_norm(x, w["attn_norm"], eps)
    qkv = np.empty((T, (hq + 2 * hkv) * d), dtype=np.float64)
    qkv[~slot] = h[~slot] @ np.asarray(w["wqkv"], dtype=np.float64).T
    qkv[slot] = h[slot] @ np.asarray(w["wqkv_c2"], dtype=np.float64).T
    q = qkv[:, : hq * d].reshape(T, hq, d)
    k = qkv[:, hq * d: (hq + hkv) * d].reshape(T, hkv, d)
    v = qkv[:, (hq + hkv) * d:].reshape(T, hkv, d)
    att = extract_attn(q, k, v, doc_lens, ratio_k, sink_len, theta)
    o = np.concatenate([att[b][0] for b in range(len(doc_lens))]).reshape(T, hq * d)
    x = x + o @ np.asarray(w["wo"], dtype=np.float64).T
    h2 = rms_norm(x, w["ffn_norm"], eps)
    act = silu(h2 @ np.asarray(w["w_gate"], dtype=np.float64).T) * (h2 @ np.asarray(w["w_up"], dtype=np.float64).T)
    x = x + act @ np.asarray(w["w_down"], dtype=np.float64).T
    return x, k[slot], v[slot]
