"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, on sampled outputs the oracle computes one by one.

* Llama3.1-8B layer: all 8 documents of 4096 tokens extracted in one call
  (sampled document and slot rows of the first and last document, every
  head), the full 8192-slot compose in the seeded order (every row), the
  64-token question prefill and 256 decode steps replayed from a HIP graph
  (steps 0, 127 and 255 checked, plus every appended cache row).
* Qwen2.5-7B pool: 32 requests composed in one call from a 64-document pool
  (k = 16, ragged lengths), then 3 decode steps of all 32 requests; 4
  requests checked in full.
* Long-context decode: 64 requests at 16k/32k/64k/128k original tokens
  (4096..32768 slots), two layer caches, two steps; 2 requests x 2 layers
  x 2 steps checked per length.
* Qwen3-14B extraction: 64 documents of 8192 tokens in one call at
  k = 4, 8, 16; sampled rows of the first and last document, every head;
  plus the GPU mask-cell counts of the whole batch.
* The anchor-token ablation over the whole Llama batch (sampled rows, exact
  cell counts), and the Qwen2.5 pool composed from pinned host memory
  (bit-identical to the device-source compose).

Decode step s over a cache equals the last query row of a prefill of the
question and decode tokens 0..s (an oracle identity pinned on the CPU), so
the oracle side evaluates the checked steps with one prefill call.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import assert_close, assert_lse_close, assert_rotated_close, np32, oracle_extract_rows

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def c2kv():
    import compressed_composable_kv_amd as m
    return m


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _doc_sample_rows(n, m):
    """Packed rows to check in one document: the first rows, tile and block
    edges, the end of the document, and slot rows at the same kinds of
    places (first, block edges, last)."""
    doc = sorted({r for r in (0, 1, 2, 3, 4, 5, 31, 32, 63, 64, 65, 127, 128, 1000, n // 2, n - 2, n - 1)
                  if 0 <= r < n})
    slot = sorted({j for j in (0, 1, 2, 15, 16, 31, 32, 63, 64, m // 2, m - 2, m - 1) if 0 <= j < m})
    return doc + [n + j for j in slot]


def _check_extract_rows(og, lg, q, k, v, n, ratio_k, sink, theta, what, anchor=False):
    """og/lg: GPU output rows [rows][Hq][d] / lse [Hq][rows] of one
    document's packed rows; q/k/v: CPU inputs of the same rows."""
    rows = _doc_sample_rows(n, O.num_slots(n, ratio_k))
    ro, rl = oracle_extract_rows(q, k, v, n, ratio_k, sink, theta, rows, anchor)
    assert_close(og[rows], ro, "bf16", f"{what}: sampled rows")
    assert_lse_close(lg[:, rows], rl, "bf16", f"{what}: sampled rows")


# ------------------------------------------------------- Llama3.1-8B layer

def test_llama_layer_full(c2kv):
    w = W.LLAMA
    d, hq, hkv, k, theta, dt = w.head_dim, w.hq, w.hkv, w.ratio_k, w.rope_theta, w.dtype
    lens = list(w.doc_lens)
    rows = c2kv.packed_rows(lens, k)
    print("llama layer: generating inputs", flush=True)
    q = W.normal((rows, hq, d), dt, w.wid, W.P_Q)
    kk = W.normal((rows, hkv, d), dt, w.wid, W.P_K)
    v = W.normal((rows, hkv, d), dt, w.wid, W.P_V)
    qd, kd, vd = q.to(DEV), kk.to(DEV), v.to(DEV)

    print("llama layer: extraction of 8 x 4096 in one call", flush=True)
    o, lse = c2kv.extract_attn(qd, kd, vd, lens, k, w.sink_len, theta, return_lse=True)
    offs = O.doc_row_offsets(lens, k)
    for b in (0, len(lens) - 1):
        r0, r1 = offs[b], offs[b + 1]
        _check_extract_rows(np32(o[r0:r1]), np32(lse[:, r0:r1]), q[r0:r1].float().numpy(),
                            kk[r0:r1].float().numpy(), v[r0:r1].float().numpy(), lens[b], k, w.sink_len,
                            theta, f"document {b}")
    del o, lse, qd

    print("llama layer: compose 8192 slots in the seeded order", flush=True)
    order = W.llama_doc_order(w)
    views = c2kv.slot_views(kd, vd, lens, k)
    M = sum(O.num_slots(n, k) for n in lens)
    tq, S = w.tq, w.decode_steps
    cap = M + tq + S
    ck = torch.zeros((1, hkv, cap, d), dtype=dt, device=DEV)
    cv = torch.zeros_like(ck)
    pos = torch.full((1, cap), -1, dtype=torch.int32, device=DEV)
    clen, nxt = c2kv.compose([[views[t] for t in order]], k, theta, ck, cv, pos_out=pos)
    hviews = c2kv.slot_views(kk, v, lens, k)
    rk, rv, rpos, P = O.compose([hviews[t][0].float().numpy() for t in order],
                                [hviews[t][1].float().numpy() for t in order],
                                [lens[t] for t in order], k, theta, "bf16")
    assert clen == [M] and nxt == [P] and P == sum(lens)
    assert np.array_equal(pos[0, :M].cpu().numpy(), rpos)
    pre = np.concatenate([hviews[t][0].float().numpy() for t in order])
    assert_rotated_close(np32(ck[0, :, :M]).transpose(1, 0, 2), rk, pre, "bf16", "composed keys")
    assert torch.equal(cv[0, :, :M].transpose(0, 1).cpu(), torch.cat([hviews[t][1] for t in order]))

    print("llama layer: prefill 64 + 256 decode steps (graph)", flush=True)
    qp = W.normal((1, tq, hq, d), dt, w.wid, W.P_PREFILL)
    kp = W.normal((1, tq, hkv, d), dt, w.wid, W.P_NEW_KV)
    vp = W.normal((1, tq, hkv, d), dt, w.wid, W.P_NEW_KV, salt=1)
    qs = W.normal((S, 1, hq, d), dt, w.wid, W.P_DEC_Q)
    ks = W.normal((S, 1, hkv, d), dt, w.wid, W.P_NEW_KV, salt=2)
    vs = W.normal((S, 1, hkv, d), dt, w.wid, W.P_NEW_KV, salt=3)
    op, lp = c2kv.attn_prefill(qp.to(DEV), kp.to(DEV), vp.to(DEV), ck, cv, [M], [P], theta, return_lse=True)
    qsd, ksd, vsd = qs.to(DEV), ks.to(DEV), vs.to(DEV)
    ws = torch.empty(max(c2kv.workspace_size_decode([M + tq + s], hq, hkv, d, dt) for s in range(S)),
                     dtype=torch.uint8, device=DEV)
    outs = torch.empty((S, 1, hq, d), dtype=dt, device=DEV)
    lses = torch.empty((S, 1, hq), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(S):
            o_s, l_s = c2kv.attn_decode(qsd[s], ksd[s], vsd[s], ck, cv, [M + tq + s], [P + tq + s], theta,
                                        return_lse=True, workspace=ws)
            outs[s].copy_(o_s)
            lses[s].copy_(l_s)
    graph.replay()
    torch.cuda.synchronize()

    for s in (0, 127, 255):
        qa = np.concatenate([qp[0].float().numpy(), qs[:s + 1, 0].float().numpy()])
        ka = np.concatenate([kp[0].float().numpy(), ks[:s + 1, 0].float().numpy()])
        va = np.concatenate([vp[0].float().numpy(), vs[:s + 1, 0].float().numpy()])
        ro, rl, rk2, rv2 = O.append_and_attend(qa, ka, va, rk, rv, P, theta, "bf16")
        if s == 0:
            assert_close(np32(op[0]), ro[:tq], "bf16", "prefill output")
            assert_lse_close(np32(lp[0]), rl[:, :tq], "bf16", "prefill")
        assert_close(np32(outs[s, 0]), ro[-1], "bf16", f"decode step {s}")
        assert_lse_close(np32(lses[s, 0]), rl[:, -1], "bf16", f"decode step {s}")
    # every appended row (64 question + 256 decode keys and values)
    L = M + tq + S
    gk = np32(ck[0, :, M:L]).transpose(1, 0, 2)
    assert_rotated_close(gk, rk2[M:L], np.concatenate([kp[0].float().numpy(), ks[:, 0].float().numpy()]),
                         "bf16", "appended keys")
    assert torch.equal(cv[0, :, M:L].transpose(0, 1).cpu(), torch.cat([vp[0], vs[:, 0]]))
    del ck, cv, kd, vd, graph
    _free()


# --------------------------------------------------- Qwen2.5-7B pool decode

def test_qwen25_pool_full(c2kv):
    w = W.QWEN25
    d, hq, hkv, k, theta, dt = w.head_dim, w.hq, w.hkv, w.ratio_k, w.rope_theta, w.dtype
    pool_n = W.qwen25_pool(w)
    reqs = W.qwen25_requests(w)
    assert len(reqs) == 32
    print("qwen25 pool: generating the 64-document pool", flush=True)
    pool_k = [W.normal((O.num_slots(n, k), hkv, d), dt, w.wid, W.P_K, salt=t) for t, n in enumerate(pool_n)]
    pool_v = [W.normal((O.num_slots(n, k), hkv, d), dt, w.wid, W.P_V, salt=t) for t, n in enumerate(pool_n)]
    dk = [x.to(DEV) for x in pool_k]
    dv = [x.to(DEV) for x in pool_v]
    Ms = [sum(O.num_slots(pool_n[t], k) for t in r) for r in reqs]
    S = 3
    cap = max(Ms) + w.decode_steps
    R = len(reqs)
    ck = torch.zeros((R, hkv, cap, d), dtype=dt, device=DEV)
    cv = torch.zeros_like(ck)
    pos = torch.full((R, cap), -1, dtype=torch.int32, device=DEV)
    print(f"qwen25 pool: compose 32 requests (M = {min(Ms)}..{max(Ms)}) in one call", flush=True)
    clen, nxt = c2kv.compose([[(dk[t], dv[t], pool_n[t]) for t in r] for r in reqs], k, theta, ck, cv, pos_out=pos)
    assert clen == Ms
    gpos = pos.cpu().numpy()
    for r, docs in enumerate(reqs):
        rp, _, rnext = O.compose_positions([pool_n[t] for t in docs], k)
        assert nxt[r] == rnext and np.array_equal(gpos[r, :Ms[r]], rp)
    qs = W.normal((S, R, hq, d), dt, w.wid, W.P_DEC_Q)
    ks = W.normal((S, R, hkv, d), dt, w.wid, W.P_NEW_KV)
    vs = W.normal((S, R, hkv, d), dt, w.wid, W.P_NEW_KV, salt=1)
    outs, lses = [], []
    print("qwen25 pool: 3 decode steps of all 32 requests", flush=True)
    for s in range(S):
        o_s, l_s = c2kv.attn_decode(qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV), ck, cv, [m + s for m in Ms],
                                    [x + s for x in nxt], theta, return_lse=True)
        outs.append(np32(o_s))
        lses.append(np32(l_s))
    torch.cuda.synchronize()
    for r in (0, 7, 19, 31):
        docs = reqs[r]
        rk, rv, _, P = O.compose([pool_k[t].float().numpy() for t in docs], [pool_v[t].float().numpy() for t in docs],
                                 [pool_n[t] for t in docs], k, theta, "bf16")
        pre = np.concatenate([pool_k[t].float().numpy() for t in docs])
        assert_rotated_close(np32(ck[r, :, :Ms[r]]).transpose(1, 0, 2), rk, pre, "bf16", f"request {r} keys")
        assert torch.equal(cv[r, :, :Ms[r]].transpose(0, 1).cpu(), torch.cat([pool_v[t] for t in docs]))
        ro, rl, _, _ = O.append_and_attend(qs[:, r].float().numpy(), ks[:, r].float().numpy(),
                                           vs[:, r].float().numpy(), rk, rv, P, theta, "bf16")
        for s in range(S):
            assert_close(outs[s][r], ro[s], "bf16", f"request {r} step {s}")
            assert_lse_close(lses[s][r], rl[:, s], "bf16", f"request {r} step {s}")
    del ck, cv, dk, dv
    _free()


# ---------------------------------------------------- long-context decode

@pytest.mark.parametrize("ndocs", W.longctx_doc_counts(), ids=lambda n: f"{4 * n}k")
def test_longctx_decode_full(c2kv, ndocs):
    w = W.LONGCTX
    d, hq, hkv, k, theta, dt = w.head_dim, w.hq, w.hkv, w.ratio_k, w.rope_theta, w.dtype
    R, layers, S = w.num_reqs, 2, 2
    L_orig = 4096 * ndocs
    M = ndocs * O.num_slots(4096, k)
    cap = M + S
    print(f"longctx {L_orig}: {R} requests x {M} slots x {layers} layer caches", flush=True)
    caches = []
    for layer in range(layers):
        ck = W.device_normal((R, hkv, cap, d), dt, w.wid, W.P_K, DEV, salt=10 * ndocs + layer)
        cv = W.device_normal((R, hkv, cap, d), dt, w.wid, W.P_V, DEV, salt=10 * ndocs + layer)
        caches.append((ck, cv))
    checked = (0, R - 1)
    ref_in = {(layer, r): (caches[layer][0][r, :, :M].transpose(0, 1).float().cpu().numpy(),
                           caches[layer][1][r, :, :M].transpose(0, 1).float().cpu().numpy())
              for layer in range(layers) for r in checked}
    qs = W.normal((layers, S, R, hq, d), dt, w.wid, W.P_DEC_Q, salt=ndocs)
    ks = W.normal((layers, S, R, hkv, d), dt, w.wid, W.P_NEW_KV, salt=ndocs)
    vs = W.normal((layers, S, R, hkv, d), dt, w.wid, W.P_NEW_KV, salt=100 + ndocs)
    outs = {}
    for s in range(S):
        for layer in range(layers):
            ck, cv = caches[layer]
            o_s, l_s = c2kv.attn_decode(qs[layer, s].to(DEV), ks[layer, s].to(DEV), vs[layer, s].to(DEV), ck, cv,
                                        [M + s] * R, [L_orig + s] * R, theta, return_lse=True)
            outs[(layer, s)] = (np32(o_s), np32(l_s))
    torch.cuda.synchronize()
    for layer in range(layers):
        for r in checked:
            rk, rv = ref_in[(layer, r)]
            ro, rl, _, _ = O.append_and_attend(qs[layer, :, r].float().numpy(), ks[layer, :, r].float().numpy(),
                                               vs[layer, :, r].float().numpy(), rk, rv, L_orig, theta, "bf16")
            for s in range(S):
                og, lg = outs[(layer, s)]
                assert_close(og[r], ro[s], "bf16", f"{L_orig}: layer {layer} request {r} step {s}")
                assert_lse_close(lg[r], rl[:, s], "bf16", f"{L_orig}: layer {layer} request {r} step {s}")
    del caches
    _free()


# ------------------------------------- full-cache comparator (uncompressed)

@pytest.mark.parametrize("ndocs", [16, 32], ids=lambda n: f"{4 * n}k")
def test_full_cache_decode_full(c2kv, ndocs):
    """The uncompressed comparator of the long-context sweep at 64k and 128k
    rows per request: 64 requests of the Llama shapes in one launch (the
    benchmark's launch shape), two steps; the first and last request
    checked against the oracle."""
    w = W.LONGCTX
    d, hq, hkv, theta, dt = w.head_dim, w.hq, w.hkv, w.rope_theta, w.dtype
    R, S = w.num_reqs, 2
    L = 4096 * ndocs
    cap = L + S
    print(f"full cache {L}: {R} requests x {L} rows", flush=True)
    ck = W.device_normal((R, hkv, cap, d), dt, w.wid, W.P_K, DEV, salt=500 + ndocs)
    cv = W.device_normal((R, hkv, cap, d), dt, w.wid, W.P_V, DEV, salt=500 + ndocs)
    checked = (0, R - 1)
    ref_in = {r: (ck[r, :, :L].transpose(0, 1).float().cpu().numpy(), cv[r, :, :L].transpose(0, 1).float().cpu().numpy())
              for r in checked}
    qs = W.normal((S, R, hq, d), dt, w.wid, W.P_DEC_Q, salt=500 + ndocs)
    ks = W.normal((S, R, hkv, d), dt, w.wid, W.P_NEW_KV, salt=500 + ndocs)
    vs = W.normal((S, R, hkv, d), dt, w.wid, W.P_NEW_KV, salt=600 + ndocs)
    outs = []
    for s_ in range(S):
        o_s, l_s = c2kv.attn_decode(qs[s_].to(DEV), ks[s_].to(DEV), vs[s_].to(DEV), ck, cv, [L + s_] * R,
                                    [L + s_] * R, theta, return_lse=True)
        outs.append((np32(o_s), np32(l_s)))
    torch.cuda.synchronize()
    for r in checked:
        rk, rv = ref_in[r]
        ro, rl, _, _ = O.append_and_attend(qs[:, r].float().numpy(), ks[:, r].float().numpy(), vs[:, r].float().numpy(),
                                           rk, rv, L, theta, "bf16")
        for s_ in range(S):
            assert_close(outs[s_][0][r], ro[s_], "bf16", f"full {L}: request {r} step {s_}")
            assert_lse_close(outs[s_][1][r], rl[:, s_], "bf16", f"full {L}: request {r} step {s_}")
    del ck, cv
    _free()


def test_full_cache_reuse_llama_k1_compose_then_decode(c2kv):
    """Full-cache reuse: the 8 Llama documents' whole pre-RoPE K/V (4096
    tokens each) composed at k = 1 in the seeded order (every token a slot,
    realigned at the cumulative original lengths: 32768 rows), then a
    64-token question prefill and two decode steps over it, against the
    oracle's compose, prefill and decode."""
    w = W.LLAMA
    d, hq, hkv, theta, dt = w.head_dim, w.hq, w.hkv, w.rope_theta, w.dtype
    order = W.llama_doc_order(w)
    pool_k = [W.normal((4096, hkv, d), dt, w.wid, W.P_K, salt=700 + i) for i in range(8)]
    pool_v = [W.normal((4096, hkv, d), dt, w.wid, W.P_V, salt=700 + i) for i in range(8)]
    M, tq, S = 8 * 4096, 8, 2
    cap = M + tq + S
    ck = torch.zeros((1, hkv, cap, d), dtype=dt, device=DEV)
    cv = torch.zeros_like(ck)
    dk = [x.to(DEV) for x in pool_k]
    dv = [x.to(DEV) for x in pool_v]
    lens, nxt = c2kv.compose([[(dk[t], dv[t], 4096) for t in order]], 1, theta, ck, cv)
    assert lens == [M] and nxt == [M]
    qp = W.normal((1, tq, hq, d), dt, w.wid, W.P_PREFILL, salt=700)
    kp = W.normal((1, tq, hkv, d), dt, w.wid, W.P_NEW_KV, salt=700)
    vp = W.normal((1, tq, hkv, d), dt, w.wid, W.P_NEW_KV, salt=701)
    op, lp = c2kv.attn_prefill(qp.to(DEV), kp.to(DEV), vp.to(DEV), ck, cv, [M], [M], theta, return_lse=True)
    qd = W.normal((S, 1, hq, d), dt, w.wid, W.P_DEC_Q, salt=700)
    kd = W.normal((S, 1, hkv, d), dt, w.wid, W.P_NEW_KV, salt=702)
    vd = W.normal((S, 1, hkv, d), dt, w.wid, W.P_NEW_KV, salt=703)
    dec = []
    for s_ in range(S):
        o_s, l_s = c2kv.attn_decode(qd[s_].to(DEV), kd[s_].to(DEV), vd[s_].to(DEV), ck, cv, [M + tq + s_],
                                    [M + tq + s_], theta, return_lse=True)
        dec.append((np32(o_s)[0], np32(l_s)[0]))
    torch.cuda.synchronize()
    rk, rv, rpos, rnext = O.compose([pool_k[t].float().numpy() for t in order], [pool_v[t].float().numpy() for t in order],
                                    [4096] * 8, 1, theta, "bf16")
    assert rnext == M and np.array_equal(rpos, np.arange(M))
    gk = np32(ck[0, :, :M]).transpose(1, 0, 2)
    pre = np.concatenate([pool_k[t].float().numpy() for t in order])
    assert_rotated_close(gk, rk, pre, "bf16", "k=1 composed keys")
    # the oracle continues from its own composed cache
    ro, rl, _, _ = O.append_and_attend(qp[0].float().numpy(), kp[0].float().numpy(), vp[0].float().numpy(),
                                       rk, rv, M, theta, "bf16")
    assert_close(np32(op)[0], ro, "bf16", "k=1 prefill")
    assert_lse_close(np32(lp)[0], rl, "bf16", "k=1 prefill")
    qs = np.concatenate([qp[0].float().numpy(), qd[:, 0].float().numpy()])
    ks_ = np.concatenate([kp[0].float().numpy(), kd[:, 0].float().numpy()])
    vs_ = np.concatenate([vp[0].float().numpy(), vd[:, 0].float().numpy()])
    ro2, rl2, _, _ = O.append_and_attend(qs, ks_, vs_, rk, rv, M, theta, "bf16")
    for s_ in range(S):
        assert_close(dec[s_][0], ro2[tq + s_], "bf16", f"k=1 decode step {s_}")
        assert_lse_close(dec[s_][1], rl2[:, tq + s_], "bf16", f"k=1 decode step {s_}")
    del ck, cv, dk, dv
    _free()


# ------------------------------------------------- Qwen3-14B extraction

@pytest.mark.parametrize("ratio_k", [4, 8, 16])
def test_qwen3_14b_extract_full(c2kv, ratio_k):
    w = W.QWEN3_14B
    d, hq, hkv, theta, dt = w.head_dim, w.hq, w.hkv, w.rope_theta, w.dtype
    lens = list(w.doc_lens)
    rows = c2kv.packed_rows(lens, ratio_k)
    offs = O.doc_row_offsets(lens, ratio_k)
    print(f"qwen3-14b extraction: 64 x 8192 at k={ratio_k} ({rows} packed rows) in one call", flush=True)
    q = W.device_normal((rows, hq, d), dt, w.wid, W.P_Q, DEV, salt=ratio_k)
    kk = W.device_normal((rows, hkv, d), dt, w.wid, W.P_K, DEV, salt=ratio_k)
    v = W.device_normal((rows, hkv, d), dt, w.wid, W.P_V, DEV, salt=ratio_k)
    checked = (0, len(lens) - 1)
    ref_in = {b: tuple(x[offs[b]:offs[b + 1]].float().cpu().numpy() for x in (q, kk, v)) for b in checked}
    o, lse = c2kv.extract_attn(q, kk, v, lens, ratio_k, ratio_k, theta, return_lse=True)
    torch.cuda.synchronize()
    for b in checked:
        r0, r1 = offs[b], offs[b + 1]
        _check_extract_rows(np32(o[r0:r1]), np32(lse[:, r0:r1]), *ref_in[b], lens[b], ratio_k, ratio_k,
                            theta, f"k={ratio_k} document {b}")
    del q, kk, v, o, lse
    _free()
    got = c2kv.mask_cells(lens, ratio_k, ratio_k)
    dd, sd, ss = O.mask_cell_counts(8192, ratio_k, ratio_k)
    assert got[:3] == (64 * dd, 64 * sd, 64 * ss) and got[3] == 0


# ------------------------------------------- anchor ablation, host-pool load

def test_llama_anchor_extract_full(c2kv):
    """The anchor-token ablation over the whole Llama batch (8 x 4096 tokens,
    k = 4) in one call: sampled document and slot rows of the first and last
    document, every head, against the oracle's anchor mask; exact cell
    counts of the batch."""
    w = W.LLAMA
    d, hq, hkv, k, theta, dt = w.head_dim, w.hq, w.hkv, w.ratio_k, w.rope_theta, w.dtype
    lens = list(w.doc_lens)
    rows = c2kv.packed_rows(lens, k)
    offs = O.doc_row_offsets(lens, k)
    print("llama anchor ablation: extraction of 8 x 4096 in one call", flush=True)
    q = W.normal((rows, hq, d), dt, w.wid, W.P_Q, salt=5)
    kk = W.normal((rows, hkv, d), dt, w.wid, W.P_K, salt=5)
    v = W.normal((rows, hkv, d), dt, w.wid, W.P_V, salt=5)
    o, lse = c2kv.extract_attn(q.to(DEV), kk.to(DEV), v.to(DEV), lens, k, w.sink_len, theta, return_lse=True,
                               anchor=True)
    torch.cuda.synchronize()
    for b in (0, len(lens) - 1):
        r0, r1 = offs[b], offs[b + 1]
        _check_extract_rows(np32(o[r0:r1]), np32(lse[:, r0:r1]), q[r0:r1].float().numpy(),
                            kk[r0:r1].float().numpy(), v[r0:r1].float().numpy(), lens[b], k, w.sink_len,
                            theta, f"anchor document {b}", anchor=True)
    del o, lse
    _free()
    n, m = 4096, O.num_slots(4096, k)
    got = c2kv.mask_cells(lens, k, k, anchor=True)
    assert got[:3] == (8 * n * (n + 1) // 2, 8 * m * n, 8 * (n * m + m * m)) and got[3] == 0


def test_qwen25_pool_from_host_full(c2kv):
    """The Qwen2.5-7B pool kept in pinned host memory: all 32 requests
    composed in one call by reading the slot caches in place, bit-identical
    to composing device copies; positions against the oracle."""
    w = W.QWEN25
    d, hkv, k, theta, dt = w.head_dim, w.hkv, w.ratio_k, w.rope_theta, w.dtype
    pool_n = W.qwen25_pool(w)
    reqs = W.qwen25_requests(w)
    print("qwen25 pool in host memory: generating the 64-document pool", flush=True)
    pool_k = [W.normal((O.num_slots(n, k), hkv, d), dt, w.wid, W.P_K, salt=t) for t, n in enumerate(pool_n)]
    pool_v = [W.normal((O.num_slots(n, k), hkv, d), dt, w.wid, W.P_V, salt=t) for t, n in enumerate(pool_n)]

    def pinned(t):
        p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        p.copy_(t)
        return p
    hk = [pinned(x) for x in pool_k]
    hv = [pinned(x) for x in pool_v]
    dk = [x.to(DEV) for x in pool_k]
    dv = [x.to(DEV) for x in pool_v]
    Ms = [sum(O.num_slots(pool_n[t], k) for t in r) for r in reqs]
    R, cap = len(reqs), max(Ms)
    res = []
    for src_k, src_v in ((hk, hv), (dk, dv)):
        ck = torch.zeros((R, hkv, cap, d), dtype=dt, device=DEV)
        cv = torch.zeros_like(ck)
        pos = torch.full((R, cap), -1, dtype=torch.int32, device=DEV)
        print("qwen25 pool: compose 32 requests in one call", flush=True)
        clen, nxt = c2kv.compose([[(src_k[t], src_v[t], pool_n[t]) for t in r] for r in reqs], k, theta, ck, cv,
                                 pos_out=pos)
        torch.cuda.synchronize()
        res.append((ck, cv, pos, clen, nxt))
    (hck, hcv, hpos, hl, hn), (dck, dcv, dpos, dl, dn) = res
    assert hl == dl == Ms and hn == dn
    assert torch.equal(hck, dck) and torch.equal(hcv, dcv) and torch.equal(hpos, dpos)
    gpos = hpos.cpu().numpy()
    for r, docs in enumerate(reqs):
        rp, _, rnext = O.compose_positions([pool_n[t] for t in docs], k)
        assert hn[r] == rnext and np.array_equal(gpos[r, :Ms[r]], rp)
    del res, hck, hcv, dck, dcv, dk, dv
    _free()
