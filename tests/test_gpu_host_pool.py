"""Compose from stored slot caches kept in pinned host memory.

Stored caches live in host memory and move to the GPU when a request uses
them ([Explainer] problem section, Fig. 1).  c2kv_compose reads such
segments in place across the host link.  The result must be bit-identical
to composing device copies of the same segments (same kernel, same
arithmetic; only the source address space differs) and match the oracle to
the compose bar: positions, lengths and V bit-exact, K within the rotation
bound.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import assert_rotated_close, np32

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
INVALID = 1


@pytest.fixture(scope="module")
def c2kv():
    import compressed_composable_kv_amd as m
    return m


def pinned(t: torch.Tensor) -> torch.Tensor:
    p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    p.copy_(t)
    return p


def test_host_device_ptr_maps_pinned_memory(c2kv):
    from compressed_composable_kv_amd import _lib
    lib = _lib.load()
    t = pinned(torch.arange(4096 * 2, dtype=torch.float32).view(4096, 2))
    base = c2kv.host_device_ptr(t)
    assert base != 0
    assert c2kv.host_device_ptr(t[100:200]) == base + 100 * 2 * 4
    out = ctypes.c_void_p()
    pageable = np.zeros(1024, dtype=np.float32)
    assert lib.c2kv_host_device_ptr(ctypes.c_void_p(pageable.ctypes.data), pageable.nbytes, ctypes.byref(out)) == INVALID
    dev = torch.zeros(1024, device=DEV)
    assert lib.c2kv_host_device_ptr(ctypes.c_void_p(dev.data_ptr()), 4096, ctypes.byref(out)) == INVALID
    # the library's own queries leave no error behind for the next launch
    assert c2kv.compose([[(dev.view(8, 1, 128)[:1].to(torch.float32), dev.view(8, 1, 128)[:1], 4)]], 4, 1e4,
                        torch.zeros((1, 1, 2, 128), device=DEV), torch.zeros((1, 1, 2, 128), device=DEV)) == ([1], [4])


def _host_vs_device(c2kv, reqs_docs, pool_k, pool_v, pool_n, ratio_k, theta, dt, pos_base=None, mix=False,
                    oracle_reqs=None):
    """Compose the same requests from pinned host segments and from device
    copies; both must agree bit for bit, and the requests listed in
    oracle_reqs (all by default) must match the oracle."""
    R = len(reqs_docs)
    hkv, d = pool_k[0].shape[1], pool_k[0].shape[2]
    Ms = [sum(O.num_slots(pool_n[t], ratio_k) for t in docs) for docs in reqs_docs]
    cap = max(Ms) + 2
    hk = [pinned(x) for x in pool_k]
    hv = [pinned(x) for x in pool_v]
    dk = [x.to(DEV) for x in pool_k]
    dv = [x.to(DEV) for x in pool_v]
    out = {}
    for src in ("host", "device"):
        ck = torch.zeros((R, hkv, cap, d), dtype=dt, device=DEV)
        cv = torch.zeros_like(ck)
        pos = torch.full((R, cap), -1, dtype=torch.int32, device=DEV)
        if src == "host":
            # with mix, every other segment stays on the device
            reqs = [[(dk[t], dv[t], pool_n[t]) if mix and i % 2 else (hk[t], hv[t], pool_n[t])
                     for i, t in enumerate(docs)] for docs in reqs_docs]
        else:
            reqs = [[(dk[t], dv[t], pool_n[t]) for t in docs] for docs in reqs_docs]
        lens, nxt = c2kv.compose(reqs, ratio_k, theta, ck, cv, pos_base=pos_base, pos_out=pos)
        torch.cuda.synchronize()
        out[src] = (ck, cv, pos, lens, nxt)
    (hck, hcv, hpos, hl, hn), (dck, dcv, dpos, dl, dn) = out["host"], out["device"]
    assert hl == dl == Ms and hn == dn
    assert torch.equal(hck, dck) and torch.equal(hcv, dcv) and torch.equal(hpos, dpos)
    for r in (range(R) if oracle_reqs is None else oracle_reqs):
        docs = reqs_docs[r]
        base = pos_base[r] if pos_base else 0
        rk, rv, rpos, rnext = O.compose([pool_k[t].float().numpy() for t in docs],
                                        [pool_v[t].float().numpy() for t in docs],
                                        [pool_n[t] for t in docs], ratio_k, theta,
                                        "bf16" if dt == torch.bfloat16 else "f32", base)
        assert hn[r] == rnext
        assert np.array_equal(hpos[r, :Ms[r]].cpu().numpy(), rpos)
        assert torch.equal(hcv[r, :, :Ms[r]].transpose(0, 1).cpu(), torch.cat([pool_v[t] for t in docs]))
        pre = np.concatenate([pool_k[t].float().numpy() for t in docs])
        assert_rotated_close(np32(hck[r, :, :Ms[r]]).transpose(1, 0, 2), rk, pre,
                             "bf16" if dt == torch.bfloat16 else "f32", f"request {r} keys")


def test_host_pool_tiny(c2kv):
    """The tiny two-document workload, slot caches in host memory:
    positions 3..63 then 67..103."""
    w = W.TINY
    rows = c2kv.packed_rows(w.doc_lens, w.ratio_k)
    k = W.normal((rows, w.hkv, w.head_dim), w.dtype, w.wid, W.P_K)
    v = W.normal((rows, w.hkv, w.head_dim), w.dtype, w.wid, W.P_V)
    views = c2kv.slot_views(k, v, w.doc_lens, w.ratio_k)
    _host_vs_device(c2kv, [[0, 1]], [s[0] for s in views], [s[1] for s in views], list(w.doc_lens),
                    w.ratio_k, w.rope_theta, w.dtype)


def test_host_pool_packed_views(c2kv):
    """Segments that are slot-row views into pinned packed extraction
    outputs ([n doc | m slot] rows per document)."""
    doc_lens, k, hkv, d, dt = [300, 129, 7, 1000], 4, 2, 128, torch.bfloat16
    rows = c2kv.packed_rows(doc_lens, k)
    kk = pinned(W.normal((rows, hkv, d), dt, 31, W.P_K))
    vv = pinned(W.normal((rows, hkv, d), dt, 31, W.P_V))
    views = c2kv.slot_views(kk, vv, doc_lens, k)
    cap = sum(O.num_slots(n, k) for n in doc_lens)
    ck = torch.zeros((1, hkv, cap, d), dtype=dt, device=DEV)
    cv = torch.zeros_like(ck)
    lens, nxt = c2kv.compose([[(s[0], s[1], s[2]) for s in views[::-1]]], k, 5e5, ck, cv)
    torch.cuda.synchronize()
    rk, rv, _, rnext = O.compose([s[0].float().numpy() for s in views[::-1]], [s[1].float().numpy() for s in views[::-1]],
                                 doc_lens[::-1], k, 5e5, "bf16", 0)
    assert lens == [cap] and nxt == [rnext] == [sum(doc_lens)]
    assert torch.equal(cv[0].transpose(0, 1).cpu(), torch.cat([s[1] for s in views[::-1]]))
    pre = np.concatenate([s[0].float().numpy() for s in views[::-1]])
    assert_rotated_close(np32(ck[0]).transpose(1, 0, 2), rk, pre, "bf16", "keys")


@pytest.mark.parametrize("mix", [False, True])
def test_host_pool_ragged_requests(c2kv, mix):
    """Ragged documents at k = 16 (partial last blocks), several requests
    with their own orders and bases; optionally half of the segments on the
    device and half in host memory within one request."""
    g = torch.Generator().manual_seed(41)
    pool_n = [int(x) for x in torch.randint(1, 900, (12,), generator=g)] + [1, 16, 17]
    k, hkv, d, dt = 16, 4, 128, torch.bfloat16
    pool_k = [W.normal((O.num_slots(n, k), hkv, d), dt, 41, W.P_K, salt=i) for i, n in enumerate(pool_n)]
    pool_v = [W.normal((O.num_slots(n, k), hkv, d), dt, 41, W.P_V, salt=i) for i, n in enumerate(pool_n)]
    reqs = [[3, 1, 4, 11, 9, 2, 6], [14, 13, 12], [0], list(range(15))[::-1], [7, 7, 8]]
    _host_vs_device(c2kv, reqs, pool_k, pool_v, pool_n, k, 1e6, dt, pos_base=[0, 5, 100000, 3, 0], mix=mix)


def test_host_pool_full_cache_k1(c2kv):
    """k = 1: every token of a document is kept, so composing from host is
    the full-cache reuse load with positions realigned (fp32 and bf16)."""
    for dt in (torch.float32, torch.bfloat16):
        pool_n = [300, 129, 7]
        pool_k = [W.normal((n, 2, 64), dt, 43, W.P_K, salt=i) for i, n in enumerate(pool_n)]
        pool_v = [W.normal((n, 2, 64), dt, 43, W.P_V, salt=i) for i, n in enumerate(pool_n)]
        _host_vs_device(c2kv, [[2, 0, 1], [1]], pool_k, pool_v, pool_n, 1, 1e4, dt, pos_base=[0, 17])


def test_host_pool_llama_layer(c2kv):
    """The Llama3.1-8B layer at full size: 8 documents of 4096 tokens at
    k = 4 (1024 slots each, 8 KV heads, d = 128, bf16) composed from host
    memory in a seeded order into 8192 rows covering 32768 positions;
    bit-identical to the device-source compose, two requests checked
    against the oracle."""
    w = W.LLAMA
    slots = O.num_slots(4096, w.ratio_k)
    pool_k = [W.normal((slots, w.hkv, w.head_dim), w.dtype, w.wid, W.P_K, salt=50 + i) for i in range(8)]
    pool_v = [W.normal((slots, w.hkv, w.head_dim), w.dtype, w.wid, W.P_V, salt=50 + i) for i in range(8)]
    order = W.llama_doc_order(w)
    _host_vs_device(c2kv, [order, order[:3]], pool_k, pool_v, [4096] * 8, w.ratio_k, w.rope_theta, w.dtype,
                    oracle_reqs=[0])
