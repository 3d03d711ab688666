"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: positions, offsets, cache lengths, composed V, mask cell counts.
Composed/appended K: within 1 bf16 ulp (fp32: 2^-21 relative bound).
Attention outputs: 2e-2 max-abs for bf16 (1e-5 for fp32) plus a per-row
relative bound of 1e-2 (1e-5).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_util import (assert_close, assert_lse_close, assert_rotated_close, np32,
                         oracle_extract_rows)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def c2kv():
    import compressed_composable_kv_amd as m
    return m


def dtname(dt):
    return "bf16" if dt == torch.bfloat16 else "f32"


def packed_inputs(wid, doc_lens, ratio_k, hq, hkv, d, dt, c2kv, salt=0):
    rows = c2kv.packed_rows(doc_lens, ratio_k)
    assert rows == O.doc_row_offsets(doc_lens, ratio_k)[-1]
    q = W.normal((rows, hq, d), dt, wid, W.P_Q, salt)
    k = W.normal((rows, hkv, d), dt, wid, W.P_K, salt)
    v = W.normal((rows, hkv, d), dt, wid, W.P_V, salt)
    return q, k, v


# ------------------------------------------------------------------ extraction

EXTRACT_CASES = [
    # (doc_lens, k, sink, hq, hkv, d, dtype)
    ((64, 40), 4, 4, 1, 1, 64, torch.float32),                  # tiny workload
    ((300, 129, 7, 1000), 4, 4, 8, 2, 128, torch.bfloat16),    # ragged, several tiles
    ((513, 65, 3), 8, 8, 5, 1, 128, torch.bfloat16),            # G = 5, k not dividing n
    ((250, 97), 16, 16, 7, 1, 128, torch.bfloat16),             # G = 7, partial blocks
    ((1, 2, 5, 33), 4, 4, 2, 2, 64, torch.float32),             # n < k, single token
    ((200, 131), 4, 2, 4, 2, 64, torch.bfloat16),               # sink shorter than k
    ((180,), 4, 0, 2, 1, 128, torch.float32),                   # no sink
    ((96, 70), 4, 9, 4, 4, 64, torch.float32),                  # sink longer than k
    # bf16 on the 32x32 tile at both head sizes, with the predicates above
    ((180,), 4, 0, 2, 1, 128, torch.bfloat16),                  # no sink
    ((96, 70), 4, 9, 4, 4, 64, torch.bfloat16),                 # sink longer than k
    ((1, 2, 5, 33), 4, 4, 2, 2, 64, torch.bfloat16),            # n < k, single token
    ((700, 333), 4, 4, 10, 2, 64, torch.bfloat16),              # G = 5, ragged, several tiles
    ((517, 64), 8, 8, 3, 3, 128, torch.bfloat16),               # G = 1
]


@pytest.mark.parametrize("case", EXTRACT_CASES, ids=lambda c: f"n{'-'.join(map(str, c[0]))}_k{c[1]}_s{c[2]}_G{c[3]//c[4]}_d{c[5]}_{dtname(c[6])}")
def test_extract_parity(c2kv, case):
    doc_lens, k, sink, hq, hkv, d, dt = case
    theta = 1e4 if dt == torch.float32 else 5e5
    q, kk, v = packed_inputs(11, doc_lens, k, hq, hkv, d, dt, c2kv, salt=EXTRACT_CASES.index(case))
    print(f"extract case {case}", flush=True)
    o, lse = c2kv.extract_attn(q.to(DEV), kk.to(DEV), v.to(DEV), doc_lens, k, sink, theta, return_lse=True)
    torch.cuda.synchronize()
    ref = O.extract_attn(q.float().numpy(), kk.float().numpy(), v.float().numpy(), doc_lens, k, sink, theta)
    offs = O.doc_row_offsets(doc_lens, k)
    og, lg = np32(o), np32(lse)
    for b in range(len(doc_lens)):
        ro, rl = ref[b]
        assert_close(og[offs[b]:offs[b + 1]], ro, dtname(dt), f"doc {b} output")
        assert_lse_close(lg[:, offs[b]:offs[b + 1]], rl, dtname(dt), f"doc {b}")


def test_extract_doc_rows_independent_of_slots(c2kv):
    """Document rows never see slots: changing every slot row's K/V leaves
    the document rows' outputs bitwise unchanged."""
    doc_lens, k, hq, hkv, d = (200, 77), 4, 4, 2, 128
    q, kk, v = packed_inputs(12, doc_lens, k, hq, hkv, d, torch.bfloat16, c2kv)
    o1, _ = c2kv.extract_attn(q.to(DEV), kk.to(DEV), v.to(DEV), doc_lens, k, k, 5e5)
    offs = O.doc_row_offsets(doc_lens, k)
    k2, v2 = kk.clone(), v.clone()
    for b, n in enumerate(doc_lens):
        k2[offs[b] + n: offs[b + 1]] *= -3
        v2[offs[b] + n: offs[b + 1]] += 1
    o2, _ = c2kv.extract_attn(q.to(DEV), k2.to(DEV), v2.to(DEV), doc_lens, k, k, 5e5)
    for b, n in enumerate(doc_lens):
        assert torch.equal(o1[offs[b]:offs[b] + n], o2[offs[b]:offs[b] + n])
        assert not torch.equal(o1[offs[b] + n:offs[b + 1]], o2[offs[b] + n:offs[b + 1]])


@pytest.mark.parametrize("doc_lens,k,sink", [((12,), 4, 4), ((64, 40), 4, 4), ((4096,) * 8, 4, 4),
                                             ((1023, 1, 7, 4097), 16, 16), ((8192,) * 3, 8, 8),
                                             ((300, 5), 4, 2), ((70,), 4, 0), ((33, 9), 3, 5)])
def test_mask_cells_bit_exact(c2kv, doc_lens, k, sink):
    got = c2kv.mask_cells(doc_lens, k, sink)
    dd = sd = ss = 0
    for n in doc_lens:
        a, b, c = O.mask_cell_counts(n, k, sink)
        dd, sd, ss = dd + a, sd + b, ss + c
    assert got[:3] == (dd, sd, ss)
    assert got[3] == 0, "an enumerated tile holds no visible cell"


def test_mask_cells_worked_example(c2kv):
    # the 12-token, k=4 figure: 4 + 8 + 8 = 20 slot->doc cells
    assert c2kv.mask_cells([12], 4, 4)[1] == 20


# ---------------------------------------------------------------- composition

def _compose_check(c2kv, reqs_docs, pool_k, pool_v, pool_n, ratio_k, theta, dt, pos_base=None, cap_extra=0):
    R = len(reqs_docs)
    hkv, d = pool_k[0].shape[1], pool_k[0].shape[2]
    Ms = [sum(O.num_slots(pool_n[t], ratio_k) for t in docs) for docs in reqs_docs]
    cap = max(Ms) + cap_extra
    ck = torch.zeros((R, hkv, cap, d), dtype=dt, device=DEV)
    cv = torch.zeros_like(ck)
    pos = torch.full((R, cap), -1, dtype=torch.int32, device=DEV)
    dk = [x.to(DEV) for x in pool_k]
    dv = [x.to(DEV) for x in pool_v]
    requests = [[(dk[t], dv[t], pool_n[t]) for t in docs] for docs in reqs_docs]
    lens, nxt = c2kv.compose(requests, ratio_k, theta, ck, cv, pos_base=pos_base, pos_out=pos)
    torch.cuda.synchronize()
    assert lens == Ms
    for r, docs in enumerate(reqs_docs):
        base = pos_base[r] if pos_base else 0
        rk, rv, rpos, rnext = O.compose([pool_k[t].float().numpy() for t in docs],
                                        [pool_v[t].float().numpy() for t in docs],
                                        [pool_n[t] for t in docs], ratio_k, theta, dtname(dt), base)
        assert nxt[r] == rnext
        assert np.array_equal(pos[r, :Ms[r]].cpu().numpy(), rpos)
        gk = np32(ck[r, :, :Ms[r]]).transpose(1, 0, 2)
        gv = cv[r, :, :Ms[r]].transpose(0, 1).contiguous()
        assert torch.equal(gv.cpu(), torch.cat([pool_v[t] for t in docs]))
        pre = np.concatenate([pool_k[t].float().numpy() for t in docs])
        assert_rotated_close(gk, rk, pre, dtname(dt), f"request {r} keys")
        assert (pos[r, Ms[r]:] == -1).all()
    return ck, cv, lens, nxt


def test_compose_tiny(c2kv):
    w = W.TINY
    q, kk, v = packed_inputs(w.wid, w.doc_lens, w.ratio_k, w.hq, w.hkv, w.head_dim, w.dtype, c2kv)
    views = c2kv.slot_views(kk, v, w.doc_lens, w.ratio_k)
    ck, cv, lens, nxt = _compose_check(c2kv, [[0, 1]], [s[0] for s in views], [s[1] for s in views],
                                       list(w.doc_lens), w.ratio_k, w.rope_theta, w.dtype, cap_extra=24)
    assert lens == [26] and nxt == [104]


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_compose_multi_request_ragged(c2kv, dt):
    g = torch.Generator().manual_seed(5)
    pool_n = [int(x) for x in torch.randint(1, 700, (20,), generator=g)] + [1, 16, 17]
    k = 16 if dt == torch.bfloat16 else 4
    pool_k = [W.normal((O.num_slots(n, k), 3, 128), dt, 13, W.P_K, salt=i) for i, n in enumerate(pool_n)]
    pool_v = [W.normal((O.num_slots(n, k), 3, 128), dt, 13, W.P_V, salt=i) for i, n in enumerate(pool_n)]
    reqs = [[3, 1, 4, 15, 9, 2, 6], [22, 21, 20], [0], list(range(23))[::-1], [7, 7, 8]]
    _compose_check(c2kv, reqs, pool_k, pool_v, pool_n, k, 1e6, dt, pos_base=[0, 5, 100000, 3, 0], cap_extra=3)


def test_compose_launch_table_limits(c2kv):
    """More document occurrences (1120), requests (70) and distinct
    documents (80) than one compose launch's table holds, with documents
    repeated within and across requests: the table is cut into several
    launches, each rebuilding cache rows and positions from its runs."""
    g = torch.Generator().manual_seed(71)
    pool_n = [int(x) for x in torch.randint(1, 60, (80,), generator=g)]
    k, hkv, d, dt = 4, 2, 64, torch.bfloat16
    pool_k = [W.normal((O.num_slots(n, k), hkv, d), dt, 71, W.P_K, salt=i) for i, n in enumerate(pool_n)]
    pool_v = [W.normal((O.num_slots(n, k), hkv, d), dt, 71, W.P_V, salt=i) for i, n in enumerate(pool_n)]
    reqs = [[int(x) for x in torch.randint(0, 80, (16,), generator=g)] for _ in range(70)]
    _compose_check(c2kv, reqs, pool_k, pool_v, pool_n, k, 1e4, dt, pos_base=[3 * r for r in range(70)], cap_extra=1)


@pytest.mark.parametrize("hkv,d,dt", [(5, 64, torch.float32), (6, 128, torch.bfloat16), (80, 128, torch.bfloat16)])
def test_compose_head_counts(c2kv, hkv, d, dt):
    """Head counts whose pairs do not fill a power of two (a workgroup's
    spare pair slots load and store nothing) and more pairs than one
    workgroup covers (a row tile takes several units)."""
    g = torch.Generator().manual_seed(27)
    pool_n = [int(x) for x in torch.randint(1, 300, (6,), generator=g)]
    k = 4
    pool_k = [W.normal((O.num_slots(n, k), hkv, d), dt, 27, W.P_K, salt=i) for i, n in enumerate(pool_n)]
    pool_v = [W.normal((O.num_slots(n, k), hkv, d), dt, 27, W.P_V, salt=i) for i, n in enumerate(pool_n)]
    reqs = [[0, 1, 2], [5, 4, 3, 2], [1]]
    _compose_check(c2kv, reqs, pool_k, pool_v, pool_n, k, 1e6, dt, pos_base=[0, 7, 123], cap_extra=1)


# ------------------------------------------------- prefill / decode parity

def _oracle_cache(slot_k, slot_v, lens, k, theta, dt, base=0):
    return O.compose([x.float().numpy() for x in slot_k], [x.float().numpy() for x in slot_v], lens, k,
                     theta, dtname(dt), base)


def test_tiny_end_to_end(c2kv):
    """Tiny workload: extraction, compose (positions 3..63, 67..103),
    8-token prefill at 104..111, 16 decode steps at 112..127."""
    w = W.TINY
    q, kk, v = packed_inputs(w.wid, w.doc_lens, w.ratio_k, w.hq, w.hkv, w.head_dim, w.dtype, c2kv)
    qd, kd, vd = q.to(DEV), kk.to(DEV), v.to(DEV)
    o, _ = c2kv.extract_attn(qd, kd, vd, w.doc_lens, w.ratio_k, w.sink_len, w.rope_theta)
    views = c2kv.slot_views(kd, vd, w.doc_lens, w.ratio_k)
    cap = 26 + w.tq + w.decode_steps
    ck = torch.zeros((1, 1, cap, 64), dtype=w.dtype, device=DEV)
    cv = torch.zeros_like(ck)
    pos = torch.zeros((1, cap), dtype=torch.int32, device=DEV)
    lens, nxt = c2kv.compose([[(s[0], s[1], s[2]) for s in views]], w.ratio_k, w.rope_theta, ck, cv, pos_out=pos)
    assert lens == [26] and nxt == [104]
    assert pos[0, :26].tolist() == list(range(3, 64, 4)) + list(range(67, 104, 4))
    hviews = c2kv.slot_views(kk, v, w.doc_lens, w.ratio_k)
    rk, rv, _, P = _oracle_cache([s[0] for s in hviews], [s[1] for s in hviews], list(w.doc_lens),
                                 w.ratio_k, w.rope_theta, w.dtype)
    qp = W.normal((1, w.tq, 1, 64), w.dtype, w.wid, W.P_PREFILL)
    kp = W.normal((1, w.tq, 1, 64), w.dtype, w.wid, W.P_NEW_KV)
    vp = W.normal((1, w.tq, 1, 64), w.dtype, w.wid, W.P_NEW_KV, salt=1)
    op, lp = c2kv.attn_prefill(qp.to(DEV), kp.to(DEV), vp.to(DEV), ck, cv, lens, [P], w.rope_theta, return_lse=True)
    ro, rl, rk, rv = O.append_and_attend(qp[0].numpy(), kp[0].numpy(), vp[0].numpy(), rk, rv, P, w.rope_theta, "f32")
    assert_close(np32(op[0]), ro, "f32", "prefill output")
    assert_lse_close(np32(lp[0]), rl, "f32", "prefill")
    L = 26 + w.tq
    for s in range(w.decode_steps):
        qs = W.normal((1, 1, 64), w.dtype, w.wid, W.P_DEC_Q, salt=s)
        ks = W.normal((1, 1, 64), w.dtype, w.wid, W.P_NEW_KV, salt=100 + s)
        vs = W.normal((1, 1, 64), w.dtype, w.wid, W.P_NEW_KV, salt=200 + s)
        od, ld = c2kv.attn_decode(qs.to(DEV), ks.to(DEV), vs.to(DEV), ck, cv, [L], [P + w.tq + s], w.rope_theta,
                                  return_lse=True)
        ro, rl, rk, rv = O.decode_step(qs[0].numpy(), ks[0].numpy(), vs[0].numpy(), rk, rv, P + w.tq + s,
                                       w.rope_theta, "f32")
        assert_close(np32(od[0]), ro, "f32", f"decode step {s}")
        assert_lse_close(np32(ld[0]), rl, "f32", f"decode step {s}")
        L += 1
    gk = np32(ck[0, :, :L]).transpose(1, 0, 2)
    assert torch.equal(cv[0, :, :L].transpose(0, 1).cpu(), torch.from_numpy(rv).to(w.dtype))
    assert np.abs(gk - rk).max() <= 1e-5


@pytest.mark.parametrize("tq,hq,hkv,dt", [(1, 4, 1, torch.bfloat16), (5, 8, 2, torch.bfloat16),
                                          (33, 7, 1, torch.bfloat16), (70, 4, 4, torch.float32),
                                          (64, 32, 8, torch.bfloat16)])
def test_prefill_parity_ragged(c2kv, tq, hq, hkv, dt):
    d = 128 if dt == torch.bfloat16 else 64
    theta = 5e5
    lens = [700, 1, 2500, 64]
    R = len(lens)
    cap = max(lens) + tq + 3
    ck = W.normal((R, hkv, cap, d), dt, 14, W.P_K)
    cv = W.normal((R, hkv, cap, d), dt, 14, W.P_V)
    q = W.normal((R, tq, hq, d), dt, 14, W.P_PREFILL)
    kn = W.normal((R, tq, hkv, d), dt, 14, W.P_NEW_KV)
    vn = W.normal((R, tq, hkv, d), dt, 14, W.P_NEW_KV, salt=1)
    qpos = [lens[r] * 3 + 17 for r in range(R)]
    ckd, cvd = ck.to(DEV), cv.to(DEV)
    o, lse = c2kv.attn_prefill(q.to(DEV), kn.to(DEV), vn.to(DEV), ckd, cvd, lens, qpos, theta, return_lse=True)
    for r in range(R):
        rk = ck[r, :, :lens[r]].transpose(0, 1).float().numpy()
        rv = cv[r, :, :lens[r]].transpose(0, 1).float().numpy()
        ro, rl, rk2, rv2 = O.append_and_attend(q[r].float().numpy(), kn[r].float().numpy(), vn[r].float().numpy(),
                                                rk, rv, qpos[r], theta, dtname(dt))
        assert_close(np32(o[r]), ro, dtname(dt), f"request {r}")
        assert_lse_close(np32(lse[r]), rl, dtname(dt), f"request {r}")
        gk = np32(ckd[r, :, :lens[r] + tq]).transpose(1, 0, 2)
        assert_rotated_close(gk[lens[r]:], rk2[lens[r]:], kn[r].float().numpy(), dtname(dt), f"appended keys {r}")
        assert torch.equal(cvd[r, :, lens[r]:lens[r] + tq].transpose(0, 1).cpu(), vn[r])
        # rows outside [cache_len, cache_len + tq) untouched
        assert torch.equal(ckd[r, :, :lens[r]].cpu(), ck[r, :, :lens[r]])
        assert torch.equal(ckd[r, :, lens[r] + tq:].cpu(), ck[r, :, lens[r] + tq:])


@pytest.mark.parametrize("tq,hq,hkv,d,dt", [(300, 4, 4, 128, torch.bfloat16), (150, 4, 2, 128, torch.float32),
                                            (200, 14, 2, 64, torch.bfloat16)])
def test_prefill_long_question(c2kv, tq, hq, hkv, d, dt):
    """A question longer than a key chunk: its new rows fall into several
    chunks, whose workgroups each rotate and write their own before reading
    them; four query blocks per workgroup at G = 1 (the largest cos/sin
    table); fp32 at d = 128 (one LDS stage); an empty cache."""
    theta = 1e6
    lens = [1000, 37, 0]
    R = len(lens)
    cap = max(lens) + tq + 5
    ck = W.normal((R, hkv, cap, d), dt, 26, W.P_K)
    cv = W.normal((R, hkv, cap, d), dt, 26, W.P_V)
    q = W.normal((R, tq, hq, d), dt, 26, W.P_PREFILL)
    kn = W.normal((R, tq, hkv, d), dt, 26, W.P_NEW_KV)
    vn = W.normal((R, tq, hkv, d), dt, 26, W.P_NEW_KV, salt=1)
    qpos = [5 * lens[r] + 3 for r in range(R)]
    ckd, cvd = ck.to(DEV), cv.to(DEV)
    o, lse = c2kv.attn_prefill(q.to(DEV), kn.to(DEV), vn.to(DEV), ckd, cvd, lens, qpos, theta, return_lse=True)
    for r in range(R):
        rk = ck[r, :, :lens[r]].transpose(0, 1).float().numpy()
        rv = cv[r, :, :lens[r]].transpose(0, 1).float().numpy()
        ro, rl, rk2, _ = O.append_and_attend(q[r].float().numpy(), kn[r].float().numpy(), vn[r].float().numpy(),
                                             rk, rv, qpos[r], theta, dtname(dt))
        assert_close(np32(o[r]), ro, dtname(dt), f"request {r}")
        assert_lse_close(np32(lse[r]), rl, dtname(dt), f"request {r}")
        gk = np32(ckd[r, :, :lens[r] + tq]).transpose(1, 0, 2)
        assert_rotated_close(gk[lens[r]:], rk2[lens[r]:], kn[r].float().numpy(), dtname(dt), f"appended keys {r}")
        assert torch.equal(cvd[r, :, lens[r]:lens[r] + tq].transpose(0, 1).cpu(), vn[r])
        assert torch.equal(ckd[r, :, :lens[r]].cpu(), ck[r, :, :lens[r]])
        assert torch.equal(ckd[r, :, lens[r] + tq:].cpu(), ck[r, :, lens[r] + tq:])


@pytest.mark.parametrize("hq,hkv,d,dt", [(32, 8, 128, torch.bfloat16), (28, 4, 128, torch.bfloat16),
                                         (40, 8, 128, torch.bfloat16), (3, 3, 64, torch.float32)])
def test_decode_parity_varlen(c2kv, hq, hkv, d, dt):
    theta = 1e6
    lens = [9000, 1, 130, 4096, 64, 2047]
    R = len(lens)
    cap = max(lens) + 2
    ck = W.normal((R, hkv, cap, d), dt, 15, W.P_K)
    cv = W.normal((R, hkv, cap, d), dt, 15, W.P_V)
    q = W.normal((R, hq, d), dt, 15, W.P_DEC_Q)
    kn = W.normal((R, hkv, d), dt, 15, W.P_NEW_KV)
    vn = W.normal((R, hkv, d), dt, 15, W.P_NEW_KV, salt=1)
    qpos = [200000 + 7 * r for r in range(R)]
    ckd, cvd = ck.to(DEV), cv.to(DEV)
    o, lse = c2kv.attn_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), ckd, cvd, lens, qpos, theta, return_lse=True)
    for r in range(R):
        rk = ck[r, :, :lens[r]].transpose(0, 1).float().numpy()
        rv = cv[r, :, :lens[r]].transpose(0, 1).float().numpy()
        ro, rl, _, _ = O.decode_step(q[r].float().numpy(), kn[r].float().numpy(), vn[r].float().numpy(),
                                     rk, rv, qpos[r], theta, dtname(dt))
        assert_close(np32(o[r]), ro, dtname(dt), f"request {r}")
        assert_lse_close(np32(lse[r]), rl, dtname(dt), f"request {r}")


def test_decode_split_invariance(c2kv):
    """The split-K merge does not change the result beyond fp32 rounding:
    the same decode over a cache split into many chunks (long cache) and the
    same rows at the front of a request whose chunking differs."""
    d, hq, hkv, dt = 128, 8, 2, torch.bfloat16
    L = 5000
    ck = W.normal((2, hkv, L + 1, d), dt, 16, W.P_K)
    cv = W.normal((2, hkv, L + 1, d), dt, 16, W.P_V)
    ck[1] = ck[0]
    cv[1] = cv[0]
    q = W.normal((1, hq, d), dt, 16, W.P_DEC_Q).repeat(2, 1, 1)
    kn = W.normal((1, hkv, d), dt, 16, W.P_NEW_KV).repeat(2, 1, 1)
    vn = W.normal((1, hkv, d), dt, 16, W.P_NEW_KV, salt=1).repeat(2, 1, 1)
    # request 1 shares the cache; a third long request changes the chunk size
    big = 60000
    ck3 = torch.zeros((3, hkv, big + 1, d), dtype=dt)
    cv3 = torch.zeros_like(ck3)
    ck3[:2, :, :L + 1] = ck
    cv3[:2, :, :L + 1] = cv
    o_a, _ = c2kv.attn_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), ck.to(DEV), cv.to(DEV), [L, L], [L, L], 1e6)
    q3 = torch.cat([q, q[:1]])
    kn3 = torch.cat([kn, kn[:1]])
    vn3 = torch.cat([vn, vn[:1]])
    o_b, _ = c2kv.attn_decode(q3.to(DEV), kn3.to(DEV), vn3.to(DEV), ck3.to(DEV), cv3.to(DEV), [L, L, big],
                              [L, L, big], 1e6)
    assert torch.equal(o_a[0], o_a[1])
    diff = (o_a[0].float() - o_b[0].float()).abs().max().item()
    assert diff <= 2e-3


def test_extract_sink_heavy(c2kv):
    """Attention mass concentrated on the first tokens (keys of the sink
    leaning towards the mean query direction): document and slot rows."""
    doc_lens, k, hq, hkv, d = (700, 129), 4, 8, 2, 128
    dt = torch.bfloat16
    q, kk, v = packed_inputs(17, doc_lens, k, hq, hkv, d, dt, c2kv)
    offs = O.doc_row_offsets(doc_lens, k)
    for b, n in enumerate(doc_lens):
        seg = slice(offs[b], offs[b + 1])
        kk[seg] = W.sink_biased(q[seg], kk[seg], k)
    o, lse = c2kv.extract_attn(q.to(DEV), kk.to(DEV), v.to(DEV), doc_lens, k, k, 5e5, return_lse=True)
    ref = O.extract_attn(q.float().numpy(), kk.float().numpy(), v.float().numpy(), doc_lens, k, k, 5e5)
    og, lg = np32(o), np32(lse)
    for b in range(len(doc_lens)):
        ro, rl = ref[b]
        assert_close(og[offs[b]:offs[b + 1]], ro, "bf16", f"sink-heavy doc {b}")
        assert_lse_close(lg[:, offs[b]:offs[b + 1]], rl, "bf16", f"sink-heavy doc {b}")


def test_decode_sink_heavy(c2kv):
    """Decode over a cache whose first rows dominate the softmax."""
    hq, hkv, d, dt, theta = 32, 8, 128, torch.bfloat16, 5e5
    lens = [3000, 257]
    R = len(lens)
    cap = max(lens) + 1
    ck = W.normal((R, hkv, cap, d), dt, 18, W.P_K)
    cv = W.normal((R, hkv, cap, d), dt, 18, W.P_V)
    q = W.normal((R, hq, d), dt, 18, W.P_DEC_Q)
    kn = W.normal((R, hkv, d), dt, 18, W.P_NEW_KV)
    vn = W.normal((R, hkv, d), dt, 18, W.P_NEW_KV, salt=1)
    for r in range(R):
        rows = ck[r].transpose(0, 1)                                   # [cap][hkv][d]
        ck[r] = W.sink_biased(q[r:r + 1], rows, 4, sigma=6.0).transpose(0, 1)
    qpos = [4 * lens[r] for r in range(R)]
    o, lse = c2kv.attn_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), ck.to(DEV), cv.to(DEV), lens, qpos, theta,
                              return_lse=True)
    for r in range(R):
        rk = ck[r, :, :lens[r]].transpose(0, 1).float().numpy()
        rv = cv[r, :, :lens[r]].transpose(0, 1).float().numpy()
        ro, rl, _, _ = O.decode_step(q[r].float().numpy(), kn[r].float().numpy(), vn[r].float().numpy(),
                                     rk, rv, qpos[r], theta, "bf16")
        assert_close(np32(o[r]), ro, "bf16", f"sink-heavy request {r}")
        assert_lse_close(np32(lse[r]), rl, "bf16", f"sink-heavy request {r}")


# ------------------------------------------------------------- edge cases

def test_decode_and_prefill_on_empty_cache(c2kv):
    """cache_len = 0: the step sees only its own (new) rows."""
    hq, hkv, d, dt, theta = 8, 2, 128, torch.bfloat16, 1e6
    R, tq = 3, 5
    ck = torch.zeros((R, hkv, tq + 1, d), dtype=dt)
    cv = torch.zeros_like(ck)
    q = W.normal((R, tq, hq, d), dt, 19, W.P_PREFILL)
    kn = W.normal((R, tq, hkv, d), dt, 19, W.P_NEW_KV)
    vn = W.normal((R, tq, hkv, d), dt, 19, W.P_NEW_KV, salt=1)
    ckd, cvd = ck.to(DEV), cv.to(DEV)
    o, lse = c2kv.attn_prefill(q.to(DEV), kn.to(DEV), vn.to(DEV), ckd, cvd, [0] * R, [0, 7, 100000], theta,
                               return_lse=True)
    empty = np.zeros((0, hkv, d), np.float32)
    for r, p0 in enumerate([0, 7, 100000]):
        ro, rl, _, _ = O.append_and_attend(q[r].float().numpy(), kn[r].float().numpy(), vn[r].float().numpy(),
                                           empty, empty, p0, theta, "bf16")
        assert_close(np32(o[r]), ro, "bf16", f"prefill request {r}")
        assert_lse_close(np32(lse[r]), rl, "bf16", f"prefill request {r}")
    # a single decode token over an empty cache: o = v_new exactly (up to bf16)
    ck2 = torch.zeros((R, hkv, 1, d), dtype=dt, device=DEV)
    cv2 = torch.zeros_like(ck2)
    od, ld = c2kv.attn_decode(q[:, 0].to(DEV), kn[:, 0].to(DEV), vn[:, 0].to(DEV), ck2, cv2, [0] * R, [3] * R, theta,
                              return_lse=True)
    G = hq // hkv
    for r in range(R):
        ro, rl, _, _ = O.decode_step(q[r, 0].float().numpy(), kn[r, 0].float().numpy(), vn[r, 0].float().numpy(),
                                     empty, empty, 3, theta, "bf16")
        assert_close(np32(od[r]), ro, "bf16", f"decode request {r}")
        for h in range(hq):
            assert torch.equal(od[r, h].cpu(), vn[r, 0, h // G])


def test_extract_more_documents_than_one_launch(c2kv):
    """70 short documents (the kernel-argument table holds 64 per launch)."""
    g = torch.Generator().manual_seed(21)
    doc_lens = [int(x) for x in torch.randint(1, 90, (70,), generator=g)]
    k, hq, hkv, d, dt = 4, 4, 2, 64, torch.bfloat16
    q, kk, v = packed_inputs(20, doc_lens, k, hq, hkv, d, dt, c2kv)
    o, lse = c2kv.extract_attn(q.to(DEV), kk.to(DEV), v.to(DEV), doc_lens, k, k, 5e5, return_lse=True)
    ref = O.extract_attn(q.float().numpy(), kk.float().numpy(), v.float().numpy(), doc_lens, k, k, 5e5)
    offs = O.doc_row_offsets(doc_lens, k)
    og, lg = np32(o), np32(lse)
    for b in range(len(doc_lens)):
        ro, rl = ref[b]
        assert_close(og[offs[b]:offs[b + 1]], ro, "bf16", f"doc {b}")
        assert_lse_close(lg[:, offs[b]:offs[b + 1]], rl, "bf16", f"doc {b}")
    got = c2kv.mask_cells(doc_lens, k, k)
    tot = [sum(O.mask_cell_counts(n, k, k)[i] for n in doc_lens) for i in range(3)]
    assert list(got[:3]) == tot and got[3] == 0


@pytest.mark.parametrize("hq,hkv,d,dt", [(16, 1, 128, torch.bfloat16), (32, 2, 64, torch.bfloat16),
                                         (32, 16, 64, torch.bfloat16)])
def test_decode_more_requests_than_one_launch(c2kv, hq, hkv, d, dt):
    """70 requests (64 per launch), G up to 16, head_dim 64 in bf16.  With 16
    KV heads the first launch has more (request, head) pairs than the chip
    holds workgroups at once, so every request takes one key piece."""
    g = torch.Generator().manual_seed(22)
    lens = [int(x) for x in torch.randint(0, 700, (70,), generator=g)]
    R = len(lens)
    cap = max(lens) + 1
    ck = W.normal((R, hkv, cap, d), dt, 23, W.P_K)
    cv = W.normal((R, hkv, cap, d), dt, 23, W.P_V)
    q = W.normal((R, hq, d), dt, 23, W.P_DEC_Q)
    kn = W.normal((R, hkv, d), dt, 23, W.P_NEW_KV)
    vn = W.normal((R, hkv, d), dt, 23, W.P_NEW_KV, salt=1)
    qpos = [3 * x + 11 for x in lens]
    o, lse = c2kv.attn_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), ck.to(DEV), cv.to(DEV), lens, qpos, 5e5,
                              return_lse=True)
    og, lg = np32(o), np32(lse)
    for r in range(R):
        rk = ck[r, :, :lens[r]].transpose(0, 1).float().numpy()
        rv = cv[r, :, :lens[r]].transpose(0, 1).float().numpy()
        ro, rl, _, _ = O.decode_step(q[r].float().numpy(), kn[r].float().numpy(), vn[r].float().numpy(),
                                     rk, rv, qpos[r], 5e5, dtname(dt))
        assert_close(og[r], ro, dtname(dt), f"request {r}")
        assert_lse_close(lg[r], rl, dtname(dt), f"request {r}")


def test_prefill_more_requests_than_one_launch(c2kv):
    hq, hkv, d, dt, tq = 8, 8, 64, torch.bfloat16, 3
    g = torch.Generator().manual_seed(24)
    lens = [int(x) for x in torch.randint(0, 300, (66,), generator=g)]
    R = len(lens)
    cap = max(lens) + tq
    ck = W.normal((R, hkv, cap, d), dt, 25, W.P_K)
    cv = W.normal((R, hkv, cap, d), dt, 25, W.P_V)
    q = W.normal((R, tq, hq, d), dt, 25, W.P_PREFILL)
    kn = W.normal((R, tq, hkv, d), dt, 25, W.P_NEW_KV)
    vn = W.normal((R, tq, hkv, d), dt, 25, W.P_NEW_KV, salt=1)
    qpos = [x + 1 for x in lens]
    o, lse = c2kv.attn_prefill(q.to(DEV), kn.to(DEV), vn.to(DEV), ck.to(DEV), cv.to(DEV), lens, qpos, 1e4,
                               return_lse=True)
    og, lg = np32(o), np32(lse)
    for r in range(R):
        rk = ck[r, :, :lens[r]].transpose(0, 1).float().numpy()
        rv = cv[r, :, :lens[r]].transpose(0, 1).float().numpy()
        ro, rl, _, _ = O.append_and_attend(q[r].float().numpy(), kn[r].float().numpy(), vn[r].float().numpy(),
                                           rk, rv, qpos[r], 1e4, "bf16")
        assert_close(og[r], ro, "bf16", f"request {r}")
        assert_lse_close(lg[r], rl, "bf16", f"request {r}")


def test_compose_single_token_documents_and_k1(c2kv):
    """Documents of one token (one slot at position offset + 0) and k = 1
    (every token is a slot): degenerate compression ratios."""
    for k in (4, 1):
        pool_n = [1, 1, 2, 5, 1] if k == 4 else [3, 1, 7]
        pool_k = [W.normal((O.num_slots(n, k), 2, 64), torch.bfloat16, 26, W.P_K, salt=i) for i, n in enumerate(pool_n)]
        pool_v = [W.normal((O.num_slots(n, k), 2, 64), torch.bfloat16, 26, W.P_V, salt=i) for i, n in enumerate(pool_n)]
        reqs = [list(range(len(pool_n))), list(range(len(pool_n)))[::-1]]
        _compose_check(c2kv, reqs, pool_k, pool_v, pool_n, k, 5e5, torch.bfloat16, pos_base=[0, 9], cap_extra=2)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_compose_without_realignment(c2kv, dt):
    """The ablation without positional realignment: every document keeps
    its extraction positions (offset pos_base), bit-exact positions against
    the oracle, keys within the rotation bound, values copied; the first
    document equals the realigned composition."""
    g = torch.Generator().manual_seed(77)
    pool_n = [400, 400] + [int(x) for x in torch.randint(1, 300, (5,), generator=g)]
    k, hkv, d = 4, 2, 128
    pool_k = [W.normal((O.num_slots(n, k), hkv, d), dt, 77, W.P_K, salt=i) for i, n in enumerate(pool_n)]
    pool_v = [W.normal((O.num_slots(n, k), hkv, d), dt, 77, W.P_V, salt=i) for i, n in enumerate(pool_n)]
    reqs = [[0, 1], [6, 2, 5, 3, 4]]
    base = [0, 1000]
    Ms = [sum(O.num_slots(pool_n[t], k) for t in r) for r in reqs]
    cap = max(Ms)
    out = {}
    for realign in (False, True):
        ck = torch.zeros((2, hkv, cap, d), dtype=dt, device=DEV)
        cv = torch.zeros_like(ck)
        pos = torch.full((2, cap), -1, dtype=torch.int32, device=DEV)
        requests = [[(pool_k[t].to(DEV), pool_v[t].to(DEV), pool_n[t]) for t in r] for r in reqs]
        lens, nxt = c2kv.compose(requests, k, 5e5, ck, cv, pos_base=base, pos_out=pos, realign=realign)
        torch.cuda.synchronize()
        out[realign] = (ck, cv, pos, lens, nxt)
    ck, cv, pos, lens, nxt = out[False]
    assert lens == Ms and nxt == [base[r] + sum(pool_n[t] for t in reqs[r]) for r in range(2)]
    assert pos[0, :200].tolist() == list(range(3, 400, 4)) * 2
    for r, docs in enumerate(reqs):
        rk, rv, rpos, _ = O.compose([pool_k[t].float().numpy() for t in docs], [pool_v[t].float().numpy() for t in docs],
                                    [pool_n[t] for t in docs], k, 5e5, dtname(dt), base[r], realign=False)
        assert np.array_equal(pos[r, :Ms[r]].cpu().numpy(), rpos)
        assert torch.equal(cv[r, :, :Ms[r]].transpose(0, 1).cpu(), torch.cat([pool_v[t] for t in docs]))
        pre = np.concatenate([pool_k[t].float().numpy() for t in docs])
        assert_rotated_close(np32(ck[r, :, :Ms[r]]).transpose(1, 0, 2), rk, pre, dtname(dt), f"request {r} keys")
        m0 = O.num_slots(pool_n[docs[0]], k)
        assert torch.equal(ck[r, :, :m0], out[True][0][r, :, :m0])


# ------------------------------------------------ anchor-token ablation

@pytest.mark.parametrize("doc_lens,k", [((12,), 4), ((300, 129, 7, 1000), 4), ((513, 65, 3), 8), ((1, 2, 5, 33), 4)])
def test_anchor_mask_cells_exact(c2kv, doc_lens, k):
    """The kernel's own enumeration under the anchor ablation: document
    rows see their causal documents and every slot, slots see everything;
    no enumerated tile is empty for its wave."""
    got = c2kv.mask_cells(list(doc_lens), k, k, anchor=True)
    dd = sum(n * (n + 1) // 2 for n in doc_lens)
    sd = sum(O.num_slots(n, k) * n for n in doc_lens)
    xs = sum(n * O.num_slots(n, k) + O.num_slots(n, k) ** 2 for n in doc_lens)
    assert got[:3] == (dd, sd, xs)
    assert got[3] == 0
    # the structured mask's counts are unchanged by the new classification
    assert c2kv.mask_cells(list(doc_lens), k, k)[:3] == tuple(
        sum(x) for x in zip(*[O.mask_cell_counts(n, k, k) for n in doc_lens]))


ANCHOR_CASES = [
    ((64, 40), 4, 1, 1, 64, torch.float32),
    ((300, 129, 7, 1000), 4, 8, 2, 128, torch.bfloat16),
    ((513, 65, 3), 8, 5, 1, 128, torch.bfloat16),
    ((1, 2, 5, 33), 4, 2, 2, 64, torch.float32),
]


@pytest.mark.parametrize("case", ANCHOR_CASES, ids=lambda c: f"n{'-'.join(map(str, c[0]))}_k{c[1]}_G{c[2]//c[3]}_{dtname(c[5])}")
def test_anchor_extract_parity(c2kv, case):
    doc_lens, k, hq, hkv, d, dt = case
    theta = 1e4 if dt == torch.float32 else 5e5
    q, kk, v = packed_inputs(81, doc_lens, k, hq, hkv, d, dt, c2kv, salt=ANCHOR_CASES.index(case))
    o, lse = c2kv.extract_attn(q.to(DEV), kk.to(DEV), v.to(DEV), list(doc_lens), k, k, theta, return_lse=True,
                               anchor=True)
    torch.cuda.synchronize()
    ref = O.extract_attn(q.float().numpy(), kk.float().numpy(), v.float().numpy(), list(doc_lens), k, k, theta,
                         anchor=True)
    offs = O.doc_row_offsets(doc_lens, k)
    for b in range(len(doc_lens)):
        ro, rl = ref[b]
        assert_close(np32(o[offs[b]:offs[b + 1]]), ro, dtname(dt), f"doc {b} anchor output")
        assert_lse_close(np32(lse[:, offs[b]:offs[b + 1]]), rl, dtname(dt), f"doc {b} anchor")
