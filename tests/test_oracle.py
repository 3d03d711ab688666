"""Pins for the CPU oracle (no GPU).

Each check ties the oracle to something other than itself: numbers the pages
print (fixtures under tests/golden/, each with its citation), closed forms
derived by hand from the mask rules, brute force over visibility sets built
from the rule statements, torch's scaled_dot_product_attention in fp64 (an
independent library routine), complex multiplication for RoPE, and
invariants.  The last block plants plausible mistakes in a patched copy of
the oracle and checks that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- mask pins


def test_mask_worked_example_counts():
    g = load("mask_n12_k4.json")
    n, k = g["n"], g["k"]
    assert O.num_slots(n, k) == g["slots"]
    M = O.structured_mask(n, k)
    per_slot = [int(M[n + j, :n].sum()) for j in range(g["slots"])]
    assert per_slot == g["slot_doc_cells_per_slot"]
    assert sum(per_slot) == g["slot_doc_cells_total"]
    # plain causal: every slot (sitting after the document) would see all 12 tokens
    assert g["slots"] * n == g["causal_slot_doc_cells"]


def test_mask_worked_example_cells():
    g = load("mask_n12_k4.json")
    n, k = g["n"], g["k"]
    M = O.structured_mask(n, k)
    for slot1, toks in g["visible_doc_tokens_1based"].items():
        j = int(slot1) - 1
        got = [c + 1 for c in range(n) if M[n + j, c]]
        assert got == toks
    for t in g["hidden_from_slot2_1based"]:
        assert not M[n + 1, t - 1]


@pytest.mark.parametrize("n,k,sink", [(12, 4, None), (10, 4, None), (3, 4, None), (40, 4, None),
                                      (64, 4, None), (37, 8, None), (50, 16, None), (9, 1, None),
                                      (20, 4, 2), (20, 4, 7), (5, 3, 0)])
def test_mask_dense_equals_rule_sets(n, k, sink):
    M = O.structured_mask(n, k, sink)
    T = n + O.num_slots(n, k)
    assert M.shape == (T, T)
    for r in range(T):
        assert set(np.nonzero(M[r])[0].tolist()) == O.visible_set(n, k, sink, r)


@pytest.mark.parametrize("n,k", [(12, 4), (64, 4), (40, 4), (4096, 4), (8192, 16), (1000, 16),
                                 (1023, 16), (7, 4), (4, 4), (2, 4), (1, 1), (8192, 8)])
def test_mask_closed_forms(n, k):
    """Hand-derived counts with sink = k: doc->doc n(n+1)/2; slot 0 sees
    min(k, n) cells (its own block is the sink); slot j >= 1 sees the k sink
    cells plus min(k, n - jk) own cells, which sums to (m-1)k + n when n >= k
    (2n - k when k divides n); slot->slot m(m+1)/2."""
    m = (n + k - 1) // k
    dd, sd, ss = O.mask_cell_counts(n, k)
    assert dd == n * (n + 1) // 2
    assert ss == m * (m + 1) // 2
    if n >= k:
        assert sd == (m - 1) * k + n
        if n % k == 0:
            assert sd == 2 * n - k
    else:
        assert sd == n


def test_mask_tiny_counts():
    # Tiny workload documents (64 and 40 tokens at k=4)
    assert O.mask_cell_counts(64, 4) == (2080, 124, 136)
    assert O.mask_cell_counts(40, 4) == (820, 76, 55)


def test_doc_rows_never_see_slots():
    for n, k in [(12, 4), (33, 8), (64, 4)]:
        M = O.structured_mask(n, k)
        assert not M[:n, n:].any()
        assert (M[:n, :n] == np.tril(np.ones((n, n), dtype=bool))).all()
        m = O.num_slots(n, k)
        assert (M[n:, n:] == np.tril(np.ones((m, m), dtype=bool))).all()


# ----------------------------------------------------------- position pins


def test_positions_golden():
    g = load("positions.json")
    k = g["k"]
    assert [O.slot_position(100, k, j) for j in range(2)] == g["first_slot_positions"]
    n = 400
    m = O.num_slots(n, k)
    assert m == g["doc400_slots"]
    p = [O.slot_position(n, k, j) for j in range(m)]
    assert p[0] == g["doc400_first"] and p[-1] == g["doc400_last"]
    assert all(b - a == g["doc400_step"] for a, b in zip(p, p[1:]))
    pos, offs, nxt = O.compose_positions([400, 400], k)
    assert pos[m] == g["second_doc_first_slot"]
    assert offs == [0, 400] and nxt == 800
    assert O.num_slots(4000, 4) == g["compress_4000_k4"]


def test_positions_tiny_composition():
    pos, offs, nxt = O.compose_positions([64, 40], 4)
    assert pos.tolist() == list(range(3, 64, 4)) + list(range(67, 104, 4))
    assert nxt == 104


def test_positions_partial_block():
    assert O.num_slots(10, 4) == 3
    assert [O.slot_position(10, 4, j) for j in range(3)] == [3, 7, 9]
    # every slot stays inside its own document's position range
    pos, _, _ = O.compose_positions([10, 5, 3], 4, pos_base=7)
    assert pos.tolist() == [10, 14, 16, 20, 21, 24]
    assert O.extraction_positions(10, 4).tolist() == list(range(10)) + [3, 7, 9]


# ----------------------------------------------------------- rounding pins


def test_round_bf16_matches_torch():
    x = rng(1).standard_normal(100000).astype(np.float32) * np.float32(3.0)
    x = np.concatenate([x, np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, 65504.0,
                                     1e-30, -7.5e-39, 3.3895e38], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.round_bf16(x).view(np.uint32), ref.view(np.uint32))
    # ties to even by hand
    assert O.round_bf16(np.float32(1 + 2 ** -8)) == np.float32(1.0)
    assert O.round_bf16(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)


# ---------------------------------------------------------------- RoPE pins


def test_rope_inv_freq_closed_form():
    inv = O.rope_inv_freq(64, 10000.0)
    assert inv.dtype == np.float32 and inv.shape == (32,)
    assert inv[0] == np.float32(1.0)
    assert inv[16] == np.float32(0.01)          # theta^(-1/2) with theta = 1e4
    assert inv[8] == np.float32(0.1)            # theta^(-1/4)
    inv2 = O.rope_inv_freq(128, 500000.0)
    assert inv2[32] == np.float32(1.0 / math.sqrt(500000.0))


def test_rope_position_zero_is_identity():
    x = rng(2).standard_normal((5, 3, 64)).astype(np.float32)
    y = O.rope_rotate(x, np.zeros(5, dtype=np.int64), 1e4)
    assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_rope_equals_complex_multiplication():
    """Half-split RoPE is multiplication of z_i = x_i + i x_{i+d/2} by
    exp(i p theta^(-2i/d)); checked in complex128 at moderate positions."""
    d, theta = 128, 500000.0
    x = rng(3).standard_normal((64, 2, d)).astype(np.float32)
    pos = rng(4).integers(0, 5000, 64)
    y = O.rope_rotate(x, pos, theta).astype(np.float64)
    i = np.arange(d // 2)
    ang = pos[:, None] * np.power(theta, -2.0 * i / d)[None, :]
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]).astype(np.complex128) * np.exp(1j * ang)[:, None, :]
    assert np.abs(y[..., : d // 2] - z.real).max() < 2e-3
    assert np.abs(y[..., d // 2:] - z.imag).max() < 2e-3
    # at small positions the fp32 angle is near-exact: tight agreement
    pos = np.arange(64)
    y = O.rope_rotate(x, pos, theta).astype(np.float64)
    ang = pos[:, None] * np.power(theta, -2.0 * i / d)[None, :]
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]).astype(np.complex128) * np.exp(1j * ang)[:, None, :]
    assert np.abs(y[..., : d // 2] - z.real).max() < 1e-5
    assert np.abs(y[..., d // 2:] - z.imag).max() < 1e-5


def test_rope_preserves_pair_norms():
    d = 64
    x = rng(5).standard_normal((32, 1, d)).astype(np.float32)
    y = O.rope_rotate(x, rng(6).integers(0, 100000, 32), 1e6).astype(np.float64)
    x = x.astype(np.float64)
    nx = x[..., :32] ** 2 + x[..., 32:] ** 2
    ny = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert np.allclose(nx, ny, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("base,shift,tol", [(10, 1000, 2e-5), (100, 2 ** 16, 2e-3), (1000, 2 ** 18 - 2000, 1e-2)])
def test_rope_shift_invariance(base, shift, tol):
    """q(P+D).k(p+D) = q(P).k(p): relative rotations only; fp32 angles limit
    the agreement at large positions (angle ulp ~1.6e-2 rad near 2^18)."""
    d = 128
    q = rng(7).standard_normal((1, 1, d)).astype(np.float32)
    k = rng(8).standard_normal((40, 1, d)).astype(np.float32)
    P = base + 50
    kp = base + np.arange(40)
    s0 = (O.rope_rotate(q, np.array([P]), 5e5)[0, 0].astype(np.float64)
          @ O.rope_rotate(k, kp, 5e5)[:, 0].astype(np.float64).T) / math.sqrt(d)
    s1 = (O.rope_rotate(q, np.array([P + shift]), 5e5)[0, 0].astype(np.float64)
          @ O.rope_rotate(k, kp + shift, 5e5)[:, 0].astype(np.float64).T) / math.sqrt(d)
    assert np.abs(s0 - s1).max() <= tol


# ----------------------------------------------------------- attention pins


def _sdpa(q, k, v, mask):
    """torch SDPA in fp64 with GQA by repeating KV heads (contiguous groups)."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(np.asarray(k, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(np.asarray(v, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.unsqueeze(0), kt.unsqueeze(0), vt.unsqueeze(0), attn_mask=torch.from_numpy(mask))
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("n,k,hq,hkv,d", [(12, 4, 1, 1, 8), (10, 4, 4, 2, 8), (9, 2, 3, 1, 4),
                                          (7, 3, 2, 2, 6), (16, 8, 2, 1, 8), (3, 4, 1, 1, 4)])
def test_attention_dense_equals_brute(n, k, hq, hkv, d):
    r = rng(100 + n * k)
    T = n + O.num_slots(n, k)
    q = r.standard_normal((T, hq, d))
    kk = r.standard_normal((T, hkv, d))
    v = r.standard_normal((T, hkv, d))
    M = O.structured_mask(n, k)
    o, lse = O.attention(q, kk, v, M)
    vis = [O.visible_set(n, k, None, row) for row in range(T)]
    ob, lseb = O.attention_brute(q, kk, v, vis)
    assert np.abs(o - ob).max() < 1e-12
    assert np.abs(lse - lseb).max() < 1e-12


@pytest.mark.parametrize("n,k,hq,hkv,d", [(64, 4, 4, 1, 16), (40, 4, 2, 2, 32), (50, 16, 6, 2, 16)])
def test_attention_equals_torch_sdpa(n, k, hq, hkv, d):
    r = rng(200 + n)
    T = n + O.num_slots(n, k)
    q = r.standard_normal((T, hq, d))
    kk = r.standard_normal((T, hkv, d))
    v = r.standard_normal((T, hkv, d))
    M = O.structured_mask(n, k)
    o, lse = O.attention(q, kk, v, M)
    assert np.abs(o - _sdpa(q, kk, v, M)).max() < 1e-12
    # LSE against torch.logsumexp of the masked scaled scores
    G = hq // hkv
    for h in range(hq):
        s = torch.from_numpy(q[:, h] @ kk[:, h // G].T / math.sqrt(d))
        s = s.masked_fill(~torch.from_numpy(M), -float("inf"))
        assert np.abs(torch.logsumexp(s, dim=1).numpy() - lse[h]).max() < 1e-12


def test_extraction_doc_rows_equal_causal_model():
    """Document tokens see no slot, so their outputs equal plain causal
    attention over the document alone (torch SDPA is_causal, fp64)."""
    n, k, hq, hkv, d, theta = 48, 4, 4, 2, 32, 1e4
    m = O.num_slots(n, k)
    r = rng(9)
    q = r.standard_normal((n + m, hq, d)).astype(np.float32)
    kk = r.standard_normal((n + m, hkv, d)).astype(np.float32)
    v = r.standard_normal((n + m, hkv, d)).astype(np.float32)
    o, _ = O.extract_attn(q, kk, v, [n], k, None, theta)[0]
    qr = O.rope_rotate(q[:n], np.arange(n), theta)
    kr = O.rope_rotate(kk[:n], np.arange(n), theta)
    G = hq // hkv
    qt = torch.from_numpy(qr.astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(kr.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(v[:n].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2)
    assert np.abs(o[:n] - ref.numpy()).max() < 1e-12


def _slot_rows_brute(q, kk, v, n, k, theta):
    """Extraction outputs of every row by brute force, with the positions
    written out here from the positions section's rule (document token i at
    i; slot j at the last token of its block, j*k + k - 1, or n - 1 for a
    partial last block) and visibility from the rule statements."""
    m = (n + k - 1) // k
    pos = [i for i in range(n)] + [min(j * k + k - 1, n - 1) for j in range(m)]
    qr = O.rope_rotate(q, np.array(pos), theta)
    kr = O.rope_rotate(kk, np.array(pos), theta)
    vis = [O.visible_set(n, k, None, row) for row in range(n + m)]
    return O.attention_brute(qr, kr, v.astype(np.float64), vis)


@pytest.mark.parametrize("n,k", [(12, 4), (10, 4), (37, 8), (3, 4)])
@pytest.mark.parametrize("G", [1, 2])
def test_extraction_slot_rows_end_to_end(n, k, G):
    """extract_attn's slot rows (and document rows) against brute-force
    attention over q/k rotated at the slot positions the positions section
    fixes (3, 7, ... at k = 4), with visibility sets from the mask rules."""
    hkv, d, theta = 2, 8, 1e4
    hq = G * hkv
    m = O.num_slots(n, k)
    r = rng(500 + 7 * n + k + G)
    q = r.standard_normal((n + m, hq, d)).astype(np.float32)
    kk = r.standard_normal((n + m, hkv, d)).astype(np.float32)
    v = r.standard_normal((n + m, hkv, d)).astype(np.float32)
    o, lse = O.extract_attn(q, kk, v, [n], k, None, theta)[0]
    ob, lb = _slot_rows_brute(q, kk, v, n, k, theta)
    assert np.abs(o[n:] - ob[n:]).max() < 1e-12
    assert np.abs(lse[:, n:] - lb[:, n:]).max() < 1e-12
    assert np.abs(o[:n] - ob[:n]).max() < 1e-12


def test_extraction_multi_doc_independent():
    """Each document is extracted alone: packing several documents gives the
    same per-document results as extracting each by itself."""
    lens, k, theta = [12, 9, 20], 4, 1e4
    offs = O.doc_row_offsets(lens, k)
    r = rng(10)
    q = r.standard_normal((offs[-1], 2, 8)).astype(np.float32)
    kk = r.standard_normal((offs[-1], 1, 8)).astype(np.float32)
    v = r.standard_normal((offs[-1], 1, 8)).astype(np.float32)
    allr = O.extract_attn(q, kk, v, lens, k, None, theta)
    for b, n in enumerate(lens):
        s = slice(offs[b], offs[b + 1])
        one = O.extract_attn(q[s], kk[s], v[s], [n], k, None, theta)[0]
        assert np.array_equal(allr[b][0], one[0])


# ------------------------------------------------------------- compose pins


def _slot_caches(lens, k, hkv, d, seed):
    r = rng(seed)
    ks = [r.standard_normal((O.num_slots(n, k), hkv, d)).astype(np.float32) for n in lens]
    vs = [r.standard_normal((O.num_slots(n, k), hkv, d)).astype(np.float32) for n in lens]
    return ks, vs


def test_compose_v_is_copied_and_k_rounded():
    lens, k = [64, 40], 4
    ks, vs = _slot_caches(lens, k, 2, 64, 11)
    ck, cv, pos, nxt = O.compose(ks, vs, lens, k, 1e4, "bf16")
    assert np.array_equal(cv, np.concatenate(vs))
    assert np.array_equal(O.round_bf16(ck), ck)
    assert nxt == 104 and len(pos) == 26


def test_compose_associative_over_documents():
    """Composing D documents equals composing each alone at pos_base = the
    original length of everything before it."""
    lens, k, theta = [17, 40, 9, 33], 4, 5e5
    ks, vs = _slot_caches(lens, k, 2, 32, 12)
    ck, cv, pos, nxt = O.compose(ks, vs, lens, k, theta, "f32", pos_base=5)
    parts, base = [], 5
    for t, n in enumerate(lens):
        c1, _, p1, _ = O.compose([ks[t]], [vs[t]], [n], k, theta, "f32", pos_base=base)
        parts.append((c1, p1))
        base += n
    assert np.array_equal(ck, np.concatenate([p[0] for p in parts]))
    assert np.array_equal(pos, np.concatenate([p[1] for p in parts]))
    assert nxt == 5 + sum(lens)


def test_compose_first_doc_matches_extraction_rotation():
    """At pos_base 0 the first document's composed keys are exactly its
    extraction-time rotated slot keys."""
    n, k, theta = 30, 4, 1e4
    m = O.num_slots(n, k)
    kk = rng(13).standard_normal((n + m, 1, 16)).astype(np.float32)
    ext = O.rope_rotate(kk, O.extraction_positions(n, k), theta)[n:]
    ck, _, _, _ = O.compose([kk[n:]], [kk[n:]], [n], k, theta, "f32")
    assert np.array_equal(ck, ext)


def test_composed_decode_invariant_to_position_base():
    lens, k, theta, d = [40, 24], 4, 1e4, 64
    ks, vs = _slot_caches(lens, k, 2, d, 14)
    r = rng(15)
    q = r.standard_normal((4, d)).astype(np.float32)
    kn = r.standard_normal((2, d)).astype(np.float32)
    vn = r.standard_normal((2, d)).astype(np.float32)
    outs = []
    for base in (0, 1000):
        ck, cv, _, nxt = O.compose(ks, vs, lens, k, theta, "f32", pos_base=base)
        o, _, _, _ = O.decode_step(q, kn, vn, ck, cv, nxt, theta, "f32")
        outs.append(o)
    assert np.abs(outs[0] - outs[1]).max() < 1e-4


def test_k1_composition_is_full_causal_attention():
    """At k = 1 every token is its own slot at its own position, so decoding
    over the composed cache is ordinary attention over the rotated full
    sequence (torch SDPA, fp64)."""
    lens, theta, d, hq, hkv = [7, 5, 9], 1e4, 16, 4, 2
    ks, vs = _slot_caches(lens, 1, hkv, d, 16)
    ck, cv, pos, nxt = O.compose(ks, vs, lens, 1, theta, "f32")
    assert pos.tolist() == list(range(sum(lens)))
    r = rng(17)
    q = r.standard_normal((hq, d)).astype(np.float32)
    kn = r.standard_normal((hkv, d)).astype(np.float32)
    vn = r.standard_normal((hkv, d)).astype(np.float32)
    o, _, ck2, cv2 = O.decode_step(q, kn, vn, ck, cv, nxt, theta, "f32")
    fullk = O.rope_rotate(np.concatenate(ks + [kn[None]]), np.arange(nxt + 1), theta)
    fullv = np.concatenate(vs + [vn[None]])
    qr = O.rope_rotate(q[None], np.array([nxt]), theta)
    ref = _sdpa(qr, fullk, fullv, np.ones((1, nxt + 1), dtype=bool))[0]
    assert np.abs(o - ref).max() < 1e-12


# ------------------------------------------------------- prefill/decode pins


def test_decode_equals_last_prefill_row():
    lens, k, theta, d, hq, hkv = [20, 12], 4, 5e5, 32, 4, 1
    ks, vs = _slot_caches(lens, k, hkv, d, 18)
    ck, cv, _, P = O.compose(ks, vs, lens, k, theta, "bf16")
    r = rng(19)
    Tq, S = 5, 3
    q = r.standard_normal((Tq + S, hq, d)).astype(np.float32)
    kn = r.standard_normal((Tq + S, hkv, d)).astype(np.float32)
    vn = r.standard_normal((Tq + S, hkv, d)).astype(np.float32)
    # prefill Tq then S decode steps
    _, _, c1k, c1v = O.append_and_attend(q[:Tq], kn[:Tq], vn[:Tq], ck, cv, P, theta, "bf16")
    for s in range(S):
        od, lsed, c1k, c1v = O.decode_step(q[Tq + s], kn[Tq + s], vn[Tq + s], c1k, c1v, P + Tq + s, theta, "bf16")
    # one prefill of all Tq + S tokens: its last row is the last decode step
    op, lsep, c2k, c2v = O.append_and_attend(q, kn, vn, ck, cv, P, theta, "bf16")
    assert np.array_equal(c1k, c2k) and np.array_equal(c1v, c2v)
    assert np.abs(op[-1] - od).max() < 1e-12
    assert np.abs(lsep[:, -1] - lsed).max() < 1e-12


def test_prefill_question_rows_are_causal():
    """Question row t ignores question rows after t (changing a later key
    leaves earlier rows untouched)."""
    r = rng(20)
    ck = r.standard_normal((10, 1, 8)).astype(np.float32)
    cv = r.standard_normal((10, 1, 8)).astype(np.float32)
    q = r.standard_normal((4, 2, 8)).astype(np.float32)
    kn = r.standard_normal((4, 1, 8)).astype(np.float32)
    vn = r.standard_normal((4, 1, 8)).astype(np.float32)
    o1, _, _, _ = O.append_and_attend(q, kn, vn, ck, cv, 40, 1e4, "f32")
    kn2 = kn.copy(); kn2[3] += 5
    vn2 = vn.copy(); vn2[3] -= 5
    o2, _, _, _ = O.append_and_attend(q, kn2, vn2, ck, cv, 40, 1e4, "f32")
    assert np.array_equal(o1[:3], o2[:3])
    assert np.abs(o1[3] - o2[3]).max() > 1e-3


# ---------------------------------------------------------------- byte pins


def test_kv_bytes_golden():
    g = load("kv_bytes.json")
    b = O.kv_bytes_per_token(g["llama3_layers"], g["llama3_kv_heads"], g["llama3_head_dim"], g["bf16_bytes"])
    assert b == g["llama3_kv_bytes_per_token"] == 128 * 1024
    n, k = 4096, 4
    frac = O.decode_kv_bytes(O.num_slots(n, k), 8, 128, 2) / O.decode_kv_bytes(n, 8, 128, 2)
    assert frac == g["decode_read_fraction_k4"]


# ------------------------------------------------------ extractor layer pins

LAYER = dict(dm=64, hq=4, hkv=2, d=16, ffn=96, theta=1e4, eps=1e-5)


def _layer_weights(seed, dm=64, hq=4, hkv=2, d=16, ffn=96):
    r = rng(seed)

    def lin(o, i):
        return r.standard_normal((o, i)) / math.sqrt(i)
    return {"attn_norm": 1.0 + 0.1 * r.standard_normal(dm), "wqkv": lin((hq + 2 * hkv) * d, dm),
            "wqkv_c2": lin((hq + 2 * hkv) * d, dm), "wo": lin(dm, hq * d),
            "ffn_norm": 1.0 + 0.1 * r.standard_normal(dm), "w_gate": lin(ffn, dm), "w_up": lin(ffn, dm),
            "w_down": lin(dm, ffn)}


def _base_layer_torch(x, w, hq, hkv, d, theta, eps):
    """The frozen model's layer over one document alone, written with torch
    ops in fp64: RMSNorm by its formula, RoPE as complex multiplication,
    causal attention by torch SDPA, SwiGLU by torch's silu."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    X = t(x)
    n = X.shape[0]

    def norm(z, g):
        return z * torch.rsqrt((z * z).mean(-1, keepdim=True) + eps) * t(g)
    h = norm(X, w["attn_norm"])
    qkv = h @ t(w["wqkv"]).T
    q = qkv[:, : hq * d].reshape(n, hq, d)
    k = qkv[:, hq * d: (hq + hkv) * d].reshape(n, hkv, d)
    v = qkv[:, (hq + hkv) * d:].reshape(n, hkv, d)
    ang = torch.arange(n, dtype=torch.float64)[:, None] * (theta ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d))
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

    def rope(z):
        c = torch.complex(z[..., : d // 2], z[..., d // 2:]) * rot
        return torch.cat([c.real, c.imag], dim=-1)
    G = hq // hkv
    qt = rope(q).permute(1, 0, 2)[None]
    kt = rope(k).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = v.permute(1, 0, 2).repeat_interleave(G, 0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2)
    X = X + o.reshape(n, hq * d) @ t(w["wo"]).T
    h2 = norm(X, w["ffn_norm"])
    X = X + (torch.nn.functional.silu(h2 @ t(w["w_gate"]).T) * (h2 @ t(w["w_up"]).T)) @ t(w["w_down"]).T
    return X.numpy()


def test_rms_norm_closed_forms():
    g = rng(3).standard_normal(8)
    # a constant row c*1 normalises to sign(c) / sqrt(1 + eps/c^2) times the gain
    for c in (2.0, -0.5):
        y = O.rms_norm(np.full((1, 8), c), g, 1e-5)
        assert np.allclose(y, np.sign(c) / math.sqrt(1 + 1e-5 / c ** 2) * g, rtol=0, atol=1e-15)
    # with eps = 0 the result is invariant to a positive scale and has unit rms before the gain
    x = rng(4).standard_normal((5, 8))
    assert np.allclose(O.rms_norm(3.7 * x, np.ones(8), 0.0), O.rms_norm(x, np.ones(8), 0.0), atol=1e-14)
    assert np.allclose((O.rms_norm(x, np.ones(8), 0.0) ** 2).mean(-1), 1.0, atol=1e-14)


def test_silu_values():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_layer_doc_rows_equal_base_model_layer():
    """Document tokens keep the frozen projections and never see a slot, so
    the document rows of the extractor layer equal the frozen model's layer
    run on the document alone."""
    c = LAYER
    lens, k = [37, 20], 4
    w = _layer_weights(11)
    rows = O.doc_row_offsets(lens, k)
    x = rng(12).standard_normal((rows[-1], c["dm"]))
    out, _, _ = O.extractor_layer(x, w, lens, k, None, c["hq"], c["hkv"], c["d"], c["theta"], c["eps"])
    for b, n in enumerate(lens):
        ref = _base_layer_torch(x[rows[b]: rows[b] + n], w, c["hq"], c["hkv"], c["d"], c["theta"], c["eps"])
        assert np.abs(out[rows[b]: rows[b] + n] - ref).max() < 1e-5


def test_layer_slot_kv_are_c2_projections():
    """The stored slot K/V of a layer are the C2 projections of the slot
    rows' normalised input, before RoPE."""
    c = LAYER
    lens, k = [37, 20], 4
    w = _layer_weights(13)
    x = rng(14).standard_normal((O.doc_row_offsets(lens, k)[-1], c["dm"]))
    _, sk, sv = O.extractor_layer(x, w, lens, k, None, c["hq"], c["hkv"], c["d"], c["theta"], c["eps"])
    xs = x[O.slot_row_mask(lens, k)]
    h = xs / np.sqrt((xs * xs).mean(-1, keepdims=True) + c["eps"]) * w["attn_norm"]
    hd, q0 = c["hkv"] * c["d"], c["hq"] * c["d"]
    assert np.abs(sk.reshape(len(xs), hd) - h @ w["wqkv_c2"][q0: q0 + hd].T).max() < 1e-12
    assert np.abs(sv.reshape(len(xs), hd) - h @ w["wqkv_c2"][q0 + hd:].T).max() < 1e-12


def test_layer_slot_rows_and_c2_weights_leave_doc_rows_alone():
    """Changing the slot rows' input or the C2 projections changes slot rows
    and leaves every document row bit for bit the same."""
    c = LAYER
    lens, k = [29, 8], 4
    w = _layer_weights(15)
    slot = O.slot_row_mask(lens, k)
    x = rng(16).standard_normal((len(slot), c["dm"]))
    base, _, _ = O.extractor_layer(x, w, lens, k, None, c["hq"], c["hkv"], c["d"], c["theta"], c["eps"])
    x2 = x.copy()
    x2[slot] += 1.0
    w2 = dict(w, wqkv_c2=_layer_weights(17)["wqkv_c2"])
    for xx, ww in ((x2, w), (x, w2)):
        out, _, _ = O.extractor_layer(xx, ww, lens, k, None, c["hq"], c["hkv"], c["d"], c["theta"], c["eps"])
        assert np.array_equal(out[~slot], base[~slot])
        assert np.abs(out[slot] - base[slot]).max() > 1e-3


def test_layer_slot_embed_sets_slot_inputs():
    """With the shared slot vector given, the slot rows' own input values no
    longer matter, and the result equals writing that vector into them."""
    c = LAYER
    lens, k = [30, 9], 4
    w = _layer_weights(18)
    slot = O.slot_row_mask(lens, k)
    x = rng(19).standard_normal((len(slot), c["dm"]))
    e = rng(20).standard_normal(c["dm"])
    a = O.extractor_layer(x, w, lens, k, None, c["hq"], c["hkv"], c["d"], c["theta"], c["eps"], slot_embed=e)
    x2 = x.copy()
    x2[slot] = e
    b = O.extractor_layer(x2, w, lens, k, None, c["hq"], c["hkv"], c["d"], c["theta"], c["eps"])
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ------------------------------------------- ablation without realignment

def test_no_realignment_positions_golden():
    """Without realignment both 400-token documents of the worked example
    keep slots 3, 7, ..., 399 (the second document's first slot is 3, not
    403); the question still starts after both original lengths."""
    g = load("positions.json")
    pos, offs, nxt = O.compose_positions([400, 400], 4, realign=False)
    first = list(range(3, 400, 4))
    assert pos.tolist() == first + first
    assert offs == [0, 0] and nxt == 800
    # with realignment, the printed 403
    assert O.compose_positions([400, 400], 4)[0][100] == 403 == g["second_doc_first_slot"]


def test_no_realignment_equals_each_document_alone():
    """Composing without realignment gives, row for row, what composing each
    document alone at the same base gives; the first document is the same
    with or without realignment."""
    lens, k, hkv, d = [37, 20, 9], 4, 2, 16
    sk, sv = _slot_caches(lens, k, hkv, d, 31)
    ck, cv, pos, _ = O.compose(sk, sv, lens, k, 1e4, "f32", 5, realign=False)
    row = 0
    for t, n in enumerate(lens):
        a_k, a_v, a_pos, _ = O.compose([sk[t]], [sv[t]], [n], k, 1e4, "f32", 5)
        m = len(a_pos)
        assert np.array_equal(ck[row:row + m], a_k) and np.array_equal(cv[row:row + m], a_v)
        assert np.array_equal(pos[row:row + m], a_pos)
        row += m
    r_k, _, r_pos, _ = O.compose(sk, sv, lens, k, 1e4, "f32", 5)
    m0 = O.num_slots(lens[0], k)
    assert np.array_equal(r_k[:m0], ck[:m0]) and not np.array_equal(r_pos[m0:], pos[m0:])


# ------------------------------------------------ anchor-token ablation

@pytest.mark.parametrize("n,k", [(12, 4), (13, 4), (3, 4), (40, 16)])
def test_anchor_mask_dense_equals_rule_sets_and_counts(n, k):
    """The anchor ablation's mask, dense and as sets from the rule
    statement, and its closed-form counts: documents n(n+1)/2 + n m,
    anchors m n + m^2."""
    m = O.num_slots(n, k)
    M = O.structured_mask(n, k, None, anchor=True)
    for r in range(n + m):
        assert set(np.nonzero(M[r])[0].tolist()) == O.visible_set(n, k, None, r, anchor=True)
    assert M[:n].sum() == n * (n + 1) // 2 + n * m
    assert M[n:].sum() == m * n + m * m
    # the structured mask is a subset of the anchor mask
    S = O.structured_mask(n, k, None)
    assert not (S & ~M).any()


def test_anchor_attention_equals_brute_force():
    n, k, hq, hkv, d = 21, 4, 2, 1, 8
    m = O.num_slots(n, k)
    r = rng(33)
    q = r.standard_normal((n + m, hq, d))
    kk = r.standard_normal((n + m, hkv, d))
    v = r.standard_normal((n + m, hkv, d))
    M = O.structured_mask(n, k, None, anchor=True)
    o, lse = O.attention(q, kk, v, M)
    ob, lb = O.attention_brute(q, kk, v, [O.visible_set(n, k, None, i, anchor=True) for i in range(n + m)])
    assert np.abs(o - ob).max() < 1e-12 and np.abs(lse - lb).max() < 1e-12


def test_anchor_extraction_changes_document_rows():
    """Under the ablation document rows read the anchors, so they no longer
    equal the frozen model's (they do under the structured mask)."""
    n, k, hq, hkv, d, theta = 30, 4, 2, 1, 16, 1e4
    m = O.num_slots(n, k)
    r = rng(35)
    q = r.standard_normal((n + m, hq, d)).astype(np.float32)
    kk = r.standard_normal((n + m, hkv, d)).astype(np.float32)
    v = r.standard_normal((n + m, hkv, d)).astype(np.float32)
    a, _ = O.extract_attn(q, kk, v, [n], k, None, theta, anchor=True)[0]
    s_, _ = O.extract_attn(q, kk, v, [n], k, None, theta)[0]
    assert np.abs(a[:n] - s_[:n]).max() > 1e-3


# --------------------------------------------------- planted-mistake checks


def _pins_fail(monkeypatch, name, fn, pin):
    monkeypatch.setattr(O.c2kv_oracle, name, fn)
    monkeypatch.setattr(O, name, fn)
    with pytest.raises(AssertionError):
        pin()


def test_planted_position_mistake_caught(monkeypatch):
    # slot position off by one
    _pins_fail(monkeypatch, "slot_position", lambda n, k, j: min(j * k + k, n - 1), test_positions_golden)


def test_planted_mask_mistake_caught(monkeypatch):
    orig = O.c2kv_oracle.structured_mask

    def no_sink(n, k, sink_len=None):
        M = orig(n, k, sink_len)
        m = O.num_slots(n, k)
        for j in range(1, m):
            M[n + j, :min(k, n)] = False
        return M
    _pins_fail(monkeypatch, "structured_mask", no_sink, test_mask_worked_example_counts)


def test_planted_rope_sign_mistake_caught(monkeypatch):
    orig = O.c2kv_oracle.rope_cos_sin

    def flipped(pos, d, theta):
        c, s = orig(pos, d, theta)
        return c, -s
    monkeypatch.setattr(O.c2kv_oracle, "rope_cos_sin", flipped)
    with pytest.raises(AssertionError):
        test_rope_equals_complex_multiplication()


def test_planted_gqa_mapping_mistake_caught(monkeypatch):
    orig = O.c2kv_oracle.attention

    def wrong_gqa(q, k, v, mask, row_chunk=1024):
        Hq, Hkv = q.shape[1], k.shape[1]
        G = Hq // Hkv
        perm = [h % Hkv for h in range(Hq)]       # interleaved instead of contiguous groups
        kk = np.stack([k[:, p] for p in perm], axis=1)
        vv = np.stack([v[:, p] for p in perm], axis=1)
        return orig(q, kk, vv, mask, row_chunk)
    monkeypatch.setattr(O.c2kv_oracle, "attention", wrong_gqa)
    monkeypatch.setattr(O, "attention", wrong_gqa)
    with pytest.raises(AssertionError):
        test_attention_equals_torch_sdpa(50, 16, 6, 2, 16)


def test_planted_offset_mistake_caught(monkeypatch):
    orig = O.c2kv_oracle.compose_positions

    def no_cumulative(lens, k, pos_base=0):
        pos, offs, nxt = orig(lens, k, pos_base)
        m0 = O.num_slots(lens[0], k)
        pos = pos.copy()
        pos[m0:] -= lens[0]                      # forget the first document's length
        return pos, offs, nxt
    _pins_fail(monkeypatch, "compose_positions", no_cumulative, test_positions_golden)


def test_planted_layer_weight_mistake_caught(monkeypatch):
    # slot rows projected with the frozen weights instead of the C2 ones
    orig = O.c2kv_oracle.extractor_layer

    def frozen_for_slots(x, w, *a, **kw):
        return orig(x, dict(w, wqkv_c2=w["wqkv"]), *a, **kw)
    monkeypatch.setattr(O, "extractor_layer", frozen_for_slots)
    with pytest.raises(AssertionError):
        test_layer_slot_kv_are_c2_projections()


def test_planted_layer_norm_mistake_caught(monkeypatch):
    # RMSNorm without the gain
    monkeypatch.setattr(O.c2kv_oracle, "rms_norm", lambda x, g, eps: np.asarray(x, dtype=np.float64) / np.sqrt(
        np.mean(np.asarray(x, dtype=np.float64) ** 2, axis=-1, keepdims=True) + eps))
    with pytest.raises(AssertionError):
        test_layer_doc_rows_equal_base_model_layer()


def test_planted_slot_rotation_at_block_start_caught(monkeypatch):
    # slots rotated at the first token of their block (j*k) instead of its last
    def at_block_start(n, k):
        m = O.num_slots(n, k)
        return np.array(list(range(n)) + [j * k for j in range(m)], dtype=np.int64)
    monkeypatch.setattr(O.c2kv_oracle, "extraction_positions", at_block_start)
    with pytest.raises(AssertionError):
        test_extraction_slot_rows_end_to_end(12, 4, 2)


def test_planted_slot_rotation_at_row_index_caught(monkeypatch):
    # slots rotated at their packed row index (n + j) instead of their block's end
    monkeypatch.setattr(O.c2kv_oracle, "extraction_positions",
                        lambda n, k: np.arange(n + O.num_slots(n, k), dtype=np.int64))
    with pytest.raises(AssertionError):
        test_extraction_slot_rows_end_to_end(10, 4, 1)
