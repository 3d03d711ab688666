"""GPU parity of the extractor layer (c2kv_extract_layer) against the oracle.

The layer chains RMSNorm, the Q/K/V projections (frozen weights on document
rows, C2 weights on slot rows), the structured attention, the output
projection, RMSNorm and the SwiGLU FFN with residual adds.  The GPU path
rounds h, q/k/v, the attention output and the SwiGLU product to bf16
(fp32 accumulation); the oracle works in fp64 from the same bf16
inputs.  Bar, derived from that arithmetic: per row, the layer's update
x_out - x_in within 3e-2 relative (L2) of the oracle's and every element of
x_out within 0.1 absolute (a few bf16 half-ulps at |x| ~ 4 plus the
intermediate roundings); slot keys and values (one product of a bf16 input)
within 1e-2 relative per row.  Document rows must not depend on slot rows or
C2 weights at all: bit-identical on the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def c2kv():
    import compressed_composable_kv_amd as m
    return m


def make_weights(wid, dm, hq, hkv, d, ffn, salt=0):
    """bf16 weights N(0, 1) / sqrt(fan_in); gains 1 + 0.1 N(0, 1)."""
    def lin(o, i, p, s):
        return (W.normal((o, i), torch.float32, wid, p, salt=salt * 100 + s) / math.sqrt(i)).to(torch.bfloat16)
    nq = (hq + 2 * hkv) * d
    return {
        "attn_norm": (1.0 + 0.1 * W.normal((dm,), torch.float32, wid, W.P_Q, salt=salt * 100 + 1)).to(torch.bfloat16),
        "wqkv": lin(nq, dm, W.P_K, 2),
        "wqkv_c2": lin(nq, dm, W.P_K, 3),
        "wo": lin(dm, hq * d, W.P_V, 4),
        "ffn_norm": (1.0 + 0.1 * W.normal((dm,), torch.float32, wid, W.P_Q, salt=salt * 100 + 5)).to(torch.bfloat16),
        "w_gate": lin(ffn, dm, W.P_V, 6),
        "w_up": lin(ffn, dm, W.P_V, 8),
        "w_down": lin(dm, ffn, W.P_V, 7),
    }


def oracle_weights(w, ffn):
    return {k: v.float().numpy().astype(np.float64) for k, v in w.items()}


def device_weights(c2kv, w):
    """The library's layout: gate and up rows interleaved in blocks of 16."""
    d = {n: t.to(DEV) for n, t in w.items() if n not in ("w_gate", "w_up")}
    d["w_gate_up"] = c2kv.gate_up_interleave(w["w_gate"], w["w_up"]).to(DEV)
    return d


def run_layer(c2kv, x, w, doc_lens, k, hq, hkv, d, theta, eps, embed=None):
    xd = x.to(DEV).clone()
    rows = xd.shape[0]
    ko = torch.empty((rows, hkv, d), dtype=torch.bfloat16, device=DEV)
    vo = torch.empty_like(ko)
    wd = device_weights(c2kv, w)
    c2kv.extract_layer(xd, wd, ko, vo, doc_lens, k, None, hq, theta, eps,
                       slot_embed=embed.to(DEV) if embed is not None else None)
    torch.cuda.synchronize()
    return xd.cpu(), ko.cpu(), vo.cpu()


LAYER_CASES = [
    # (doc_lens, k, dm, hq, hkv, d, ffn, theta, with slot vector)
    ((100, 37, 300), 4, 256, 4, 2, 128, 512, 5e5, False),     # ragged, several row tiles, slot ranges mid-tile
    ((64, 40), 16, 512, 8, 2, 64, 384, 1e6, True),           # d = 64, G = 4, k = 16, first layer (slot vector)
    ((1, 3, 129), 4, 128, 1, 1, 128, 64, 1e4, True),        # n < k, single-token document, smallest grid
    ((200,), 4, 4096, 32, 8, 128, 14336, 5e5, False),        # Llama3.1-8B layer width, one document
    ((150,), 8, 5120, 40, 8, 128, 17408, 1e6, True),         # Qwen3-14B layer width (G = 5)
    ((97, 40), 16, 3584, 28, 4, 128, 18944, 1e6, False),     # Qwen2.5-7B layer width (G = 7), partial blocks
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: f"n{'-'.join(map(str, c[0]))}_k{c[1]}_dm{c[2]}_ffn{c[6]}")
def test_extract_layer_parity(c2kv, case):
    doc_lens, k, dm, hq, hkv, d, ffn, theta, with_embed = case
    eps = 1e-5
    wid = 61 + LAYER_CASES.index(case)
    rows = c2kv.packed_rows(doc_lens, k)
    x = W.normal((rows, dm), torch.bfloat16, wid, W.P_Q, salt=9)
    w = make_weights(wid, dm, hq, hkv, d, ffn)
    embed = W.normal((dm,), torch.bfloat16, wid, W.P_V, salt=9) if with_embed else None
    gx, gk, gv = run_layer(c2kv, x, w, doc_lens, k, hq, hkv, d, theta, eps, embed)
    fw = oracle_weights(w, ffn)
    rx, rk, rv = O.extractor_layer(x.float().numpy(), fw, doc_lens, k, None, hq, hkv, d, theta, eps,
                                   slot_embed=embed.float().numpy() if embed is not None else None)
    slot = O.slot_row_mask(doc_lens, k)
    x_in = x.float().numpy().astype(np.float64)
    if embed is not None:
        x_in[slot] = embed.float().numpy()
    got = gx.float().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert np.abs(got - rx).max() <= 0.1, f"max-abs {np.abs(got - rx).max()}"
    dg, dr = got - x_in, rx - x_in
    rel = np.linalg.norm(dg - dr, axis=1) / np.maximum(np.linalg.norm(dr, axis=1), 1e-30)
    assert rel.max() <= 3e-2, f"row-relative update error {rel.max()} at row {rel.argmax()}"
    for got_s, ref_s, nm in ((gk.float().numpy()[slot], rk, "slot keys"), (gv.float().numpy()[slot], rv, "slot values")):
        r2 = ref_s.reshape(len(ref_s), -1)
        g2 = got_s.reshape(len(ref_s), -1).astype(np.float64)
        rel = np.linalg.norm(g2 - r2, axis=1) / np.maximum(np.linalg.norm(r2, axis=1), 1e-30)
        assert rel.max() <= 1e-2, f"{nm}: row-relative error {rel.max()}"


def test_extract_layer_doc_rows_ignore_slots(c2kv):
    """Document rows are bit-identical whatever the slot rows hold and
    whatever the C2 projections are (documents never see a slot and use
    only frozen weights)."""
    doc_lens, k, dm, hq, hkv, d, ffn, theta = (130, 77), 4, 256, 4, 2, 128, 256, 5e5
    rows = c2kv.packed_rows(doc_lens, k)
    slot = torch.from_numpy(O.slot_row_mask(doc_lens, k))
    x = W.normal((rows, dm), torch.bfloat16, 70, W.P_Q)
    w = make_weights(70, dm, hq, hkv, d, ffn)
    a = run_layer(c2kv, x, w, doc_lens, k, hq, hkv, d, theta, 1e-5)
    x2 = x.clone()
    x2[slot] = W.normal((int(slot.sum()), dm), torch.bfloat16, 70, W.P_V)
    w2 = dict(w, wqkv_c2=make_weights(71, dm, hq, hkv, d, ffn)["wqkv_c2"])
    for xx, ww in ((x2, w), (x, w2)):
        b = run_layer(c2kv, xx, ww, doc_lens, k, hq, hkv, d, theta, 1e-5)
        for u, v in zip(a, b):
            assert torch.equal(u[~slot], v[~slot])
        assert not torch.equal(a[0][slot], b[0][slot])


def test_extract_layer_more_documents_than_one_launch(c2kv):
    """70 short ragged documents: the q|k|v projection and the slot fill
    run in chunks of 64 documents, and the attention in launches of 64."""
    g = torch.Generator().manual_seed(72)
    doc_lens = [int(x) for x in torch.randint(1, 40, (70,), generator=g)]
    k, dm, hq, hkv, d, ffn, theta, eps = 4, 128, 2, 1, 128, 128, 1e4, 1e-5
    rows = c2kv.packed_rows(doc_lens, k)
    x = W.normal((rows, dm), torch.bfloat16, 72, W.P_Q)
    w = make_weights(72, dm, hq, hkv, d, ffn)
    embed = W.normal((dm,), torch.bfloat16, 72, W.P_V)
    gx, gk, gv = run_layer(c2kv, x, w, doc_lens, k, hq, hkv, d, theta, eps, embed)
    rx, rk, rv = O.extractor_layer(x.float().numpy(), oracle_weights(w, ffn), doc_lens, k, None, hq, hkv, d, theta,
                                   eps, slot_embed=embed.float().numpy())
    slot = O.slot_row_mask(doc_lens, k)
    x_in = x.float().numpy().astype(np.float64)
    x_in[slot] = embed.float().numpy()
    got = gx.float().numpy().astype(np.float64)
    assert np.abs(got - rx).max() <= 0.1
    dg, dr = got - x_in, rx - x_in
    rel = np.linalg.norm(dg - dr, axis=1) / np.maximum(np.linalg.norm(dr, axis=1), 1e-30)
    assert rel.max() <= 3e-2, f"row-relative update error {rel.max()} at row {rel.argmax()}"
    r2 = rk.reshape(len(rk), -1)
    g2 = gk.float().numpy()[slot].reshape(len(rk), -1).astype(np.float64)
    assert (np.linalg.norm(g2 - r2, axis=1) / np.linalg.norm(r2, axis=1)).max() <= 1e-2
