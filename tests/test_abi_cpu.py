"""The C ABI library on a machine without a GPU: it loads, exports every
function include/c2kv.h declares, its closed forms agree with the oracle,
and invalid arguments are rejected with the documented status before any
HIP call is made."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch  # noqa: F401  (loads the HIP runtime the library shares)

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "c2kv.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, CAPACITY = 0, 1, 2, 3, 4
FAKE = 0x10000   # an aligned non-null address; never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    from compressed_composable_kv_amd import _lib
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(c2kv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), f"{n} declared in c2kv.h but not exported"
    from compressed_composable_kv_amd import _lib
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.c2kv_version()
    for s in range(6):
        assert lib.c2kv_status_string(s)


def test_closed_forms_match_oracle(lib):
    for n in list(range(0, 70)) + [400, 4000, 4096, 8191, 8192]:
        for k in (1, 2, 3, 4, 8, 16):
            m = lib.c2kv_num_slots(n, k)
            assert m == O.num_slots(n, k)
            for j in range(m):
                assert lib.c2kv_slot_position(n, k, j) == O.slot_position(n, k, j)
            assert lib.c2kv_slot_position(n, k, m) == -1
    assert lib.c2kv_num_slots(5, 0) == -1 and lib.c2kv_num_slots(-1, 4) == -1


@pytest.mark.parametrize("d,theta", [(64, 1e4), (128, 5e5), (128, 1e6), (64, 1e6)])
def test_inv_freq_bit_identical_to_oracle(lib, d, theta):
    out = (ctypes.c_float * (d // 2))()
    assert lib.c2kv_rope_inv_freq(d, theta, out) == OK
    got = np.array(out[:], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), O.rope_inv_freq(d, theta).view(np.uint32))


def _arr(vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def _extract(lib, q=FAKE, hq=4, hkv=2, d=128, dt=0, lens=(16, 9), k=4, sink=4, theta=1e4, ws=FAKE, wsb=1 << 30):
    L = _arr(list(lens))
    return lib.c2kv_extract_attn(q, FAKE, FAKE, FAKE, None, L, len(lens), k, sink, hq, hkv, d, theta, dt,
                                 ws, wsb, None)


def test_extract_validation(lib):
    assert _extract(lib, q=None) == INVALID
    assert b"q" in lib.c2kv_last_error()
    assert _extract(lib, q=FAKE + 4) == INVALID          # misaligned
    assert _extract(lib, hq=6, hkv=4) == INVALID
    assert _extract(lib, hq=34, hkv=2) == UNSUPPORTED    # group of 17
    assert _extract(lib, d=96) == UNSUPPORTED
    assert _extract(lib, dt=7) == INVALID
    assert _extract(lib, lens=(16, 0)) == INVALID
    assert _extract(lib, k=0) == INVALID
    assert _extract(lib, sink=-1) == INVALID
    assert _extract(lib, theta=0.5) == INVALID
    assert _extract(lib, theta=float("nan")) == INVALID
    assert _extract(lib, wsb=10) == WORKSPACE
    assert _extract(lib, ws=None) == WORKSPACE
    assert _extract(lib, ws=FAKE + 16) == WORKSPACE
    assert _extract(lib, lens=(1 << 25,)) == CAPACITY


def test_workspace_sizes(lib):
    L = _arr([4096] * 8)
    ext = lib.c2kv_workspace_size_extract(L, 8, 4, 8, 128, 0)
    rows = 8 * (4096 + 1024)
    assert ext >= rows * 8 * 128 * 2 + 4096 * 64 * 8
    assert lib.c2kv_workspace_size_extract(L, 8, 0, 8, 128, 0) == 0
    c = _arr([8192])
    assert lib.c2kv_workspace_size_decode(c, 1, 32, 8, 128, 0) > 0
    assert lib.c2kv_workspace_size_decode(c, 1, 30, 8, 128, 0) == 0
    assert lib.c2kv_workspace_size_prefill(c, 1, 64, 32, 8, 128, 0) > lib.c2kv_workspace_size_decode(c, 1, 32, 8, 128, 0)
    assert lib.c2kv_workspace_size_compose(100) == 0


def _decode_pieces(lib, lens, hq=32, hkv=8, d=128):
    """Key pieces per request of a decode call, from the size of its split
    partials: hq partial rows of d fp32 values and one (m, l) pair per piece
    and head (each array 256-byte aligned; one piece needs none)."""
    ws = lib.c2kv_workspace_size_decode(_arr(lens), len(lens), hq, hkv, d, 0)
    per_piece = hq * d * 4 + hq * 8
    return ws // per_piece if ws > 256 else 1


def test_decode_split_plan(lib):
    """One request: pieces of at least 288 keys (the budget is searched in
    32-key units), at most 768 workgroups (one round of resident workgroups
    at three per CU), one piece when that budget covers the request."""
    # the Llama layer's batch-1 decode after the 64-token question: 29
    # pieces per KV head (232 workgroups, fewer than the 256 CUs)
    assert _decode_pieces(lib, [8192 + 64]) == 29
    for L in list(range(0, 2000, 37)) + list(range(2000, 200000, 4099)):
        n = _decode_pieces(lib, [L])
        keys = L + 1
        assert n <= max(1, -(-keys // 288)), (L, n)
        if n > 1:
            assert n * 8 <= 768, (L, n)
        if keys <= 288:
            assert n == 1, (L, n)


def _compose(lib, segs, ptr, cap=100, k=4, d=128, hkv=2, theta=1e6, base=None):
    from compressed_composable_kv_amd._lib import Segment
    arr = (Segment * len(segs))(*[Segment(*s) for s in segs])
    lens = (ctypes.c_int32 * (len(ptr) - 1))()
    return lib.c2kv_compose(arr, len(segs), _arr(ptr), len(ptr) - 1, _arr(base) if base else None, k, hkv, d,
                            theta, FAKE, FAKE, cap, None, lens, None, 0, None, 0, None)


def test_compose_validation(lib):
    good = (FAKE, FAKE, 256, 40, 0)
    assert _compose(lib, [good], [0, 1], cap=9) == CAPACITY           # 10 slots > cap 9
    assert _compose(lib, [(FAKE, FAKE, 256, 40, 4)], [0, 1]) == INVALID      # unknown flag bit
    assert _compose(lib, [(FAKE, FAKE, 100, 40, 0)], [0, 1]) == INVALID      # stride < hkv*d
    assert _compose(lib, [(FAKE, FAKE, 256, 0, 0)], [0, 1]) == INVALID       # empty document
    assert _compose(lib, [(None, FAKE, 256, 4, 0)], [0, 1]) == INVALID
    assert _compose(lib, [good, good], [0, 1]) == INVALID                     # CSR does not cover segs
    assert _compose(lib, [good, good], [0, 2, 1]) == INVALID                  # not monotone
    assert _compose(lib, [good], [0, 1], base=[(1 << 24) - 10]) == CAPACITY   # position overflow
    assert _compose(lib, [good], [0, 1], k=0) == INVALID


def _decode(lib, lens, pos, cap=100, hq=8, hkv=2, d=128, ws=FAKE, wsb=1 << 30):
    return lib.c2kv_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, cap, _arr(lens), _arr(pos), len(lens), hq, hkv, d,
                                1e6, FAKE, None, 0, ws, wsb, None)


def test_decode_and_prefill_validation(lib):
    assert _decode(lib, [100], [5]) == CAPACITY          # no room for the new row
    assert _decode(lib, [-1], [5]) == INVALID
    assert _decode(lib, [10], [-3]) == CAPACITY
    assert _decode(lib, [10], [5], hq=3) == INVALID
    assert _decode(lib, [5000], [5], cap=6000, wsb=16) == WORKSPACE     # split-K partials need room
    assert _decode(lib, [10], [5], cap=0) == INVALID
    r = lib.c2kv_attn_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, 100, _arr([90]), _arr([0]), 1, 11, 8, 2, 128, 1e6,
                              FAKE, None, 0, FAKE, 1 << 30, None)
    assert r == CAPACITY
    r = lib.c2kv_attn_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, 100, _arr([90]), _arr([0]), 1, 0, 8, 2, 128, 1e6,
                              FAKE, None, 0, FAKE, 1 << 30, None)
    assert r == INVALID


def test_mask_cells_validation(lib):
    out = (ctypes.c_uint64 * 5)()
    assert lib.c2kv_mask_cells(_arr([12]), 1, 4, 4, None, FAKE, 256, None) == INVALID
    assert lib.c2kv_mask_cells(_arr([12]), 1, 4, 4, out, FAKE, 8, None) == WORKSPACE
    assert lib.c2kv_mask_cells(_arr([12]), 1, 0, 4, out, FAKE, 256, None) == INVALID


def test_host_device_ptr_validation(lib):
    out = ctypes.c_void_p()
    assert lib.c2kv_host_device_ptr(None, 16, ctypes.byref(out)) == INVALID
    assert lib.c2kv_host_device_ptr(FAKE, 16, None) == INVALID
    assert lib.c2kv_host_device_ptr(FAKE, 0, ctypes.byref(out)) == INVALID
    assert lib.c2kv_host_device_ptr(ctypes.c_void_p(2 ** 64 - 16), 64, ctypes.byref(out)) == INVALID   # wraps


def test_host_segment_needs_pinned_memory():
    # the binding refuses pageable host tensors before calling the library
    import compressed_composable_kv_amd as c2kv
    with pytest.raises(ValueError, match="pinned"):
        c2kv.host_device_ptr(torch.zeros(4, 2, 64))


def test_compose_staged_validation(lib):
    from compressed_composable_kv_amd._lib import Segment
    segs = (Segment * 1)(Segment(FAKE, FAKE, 256, 40, 0))
    # 10 slots x 2 heads x 128 x bf16, K and V, each 256-byte aligned
    assert lib.c2kv_workspace_size_compose_staged(segs, 1, 4, 2, 128, 0) == 2 * 5120
    assert lib.c2kv_workspace_size_compose_staged(segs, 1, 0, 2, 128, 0) == 0
    assert lib.c2kv_workspace_size_compose_staged(segs, 1, 4, 2, 96, 0) == 0
    lens, nxt = (ctypes.c_int32 * 1)(), (ctypes.c_int32 * 1)()
    ptr = _arr([0, 1])

    def call(cap=16, ws=FAKE, wsb=1 << 20, k=4):
        return lib.c2kv_compose_staged(segs, 1, ptr, 1, None, k, 2, 128, 1e4, FAKE, FAKE, cap, None, lens, nxt, 0,
                                       ws, wsb, None)
    assert call(cap=9) == CAPACITY              # 10 slots > cap, before any HIP query
    assert call(k=0) == INVALID
    assert call(wsb=100) == WORKSPACE
    assert call(ws=None) == WORKSPACE


def test_extract_layer_validation(lib):
    from compressed_composable_kv_amd._lib import LayerWeights
    lens = _arr([100, 37])
    # dm 256, 4/2 heads of 128, ffn 512
    n = lib.c2kv_workspace_size_extract_layer(lens, 2, 4, 256, 4, 2, 128, 512, 0)
    T = 100 + 25 + 37 + 10
    assert n >= T * (256 + 2 * 512 + 512) * 2       # normed input, q, attention output, SwiGLU product
    assert lib.c2kv_workspace_size_extract_layer(lens, 2, 4, 256, 4, 2, 128, 512, 1) == 0     # fp32
    assert lib.c2kv_workspace_size_extract_layer(lens, 2, 4, 200, 4, 2, 128, 512, 0) == 0     # dm off the grid
    assert lib.c2kv_workspace_size_extract_layer(lens, 2, 4, 256, 4, 2, 128, 100, 0) == 0     # ffn off the grid
    assert lib.c2kv_workspace_size_extract_layer(lens, 2, 4, 256, 3, 1, 64, 512, 0) == 0      # hkv*d = 64
    w = LayerWeights(*([FAKE] * 7))

    def call(dm=256, ffn=512, ws=FAKE, wsb=1 << 40, weights=w, eps=1e-5, dt=0):
        return lib.c2kv_extract_layer(FAKE, None, ctypes.byref(weights) if weights else None, FAKE, FAKE, lens, 2,
                                      4, 4, dm, 4, 2, 128, ffn, 5e5, eps, dt, ws, wsb, None)
    assert call(dm=200) == UNSUPPORTED
    assert call(dt=1) == UNSUPPORTED
    assert call(weights=None) == INVALID
    assert call(wsb=100) == WORKSPACE
    assert call(eps=-1.0) == INVALID
    assert call(weights=LayerWeights(*([FAKE] * 6 + [None]))) == INVALID


def test_extract_ex_flag_validation(lib):
    lens = _arr([100])
    r = lib.c2kv_extract_attn_ex(FAKE, FAKE, FAKE, FAKE, None, lens, 1, 4, 4, 8, 2, 128, 1e4, 0, 2, FAKE, 1 << 30, None)
    assert r == INVALID                                   # unknown flag bit
    out = (ctypes.c_uint64 * 5)()
    assert lib.c2kv_mask_cells_ex(lens, 1, 4, 4, 4, out, FAKE, 256, None) == INVALID


def test_implicit_workspace_refused_under_capture(monkeypatch):
    # a graph keeps the workspace address it captured; the binding's cached
    # workspaces can be replaced later, so capture needs an explicit one
    import compressed_composable_kv_amd.ops as ops
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    with pytest.raises(ValueError, match="explicit workspace"):
        ops._workspace(None, "cache", 1024, torch.device("cuda", 0))
