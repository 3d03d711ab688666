"""Python binding of the C2KV C ABI: the same entry points, taking torch
tensors.  Argument marshalling only -- every step runs in libc2kv.so's HIP
kernels; torch provides device memory and the current stream.  Raises
ImportError when the library is missing and C2KVError on any failure status.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import C2KVError, Segment, check, load

_DT = {torch.bfloat16: 0, torch.float32: 1}


def _arr_i32(vals: Sequence[int]):
    a = (ctypes.c_int32 * max(1, len(vals)))(*[int(v) for v in vals])
    return a


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t: torch.Tensor, name: str, dtype=None) -> None:
    _need(isinstance(t, torch.Tensor) and t.is_cuda, f"{name} must be a CUDA tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}")


class _Workspaces:
    """Per-device scratch buffers, grown on demand (the library ignores
    their contents on entry)."""

    def __init__(self):
        self._bufs = {}

    def get(self, key, nbytes: int, device: torch.device, zero: bool) -> torch.Tensor:
        k = (key, device.index)
        buf = self._bufs.get(k)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(256, (nbytes + 255) // 256 * 256), dtype=torch.uint8, device=device)
            if zero:
                check(load().c2kv_workspace_init(_ptr(buf), buf.numel(), _stream(device)))
            self._bufs[k] = buf
        return buf


WORKSPACES = _Workspaces()


def _workspace(given: Optional[torch.Tensor], key: str, nbytes: int, device: torch.device) -> torch.Tensor:
    if given is None:
        # a captured graph keeps the address it saw; a cached buffer can be
        # replaced (and freed) by a later, larger call, so capture needs a
        # workspace that the caller owns for the graph's lifetime
        _need(not torch.cuda.is_current_stream_capturing(),
              "pass an explicit workspace= when capturing a graph (size it with workspace_size_*)")
        return WORKSPACES.get(key, nbytes, device, zero=False)
    _dev_tensor(given, "workspace", torch.uint8)
    _need(given.numel() >= nbytes, f"workspace has {given.numel()} bytes, {nbytes} needed")
    return given


def workspace_size_extract(doc_lens: Sequence[int], ratio_k: int, hkv: int, head_dim: int, dtype) -> int:
    return int(load().c2kv_workspace_size_extract(_arr_i32(doc_lens), len(doc_lens), ratio_k, hkv, head_dim,
                                                  _DT[dtype]))


def workspace_size_prefill(cache_len: Sequence[int], tq: int, hq: int, hkv: int, head_dim: int, dtype) -> int:
    return int(load().c2kv_workspace_size_prefill(_arr_i32(cache_len), len(cache_len), tq, hq, hkv, head_dim,
                                                  _DT[dtype]))


def workspace_size_decode(cache_len: Sequence[int], hq: int, hkv: int, head_dim: int, dtype) -> int:
    return int(load().c2kv_workspace_size_decode(_arr_i32(cache_len), len(cache_len), hq, hkv, head_dim,
                                                 _DT[dtype]))


# ------------------------------------------------------------ closed forms

def version() -> str:
    return load().c2kv_version().decode()


def num_slots(n: int, k: int) -> int:
    return int(load().c2kv_num_slots(n, k))


def slot_position(n: int, k: int, j: int) -> int:
    return int(load().c2kv_slot_position(n, k, j))


def rope_inv_freq(head_dim: int, rope_theta: float) -> List[float]:
    out = (ctypes.c_float * (head_dim // 2))()
    check(load().c2kv_rope_inv_freq(head_dim, rope_theta, out))
    return list(out)


def packed_rows(doc_lens: Sequence[int], ratio_k: int) -> int:
    return sum(int(n) + num_slots(int(n), ratio_k) for n in doc_lens)


# -------------------------------------------------------------- extraction

def extract_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, doc_lens: Sequence[int],
                 ratio_k: int, sink_len: Optional[int] = None, rope_theta: float = 10000.0,
                 return_lse: bool = False, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, anchor: bool = False
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Structured-flow extraction attention (c2kv_extract_attn; with
    anchor=True the anchor-token ablation, c2kv_extract_attn_ex).

    q [sum_T][hq][d], k/v [sum_T][hkv][d], rows packed per document as
    [n doc | ceil(n/k) slots].  Returns (o [sum_T][hq][d], lse [hq][sum_T] or None).
    """
    lib = load()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, nm, q.dtype)
    _need(q.dtype in _DT, "dtype must be bfloat16 or float32")
    rows, hq, d = q.shape
    _need(k.shape == v.shape and k.shape[0] == rows and k.shape[2] == d, "k/v shape mismatch")
    hkv = k.shape[1]
    _need(rows == packed_rows(doc_lens, ratio_k), "q rows != packed rows of doc_lens")
    if sink_len is None:
        sink_len = ratio_k
    o = out if out is not None else torch.empty_like(q)
    _dev_tensor(o, "out", q.dtype)
    lse = torch.empty((hq, rows), dtype=torch.float32, device=q.device) if return_lse else None
    lens = _arr_i32(doc_lens)
    dt = _DT[q.dtype]
    nbytes = lib.c2kv_workspace_size_extract(lens, len(doc_lens), ratio_k, hkv, d, dt)
    _need(nbytes > 0, "invalid extraction arguments")
    ws = _workspace(workspace, "extract", nbytes, q.device)
    check(lib.c2kv_extract_attn_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), lens, len(doc_lens),
                                   ratio_k, sink_len, hq, hkv, d, float(rope_theta), dt,
                                   _lib.EXTRACT_ANCHOR if anchor else 0, _ptr(ws), ws.numel(), _stream(q.device)))
    return o, lse


LAYER_WEIGHTS = ("attn_norm", "wqkv", "wqkv_c2", "wo", "ffn_norm", "w_gate_up", "w_down")


def gate_up_interleave(w_gate: torch.Tensor, w_up: torch.Tensor) -> torch.Tensor:
    """The w_gate_up layout c2kv_extract_layer takes: blocks of 16 gate rows,
    each followed by the 16 up rows of the same FFN columns (a row
    permutation of [gate; up])."""
    ffn, dm = w_gate.shape
    _need(w_up.shape == w_gate.shape and ffn % 16 == 0, "gate/up shapes")
    return torch.stack([w_gate.reshape(ffn // 16, 16, dm), w_up.reshape(ffn // 16, 16, dm)], dim=1).reshape(2 * ffn, dm)


def workspace_size_extract_layer(doc_lens: Sequence[int], ratio_k: int, dm: int, hq: int, hkv: int,
                                 head_dim: int, ffn: int) -> int:
    return int(load().c2kv_workspace_size_extract_layer(_arr_i32(doc_lens), len(doc_lens), ratio_k, dm, hq, hkv,
                                                        head_dim, ffn, _DT[torch.bfloat16]))


def extract_layer(x: torch.Tensor, weights: dict, k_out: torch.Tensor, v_out: torch.Tensor,
                  doc_lens: Sequence[int], ratio_k: int, sink_len: Optional[int], hq: int,
                  rope_theta: float, rms_eps: float, slot_embed: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> None:
    """One extractor layer (c2kv_extract_layer), bf16.  x [sum_T][dm] is
    updated in place; k_out/v_out [sum_T][hkv][d] receive the layer's
    pre-RoPE keys and values (their slot rows are the stored C2KV).
    weights: {attn_norm [dm], wqkv and wqkv_c2 [(hq+2hkv)d][dm], wo [dm][hq d],
    ffn_norm [dm], w_gate_up [2 ffn][dm] (gate_up_interleave of the gate and
    up matrices), w_down [dm][ffn]} on the device."""
    lib = load()
    _dev_tensor(x, "x", torch.bfloat16)
    _dev_tensor(k_out, "k_out", torch.bfloat16)
    _dev_tensor(v_out, "v_out", torch.bfloat16)
    for nm in LAYER_WEIGHTS:
        _need(nm in weights, f"weights needs {nm}")
        _dev_tensor(weights[nm], nm, torch.bfloat16)
    rows, dm = x.shape
    _, hkv, d = k_out.shape
    ffn = weights["w_down"].shape[1]
    _need(rows == packed_rows(doc_lens, ratio_k) and k_out.shape[0] == rows and v_out.shape == k_out.shape,
          "x/k_out/v_out rows must be the packed rows of doc_lens")
    _need(weights["wqkv"].shape == ((hq + 2 * hkv) * d, dm) and weights["wqkv_c2"].shape == weights["wqkv"].shape,
          "wqkv shape")
    _need(weights["wo"].shape == (dm, hq * d) and weights["w_gate_up"].shape == (2 * ffn, dm)
          and weights["w_down"].shape == (dm, ffn), "wo / w_gate_up / w_down shape")
    _need(weights["attn_norm"].shape == (dm,) and weights["ffn_norm"].shape == (dm,), "norm gain shape")
    if slot_embed is not None:
        _dev_tensor(slot_embed, "slot_embed", torch.bfloat16)
        _need(slot_embed.shape == (dm,), "slot_embed must be [dm]")
    if sink_len is None:
        sink_len = ratio_k
    lens = _arr_i32(doc_lens)
    nbytes = lib.c2kv_workspace_size_extract_layer(lens, len(doc_lens), ratio_k, dm, hq, hkv, d, ffn,
                                                   _DT[torch.bfloat16])
    _need(nbytes > 0, "invalid extractor layer arguments (shapes off the tile grid?)")
    ws = _workspace(workspace, "layer", nbytes, x.device)
    lw = _lib.LayerWeights(*[weights[nm].data_ptr() for nm in LAYER_WEIGHTS])
    check(lib.c2kv_extract_layer(_ptr(x), _ptr(slot_embed), ctypes.byref(lw), _ptr(k_out), _ptr(v_out), lens,
                                 len(doc_lens), ratio_k, sink_len, dm, hq, hkv, d, ffn, float(rope_theta),
                                 float(rms_eps), _DT[torch.bfloat16], _ptr(ws), ws.numel(), _stream(x.device)))


def slot_views(k: torch.Tensor, v: torch.Tensor, doc_lens: Sequence[int], ratio_k: int
               ) -> List[Tuple[torch.Tensor, torch.Tensor, int]]:
    """The stored C2KV of each document: views of its slot rows in the packed
    extraction K/V (pre-RoPE), as (k [m][hkv][d], v [m][hkv][d], n)."""
    segs, row = [], 0
    for n in doc_lens:
        m = num_slots(int(n), ratio_k)
        segs.append((k[row + n: row + n + m], v[row + n: row + n + m], int(n)))
        row += n + m
    return segs


# ------------------------------------------------------------- composition

def _segment_table(requests, cache_k: torch.Tensor, staged: bool, realign: bool = True):
    R, hkv, cap, d = cache_k.shape
    _need(len(requests) == R, "one segment list per request")
    segs, ptr, keep = [], [0], []
    for req in requests:
        for sk, sv, n in req:
            _need(sk.dtype == cache_k.dtype and sv.dtype == cache_k.dtype, "segments must have the cache dtype")
            _need(sk.dim() == 3 and sk.shape[1:] == (hkv, d) and sv.shape == sk.shape, "segment shape")
            _need(sk.stride(2) == 1 and sk.stride(1) == d and sv.stride() == sk.stride(), "segment layout")
            flags = 0
            if staged:
                # copied by the library from host memory: host addresses
                _need(not sk.is_cuda and not sv.is_cuda and sk.is_pinned() and sv.is_pinned(),
                      "staged compose takes pinned (page-locked) CPU segments")
                pk, pv = sk.data_ptr(), sv.data_ptr()
            elif sk.is_cuda and sv.is_cuda:
                pk, pv = sk.data_ptr(), sv.data_ptr()
            else:
                # slot caches kept in host memory: compose reads them in place
                pk, pv = host_device_ptr(sk), host_device_ptr(sv)
                flags = _lib.SEGMENT_HOST
            if not realign:
                flags |= _lib.SEGMENT_NO_REALIGN
            segs.append(Segment(pk, pv, sk.stride(0), int(n), flags))
            keep.append((sk, sv))
        ptr.append(len(segs))
    _need(len(segs) > 0, "no segments")
    return (Segment * len(segs))(*segs), _arr_i32(ptr), keep


class _HostHolds:
    """Pinned host segments of eager compose calls, kept referenced until an
    event recorded after the launch has completed, so that the host
    allocator cannot hand their blocks out while a kernel or copy still
    reads them.  Under graph capture the caller keeps them alive for as
    long as the graph may be replayed."""

    def __init__(self):
        self._held = []

    def hold(self, tensors, device: torch.device) -> None:
        self._held = [(ev, t) for ev, t in self._held if not ev.query()]
        if tensors and not torch.cuda.is_current_stream_capturing():
            ev = torch.cuda.Event()
            ev.record(torch.cuda.current_stream(device))
            self._held.append((ev, tensors))


HOST_HOLDS = _HostHolds()


def _compose_call(fn, requests, ratio_k, rope_theta, cache_k, cache_v, pos_base, pos_out, staged, workspace,
                  realign=True):
    lib = load()
    _dev_tensor(cache_k, "cache_k")
    _dev_tensor(cache_v, "cache_v", cache_k.dtype)
    R, hkv, cap, d = cache_k.shape
    arr, ptr, keep = _segment_table(requests, cache_k, staged, realign)
    lens = (ctypes.c_int32 * R)()
    nxt = (ctypes.c_int32 * R)()
    if pos_out is not None:
        _dev_tensor(pos_out, "pos_out", torch.int32)
        _need(pos_out.shape == (R, cap), "pos_out must be [R][cap]")
    base = _arr_i32(pos_base) if pos_base is not None else None
    dt = _DT[cache_k.dtype]
    ws, nbytes = None, 0
    if staged:
        need = lib.c2kv_workspace_size_compose_staged(arr, len(arr), ratio_k, hkv, d, dt)
        _need(need > 0, "invalid staged compose arguments")
        ws = _workspace(workspace, "compose_staged", need, cache_k.device)
        nbytes = ws.numel()
    check(fn(arr, len(arr), ptr, R, base, ratio_k, hkv, d, float(rope_theta), _ptr(cache_k), _ptr(cache_v), cap,
             _ptr(pos_out), lens, nxt, dt, _ptr(ws), nbytes, _stream(cache_k.device)))
    HOST_HOLDS.hold([t for pair in keep for t in pair if not t.is_cuda], cache_k.device)
    return list(lens), list(nxt)


def compose(requests: Sequence[Sequence[Tuple[torch.Tensor, torch.Tensor, int]]], ratio_k: int,
            rope_theta: float, cache_k: torch.Tensor, cache_v: torch.Tensor,
            pos_base: Optional[Sequence[int]] = None, pos_out: Optional[torch.Tensor] = None,
            realign: bool = True) -> Tuple[List[int], List[int]]:
    """Compose per-request lists of (slot_k, slot_v, doc_len) into
    cache_k/cache_v [R][hkv][cap][d] (c2kv_compose).  A segment's tensors are
    either on the device or pinned CPU tensors (stored caches kept in host
    memory, read in place across the host link).  realign=False is the
    ablation without positional realignment (C2KV_SEGMENT_NO_REALIGN on
    every segment).  Pinned CPU segments stay referenced here until the
    launch has read them; under graph capture the caller keeps them alive
    while the graph may be replayed.  Returns (cache_len per request, next
    position per request)."""
    return _compose_call(load().c2kv_compose, requests, ratio_k, rope_theta, cache_k, cache_v, pos_base, pos_out,
                         False, None, realign)


def compose_staged(requests: Sequence[Sequence[Tuple[torch.Tensor, torch.Tensor, int]]], ratio_k: int,
                   rope_theta: float, cache_k: torch.Tensor, cache_v: torch.Tensor,
                   pos_base: Optional[Sequence[int]] = None, pos_out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, realign: bool = True) -> Tuple[List[int], List[int]]:
    """As compose, for segments in pinned CPU memory that the library first
    copies into a device workspace (c2kv_compose_staged)."""
    return _compose_call(load().c2kv_compose_staged, requests, ratio_k, rope_theta, cache_k, cache_v, pos_base,
                         pos_out, True, workspace, realign)


# ------------------------------------------------ host-resident slot caches

def host_device_ptr(t: torch.Tensor) -> int:
    """Device address of a pinned CPU tensor's first element, checked to
    cover every byte the view spans (c2kv_host_device_ptr).  Segments built
    from such tensors make c2kv_compose read the slot caches where they
    live, across the host link."""
    _need(isinstance(t, torch.Tensor) and t.device.type == "cpu", "host segment must be a CPU tensor")
    _need(t.is_pinned(), "host segment must be in pinned (page-locked) memory")
    _need(t.numel() > 0 and all(st >= 0 for st in t.stride()), "host segment must be non-empty with positive strides")
    span = (sum((sz - 1) * st for sz, st in zip(t.shape, t.stride())) + 1) * t.element_size()
    out = ctypes.c_void_p()
    check(load().c2kv_host_device_ptr(ctypes.c_void_p(t.data_ptr()), span, ctypes.byref(out)))
    return int(out.value)


# ------------------------------------------------ attention over the cache

def _cache_call(fn_name, q, k_new, v_new, cache_k, cache_v, cache_len, q_pos, rope_theta, return_lse, tq,
                workspace=None):
    lib = load()
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (cache_k, "cache_k"), (cache_v, "cache_v")):
        _dev_tensor(t, nm, cache_k.dtype)
    R, hkv, cap, d = cache_k.shape
    hq = q.shape[-2]
    _need(len(cache_len) == R and len(q_pos) == R, "cache_len/q_pos need one entry per request")
    lens = _arr_i32(cache_len)
    pos = _arr_i32(q_pos)
    dt = _DT[cache_k.dtype]
    o = torch.empty_like(q)
    if tq is None:
        _need(q.shape == (R, hq, d) and k_new.shape == (R, hkv, d) and v_new.shape == k_new.shape, "decode shapes")
        lse = torch.empty((R, hq), dtype=torch.float32, device=q.device) if return_lse else None
        nbytes = lib.c2kv_workspace_size_decode(lens, R, hq, hkv, d, dt)
        _need(nbytes > 0, "invalid decode arguments")
        ws = _workspace(workspace, "cache", nbytes, q.device)
        check(lib.c2kv_attn_decode(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cache_k), _ptr(cache_v), cap,
                                   lens, pos, R, hq, hkv, d, float(rope_theta), _ptr(o), _ptr(lse), dt,
                                   _ptr(ws), ws.numel(), _stream(q.device)))
    else:
        _need(q.shape == (R, tq, hq, d) and k_new.shape == (R, tq, hkv, d) and v_new.shape == k_new.shape,
              "prefill shapes")
        lse = torch.empty((R, hq, tq), dtype=torch.float32, device=q.device) if return_lse else None
        nbytes = lib.c2kv_workspace_size_prefill(lens, R, tq, hq, hkv, d, dt)
        _need(nbytes > 0, "invalid prefill arguments")
        ws = _workspace(workspace, "cache", nbytes, q.device)
        check(lib.c2kv_attn_prefill(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cache_k), _ptr(cache_v), cap,
                                    lens, pos, R, tq, hq, hkv, d, float(rope_theta), _ptr(o), _ptr(lse), dt,
                                    _ptr(ws), ws.numel(), _stream(q.device)))
    return o, lse


def attn_prefill(q, k_new, v_new, cache_k, cache_v, cache_len, q_pos0, rope_theta, return_lse=False,
                 workspace=None):
    """Question prefill over composed caches (c2kv_attn_prefill).
    q [R][tq][hq][d], k_new/v_new [R][tq][hkv][d]; appends to the caches."""
    return _cache_call("prefill", q, k_new, v_new, cache_k, cache_v, cache_len, q_pos0, rope_theta,
                       return_lse, q.shape[1], workspace)


def attn_decode(q, k_new, v_new, cache_k, cache_v, cache_len, q_pos, rope_theta, return_lse=False,
                workspace=None):
    """One decode step over composed caches (c2kv_attn_decode).
    q [R][hq][d], k_new/v_new [R][hkv][d]; appends one row per request."""
    return _cache_call("decode", q, k_new, v_new, cache_k, cache_v, cache_len, q_pos, rope_theta,
                       return_lse, None, workspace)


def attn_decode_noalloc(q, k_new, v_new, cache_k, cache_v, cache_len, q_pos, rope_theta, return_lse=False,
                        out=None, lse_out=None):
    """One decode step that allocates no device memory in the library
    (c2kv_attn_decode_noalloc): the split partials live in the library's
    static per-GPU scratch.  With `out` (and `lse_out`) given, nothing is
    allocated here either.  Calls that overlap in time on one GPU race."""
    lib = load()
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (cache_k, "cache_k"), (cache_v, "cache_v")):
        _dev_tensor(t, nm, cache_k.dtype)
    R, hkv, cap, d = cache_k.shape
    hq = q.shape[-2]
    _need(len(cache_len) == R and len(q_pos) == R, "cache_len/q_pos need one entry per request")
    _need(q.shape == (R, hq, d) and k_new.shape == (R, hkv, d) and v_new.shape == k_new.shape, "decode shapes")
    o = out if out is not None else torch.empty_like(q)
    _dev_tensor(o, "out", q.dtype)
    lse = lse_out
    if return_lse and lse is None:
        lse = torch.empty((R, hq), dtype=torch.float32, device=q.device)
    check(lib.c2kv_attn_decode_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cache_k), _ptr(cache_v), cap,
                                       _arr_i32(cache_len), _arr_i32(q_pos), R, hq, hkv, d, float(rope_theta),
                                       _ptr(o), _ptr(lse), _DT[cache_k.dtype], _stream(q.device)))
    return o, lse


# ----------------------------------------------------------------- testing

def mask_cells(doc_lens: Sequence[int], ratio_k: int, sink_len: Optional[int] = None,
               device: Optional[torch.device] = None, anchor: bool = False) -> Tuple[int, int, int, int, int]:
    """GPU count of visible cells (doc->doc, slot->doc, slot->slot), active
    tiles without a visible cell, and active tiles, from the extraction
    kernel's own tile enumeration (c2kv_mask_cells)."""
    lib = load()
    dev = device or torch.device("cuda", torch.cuda.current_device())
    if sink_len is None:
        sink_len = ratio_k
    ws = WORKSPACES.get("mask", lib.c2kv_workspace_size_mask_cells(), dev, zero=False)
    out = (ctypes.c_uint64 * 5)()
    check(lib.c2kv_mask_cells_ex(_arr_i32(doc_lens), len(doc_lens), ratio_k, sink_len,
                                 _lib.EXTRACT_ANCHOR if anchor else 0, out, _ptr(ws), ws.numel(), _stream(dev)))
    return tuple(int(x) for x in out)


TILE_FIELDS = tuple(f for f, _ in _lib.TileEntry._fields_)


def tile_schedule(doc_lens: Sequence[int], ratio_k: int, sink_len: Optional[int] = None, hq: int = 1,
                  hkv: int = 1, anchor: bool = False, device: Optional[torch.device] = None) -> torch.Tensor:
    """The extraction kernel's tile schedule (c2kv_tile_schedule): one row
    per (unit, key tile) pair it computes, columns TILE_FIELDS (doc, kv_head,
    q_head, q_slot, q0, q1, k_slot, key0, nkeys, masked), as an int32 CPU
    tensor in unspecified order."""
    lib = load()
    dev = device or torch.device("cuda", torch.cuda.current_device())
    if sink_len is None:
        sink_len = ratio_k
    ws = WORKSPACES.get("tiles", lib.c2kv_workspace_size_tile_schedule(), dev, zero=False)
    lens = _arr_i32(doc_lens)
    flags = _lib.EXTRACT_ANCHOR if anchor else 0
    count = ctypes.c_int64()
    check(lib.c2kv_tile_schedule(lens, len(doc_lens), ratio_k, sink_len, hq, hkv, flags, None, 0,
                                 ctypes.byref(count), _ptr(ws), ws.numel(), _stream(dev)))
    n = count.value
    nf = len(TILE_FIELDS)
    buf = torch.empty((max(1, n), nf), dtype=torch.int32, device=dev)
    check(lib.c2kv_tile_schedule(lens, len(doc_lens), ratio_k, sink_len, hq, hkv, flags, _ptr(buf), n,
                                 ctypes.byref(count), _ptr(ws), ws.numel(), _stream(dev)))
    _need(count.value == n, "tile schedule changed between calls")
    return buf[:n].cpu()
