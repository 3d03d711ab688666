"""Seeded synthetic workloads shared by the oracle side and the HIP side.

This module holds shapes, seeds and random draws only.  It does none of the
method's arithmetic (no positions, masks, rotations, slot counts or
attention): callers pass every row count they need, computed on their own
side.  Both the CPU oracle and the GPU path read the exact same values.

Seeding: one ``torch.Generator`` on the CPU per (workload, purpose), with
seed = 2026_0000 + 1000 * workload_id + purpose.  Values are drawn N(0, 1)
in fp32 and then rounded (round-to-nearest-even) to the workload's storage
dtype; the oracle upcasts those same stored values.

The shapes follow the models the C2KV explainer page lists in its
limitations section (Qwen3-4B, Llama3.1-8B, Qwen2.5-7B, Qwen3-14B), the
8-document example of its introduction, its 16k-128k decode discussion in
the results section, and compression ratios 4/8/16 from the same page.
No dataset item is used; every tensor is Gaussian noise of that shape.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import torch

# purposes
P_Q, P_K, P_V, P_LENS, P_ORDER, P_DEC_Q, P_NEW_KV, P_PREFILL = 0, 1, 2, 3, 4, 5, 6, 7


def seed_for(workload_id: int, purpose: int, salt: int = 0) -> int:
    return 2026_0000 + 1000 * workload_id + purpose + 100_000_000 * salt


def generator(workload_id: int, purpose: int, salt: int = 0) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(workload_id, purpose, salt))
    return g


def normal(shape: Sequence[int], dtype: torch.dtype, workload_id: int,
           purpose: int, salt: int = 0, scale: float = 1.0) -> torch.Tensor:
    """N(0, scale^2) draws in fp32 rounded once to ``dtype`` (CPU tensor)."""
    g = generator(workload_id, purpose, salt)
    x = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def randint(lo: int, hi_inclusive: int, count: int, workload_id: int,
            purpose: int, salt: int = 0) -> List[int]:
    g = generator(workload_id, purpose, salt)
    return [int(v) for v in torch.randint(lo, hi_inclusive + 1, (count,), generator=g)]


def permutation(n: int, workload_id: int, purpose: int, salt: int = 0) -> List[int]:
    g = generator(workload_id, purpose, salt)
    return [int(v) for v in torch.randperm(n, generator=g)]


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    dtype: torch.dtype
    hq: int
    hkv: int
    head_dim: int
    rope_theta: float
    ratio_k: int
    sink_len: int
    doc_lens: Tuple[int, ...] = ()
    tq: int = 0
    decode_steps: int = 0
    num_reqs: int = 1
    layers: int = 1

    @property
    def dtype_name(self) -> str:
        return "bf16" if self.dtype == torch.bfloat16 else "f32"


TINY = Workload(1, "tiny_fp32", torch.float32, 1, 1, 64, 10000.0, 4, 4,
                doc_lens=(64, 40), tq=8, decode_steps=16)

LLAMA = Workload(2, "llama31_8b_1layer", torch.bfloat16, 32, 8, 128, 500000.0, 4, 4,
                 doc_lens=(4096,) * 8, tq=64, decode_steps=256)

QWEN25 = Workload(3, "qwen25_7b_pool_decode", torch.bfloat16, 28, 4, 128, 1e6, 16, 16,
                  decode_steps=128, num_reqs=32)

LONGCTX = Workload(4, "llama31_8b_longctx_decode", torch.bfloat16, 32, 8, 128, 500000.0, 4, 4,
                   num_reqs=64, layers=32, decode_steps=8)

QWEN3_14B = Workload(5, "qwen3_14b_extract", torch.bfloat16, 40, 8, 128, 1e6, 4, 4,
                     doc_lens=(8192,) * 64, layers=40)

ALL = (TINY, LLAMA, QWEN25, LONGCTX, QWEN3_14B)


def llama_doc_order(w: Workload = LLAMA) -> List[int]:
    """Seeded permutation of the documents (composition order)."""
    return permutation(len(w.doc_lens), w.wid, P_ORDER)


def qwen25_pool(w: Workload = QWEN25, num_docs: int = 64) -> List[int]:
    """Pool document lengths, uniform on {1024, ..., 8192}."""
    return randint(1024, 8192, num_docs, w.wid, P_LENS)


def qwen25_requests(w: Workload = QWEN25, num_docs: int = 64) -> List[List[int]]:
    """Per request: a subset of 8..32 pool documents, drawn without
    replacement, in random order."""
    sizes = randint(8, 32, w.num_reqs, w.wid, P_ORDER, salt=1)
    reqs = []
    for r, s in enumerate(sizes):
        perm = permutation(num_docs, w.wid, P_ORDER, salt=2 + r)
        reqs.append(perm[:s])
    return reqs


def longctx_doc_counts() -> Tuple[int, ...]:
    """Original context 16k/32k/64k/128k built from 4096-token documents."""
    return (4, 8, 16, 32)


def sink_biased(q: torch.Tensor, k: torch.Tensor, sink_rows: int, sigma: float = 3.0) -> torch.Tensor:
    """Variant inputs in which the first ``sink_rows`` keys lean towards the
    mean query direction (attention mass concentrating on the first tokens,
    as the explainer page remarks in its structured-flow section).  Pure data
    shaping: returns a new key tensor of k's dtype."""
    kf = k.float().clone()
    qd = q.float().mean(dim=0)                         # [Hq, d]
    hkv = k.shape[1]
    g = q.shape[1] // hkv
    dirs = qd.reshape(hkv, g, -1).mean(dim=1)          # [Hkv, d]
    dirs = dirs / dirs.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    kf[:sink_rows] += sigma * dirs.unsqueeze(0) * (k.shape[-1] ** 0.5) / 4.0
    return kf.to(k.dtype)


def device_normal(shape: Sequence[int], dtype: torch.dtype, workload_id: int, purpose: int,
                  device: torch.device, salt: int = 0) -> torch.Tensor:
    """Bulk N(0, 1) inputs drawn by torch's device generator (for full-size
    timing runs, where the values do not matter for speed).  Seeded like
    ``normal``; a parity check reads back only the slices it compares."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(workload_id, purpose, salt))
    x = torch.empty(tuple(int(s) for s in shape), dtype=torch.float32, device=device)
    x.normal_(generator=g)
    return x.to(dtype)
