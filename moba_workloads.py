"""Seeded synthetic workloads for the MoBA prefill forward.

This module only draws inputs.  It holds none of the method's arithmetic (no
block means, scores, selection or attention), so both the fp64 oracle and the
HIP path can take their inputs from it without sharing any computation.

Shapes follow the workloads described for MoBA in "MoBA: Mixture of Block
Attention for Long-Context LLMs" as summarised by the deep-dive report page
(section 3.3, training recipes): block 512 / top-3 at 8K and 32K, and the
Llama-3.1-8B-shaped grouped-query layout (32 query heads, 8 KV heads, head
dim 128) with block 4096 / top-12 at 128K and 1M.  No dataset is used: every
tensor is N(0, 1) noise from a seeded torch generator, rounded to the storage
dtype with torch's round-to-nearest-even cast.

The 32K workload carries planted "needles": a few key blocks and one eighth of
the queries are shifted by +0.5 along a per-head random unit direction, so
that the gate has a real signal to find (the course page on MoBA uses a seeded
needle to probe block granularity).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seqlen: int
    head_dim: int
    block_size: int
    topk: int
    causal: bool = True
    needles: int = 0      # number of needle key blocks (0 = pure iid)
    needle_shift: float = 0.5
    needle_query_frac: float = 0.125
    seed: int = 0

    @property
    def num_blocks(self) -> int:
        return self.seqlen // self.block_size

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, smallest first.
WORKLOADS = {
    "tiny_f32_1k": Workload("tiny_f32_1k", "f32", 1, 1, 1, 1024, 64, 128, 3, seed=1001),
    "mha16_8k": Workload("mha16_8k", "bf16", 1, 16, 16, 8192, 128, 512, 3, seed=1002),
    "mha32_32k_needle": Workload("mha32_32k_needle", "bf16", 1, 32, 32, 32768, 128, 512, 3,
                                 needles=8, seed=1003),
    "gqa32x8_128k": Workload("gqa32x8_128k", "bf16", 1, 32, 8, 131072, 128, 4096, 12, seed=1004),
    "gqa32x8_1m": Workload("gqa32x8_1m", "bf16", 1, 32, 8, 1048576, 128, 4096, 12, seed=1005),
}


def _randn_chunked(shape, gen, device, dtype, chunk_rows: int = 1 << 16) -> torch.Tensor:
    """N(0,1) fp32 draws cast to `dtype`, produced in chunks along dim 1 so the
    fp32 staging buffer stays small for the 1M workload.  The chunking is part
    of the recipe (it fixes which draw lands where)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    S = shape[1]
    for s0 in range(0, S, chunk_rows):
        s1 = min(S, s0 + chunk_rows)
        sub = list(shape)
        sub[1] = s1 - s0
        out[:, s0:s1] = torch.randn(sub, generator=gen, device=device, dtype=torch.float32).to(dtype)
    return out


@dataclasses.dataclass
class Needles:
    blocks: torch.Tensor      # [needles] int64, key blocks that carry the shift
    queries: torch.Tensor     # [nq] int64, query positions that carry the shift
    directions: torch.Tensor  # [num_kv_heads, head_dim] fp32 unit vectors


def make_inputs(w: Workload, device: str = "cpu", seed: Optional[int] = None):
    """Return (q, k, v, needles) for workload `w`.

    Layout is BSHD contiguous: q [batch, seqlen, num_q_heads, head_dim],
    k and v [batch, seqlen, num_kv_heads, head_dim], dtype per workload.
    `needles` is None for iid workloads.
    """
    seed = w.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = w.torch_dtype
    b, S, Hq, Hkv, D = w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim
    q = _randn_chunked((b, S, Hq, D), gen, device, dt)
    k = _randn_chunked((b, S, Hkv, D), gen, device, dt)
    v = _randn_chunked((b, S, Hkv, D), gen, device, dt)
    needles = None
    if w.needles:
        n = w.num_blocks
        # distinct needle blocks in [1, n-1], the same for every head
        perm = torch.randperm(n - 1, generator=gen, device=device)[: w.needles] + 1
        blocks = torch.sort(perm).values
        nq = max(1, int(round(S * w.needle_query_frac)))
        qpos = torch.sort(torch.randperm(S, generator=gen, device=device)[:nq]).values
        u = torch.randn((Hkv, D), generator=gen, device=device, dtype=torch.float32)
        u = u / u.norm(dim=1, keepdim=True)
        shift = (w.needle_shift * u)  # [Hkv, D]
        B = w.block_size
        for i in blocks.tolist():
            seg = k[:, i * B:(i + 1) * B].to(torch.float32) + shift
            k[:, i * B:(i + 1) * B] = seg.to(dt)
        g = Hq // Hkv
        qshift = shift.repeat_interleave(g, dim=0)  # query head h uses KV head h // g
        qsel = q[:, qpos].to(torch.float32) + qshift
        q[:, qpos] = qsel.to(dt)
        needles = Needles(blocks.cpu(), qpos.cpu(), u.cpu())
    return q, k, v, needles


def sample_rows(w: Workload, per_head: int, seed: int, extra_positions=()):
    """Seeded sample of query rows (batch, position, head) for checking the big
    workloads row by row: `per_head` distinct positions per head (or all of
    the fixed ones, if more).  Always includes the first and last query, the
    first and last query of the first block, the first query after the warm-up
    blocks (where the gate first has to choose) and `extra_positions`, plus
    uniform draws."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    S, B, H = w.seqlen, w.block_size, w.num_q_heads
    fixed = [0, B - 1, min(B, S - 1), min((w.topk - 1) * B, S - 1), min(w.topk * B + B // 2, S - 1), S - 1]
    fixed = set(fixed + [int(p) for p in extra_positions])
    want = min(S, max(per_head, len(fixed)))
    rows = []
    for b in range(w.batch):
        for h in range(H):
            pos = set(fixed)
            # uniform draws until the head has `want` distinct positions
            while len(pos) < want:
                pos.update(torch.randint(0, S, (want - len(pos),), generator=gen).tolist())
            for t in sorted(pos):
                rows.append((b, t, h))
    return rows


def describe(w: Workload) -> dict:
    return {
        "workload": w.name, "dtype": w.dtype, "batch": w.batch, "seqlen": w.seqlen,
        "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
        "block_size": w.block_size, "topk": w.topk, "causal": w.causal,
        "needle_blocks": w.needles,
    }


# ---------------------------------------------------------------------------
# Decode: one new query per sequence against a cache of L_b positions
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    dtype: str  # "bf16" | "f32"
    num_q_heads: int
    num_kv_heads: int
    max_len: int
    head_dim: int
    block_size: int
    topk: int
    lens: tuple  # cached positions per sequence (the new token included)
    seed: int = 0

    @property
    def batch(self) -> int:
        return len(self.lens)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def _ragged_1m_lens():
    # eight sequences a little below 1M positions, at different points of
    # their last block (one exactly at a block boundary, one just past one)
    M = 1 << 20
    return (M, M - 1, M - 4095, M - 4096, M - 4097, M - 70001, M - 123457, M - 262143)


DECODE_WORKLOADS = {
    # the prefill 1M layout (32/8 heads, D 128, block 4096, top-12) at decode
    "decode_gqa32x8_1m_b8": DecodeWorkload("decode_gqa32x8_1m_b8", "bf16", 32, 8, 1 << 20, 128, 4096, 12,
                                           _ragged_1m_lens(), seed=2001),
}


def make_decode_inputs(w: DecodeWorkload, device: str = "cpu", seed: Optional[int] = None):
    """Return (q [b, Hq, D], k_cache, v_cache [b, max_len, Hkv, D], lens int32
    [b]): seeded N(0, 1) noise rounded to the storage dtype.  Cache entries at
    positions >= L_b hold noise too (a decode must never read them)."""
    seed = w.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = w.torch_dtype
    b, Hq, Hkv, D, Lm = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_len
    q = _randn_chunked((b, Hq, D), gen, device, dt)
    k = _randn_chunked((b, Lm, Hkv, D), gen, device, dt)
    v = _randn_chunked((b, Lm, Hkv, D), gen, device, dt)
    lens = torch.tensor(list(w.lens), dtype=torch.int32, device=device)
    return q, k, v, lens
