"""Comparison of the HIP forward against the fp64 oracle, row by row.

Selection protocol: a row's chosen blocks must equal the oracle's exactly,
unless the oracle's fp64 gap between the last chosen and the first unchosen
past score is a near tie (below 1e-4 relative, or below twice the fp32 error
bound of a score).  Such rows are counted; the GPU's set must then still be a
valid top-k within that bound, and the row's output is compared with the
oracle evaluated on the GPU's set.
"""
from __future__ import annotations

import dataclasses
import time
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle.moba_oracle as O


class RowSource:
    """Read-only (b, t, h) row access to a host tensor without an fp64 copy of
    all of it; presents the numpy-like surface the oracle uses."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)
        self.ndim = t.ndim

    def __getitem__(self, idx):
        return self.t[idx].to(torch.float64).numpy()


def to_np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy()


@dataclasses.dataclass
class ParityReport:
    rows: int
    near_ties: int
    sel_mismatch_near_tie: int
    max_abs_err: float
    worst_row: Optional[Tuple[int, int, int]]
    oracle_seconds: float

    def as_dict(self):
        return dataclasses.asdict(self)


def compare(q_dev, k_dev, v_dev, out_dev, sel_dev, block_size: int, topk: int, causal: bool,
            rows: Optional[Sequence[Tuple[int, int, int]]] = None, tol: float = 2e-2,
            mu: Optional[np.ndarray] = None, gate: str = "mean") -> ParityReport:
    """Compare GPU out / sel_idx with the oracle on `rows` (all rows if None),
    the oracle scoring blocks with `gate` ("mean" or "minmax").
    Raises AssertionError on any violation."""
    qh = q_dev.detach().cpu()
    k32, v32 = to_np32(k_dev), to_np32(v_dev)
    b, S, Hq, D = qh.shape
    if rows is None:
        rows = [(bb, t, h) for bb in range(b) for h in range(Hq) for t in range(S)]
    rows = list(rows)
    outh = out_dev.detach().cpu().to(torch.float32)
    selh = sel_dev.detach().cpu()
    t0 = time.perf_counter()
    mm = None
    if gate == "minmax":
        mm = O.block_minmax(k32, block_size)
    elif mu is None:
        mu = O.block_means(k32, block_size)
    res = O.moba_rows(RowSource(qh), k32, v32, block_size, topk, causal, rows, mu=mu, keep_scores=True,
                      gate=gate, minmax=mm)
    ties = O.near_tie_rows(res)
    gsel = np.stack([selh[bb, h, t].numpy() for (bb, t, h) in rows])
    mismatch = [r for r in range(len(rows)) if not np.array_equal(gsel[r], res.sel[r])]
    redo: List[int] = []
    for r in mismatch:
        bb, t, h = rows[r]
        if not ties[r]:
            raise AssertionError(f"row {rows[r]}: GPU chose {gsel[r].tolist()}, oracle {res.sel[r].tolist()}, "
                                 f"gap {res.gap[r]:.3e} is not a near tie (eps {res.score_eps[r]:.3e})")
        j = t // block_size
        past = [int(i) for i in gsel[r] if i >= 0 and (not causal or i != j)]
        m = min(topk - 1, j) if causal else min(topk, S // block_size)
        cand_j = j if causal else S // block_size
        if causal and j not in gsel[r].tolist():
            raise AssertionError(f"row {rows[r]}: own block missing from GPU selection {gsel[r].tolist()}")
        if not O.valid_topk_set(res.scores[r], past, cand_j, m, res.score_eps[r]):
            raise AssertionError(f"row {rows[r]}: GPU selection {gsel[r].tolist()} is not a valid top-k")
        redo.append(r)
    ref_out = res.out.copy()
    if redo:
        sub_rows = [rows[r] for r in redo]
        sub = O.moba_rows(RowSource(qh), k32, v32, block_size, topk, causal, sub_rows, mu=mu,
                          given_sel=[gsel[r] for r in redo], gate=gate, minmax=mm)
        for x, r in enumerate(redo):
            ref_out[r] = sub.out[x]
    secs = time.perf_counter() - t0
    gout = np.stack([outh[bb, t, h].numpy() for (bb, t, h) in rows]).astype(np.float64)
    err = np.abs(gout - ref_out).max(axis=1)
    if not np.all(np.isfinite(gout)):
        bad = int(np.argmax(~np.isfinite(gout).all(axis=1)))
        raise AssertionError(f"non-finite GPU output at row {rows[bad]}")
    worst = int(np.argmax(err))
    if err[worst] > tol:
        raise AssertionError(f"max |out - oracle| = {err[worst]:.3e} > {tol} at row {rows[worst]} "
                             f"(sel gpu {gsel[worst].tolist()} oracle {res.sel[worst].tolist()})")
    return ParityReport(len(rows), int(ties.sum()), len(redo), float(err[worst]), rows[worst], secs)


def compare_decode(q_dev, kc_dev, vc_dev, lens, out_dev, sel_dev, block_size: int, topk: int,
                   rows: Optional[Sequence[Tuple[int, int]]] = None, tol: float = 2e-2) -> ParityReport:
    """Decode parity, with the same selection protocol as `compare`: rows
    (b, h) (all if None) must choose the oracle's blocks unless the oracle's
    gap is a near tie; their outputs are compared with the oracle evaluated
    on the GPU's selection then."""
    qh = q_dev.detach().cpu()
    b, Hq, D = qh.shape
    lens = [int(x) for x in lens]
    if rows is None:
        rows = [(bb, h) for bb in range(b) for h in range(Hq)]
    rows = list(rows)
    # the caches stay in their storage dtype on the host; the oracle converts
    # one (sequence, KV head) prefix at a time
    k32 = RowSource(kc_dev.detach().cpu())
    v32 = RowSource(vc_dev.detach().cpu())
    q32 = to_np32(qh)
    outh = out_dev.detach().cpu().to(torch.float32)
    selh = sel_dev.detach().cpu()
    t0 = time.perf_counter()
    res = O.decode_rows(q32, k32, v32, lens, block_size, topk, keep_scores=True, rows=rows)
    ties = O.near_tie_rows(res)
    gsel = np.stack([selh[bb, h].numpy() for (bb, h) in rows])
    redo: List[int] = []
    for r in range(len(rows)):
        if np.array_equal(gsel[r], res.sel[r]):
            continue
        bb, h = rows[r]
        if not ties[r]:
            raise AssertionError(f"row {rows[r]}: GPU chose {gsel[r].tolist()}, oracle {res.sel[r].tolist()}, "
                                 f"gap {res.gap[r]:.3e} is not a near tie (eps {res.score_eps[r]:.3e})")
        j = (lens[bb] - 1) // block_size
        past = [int(i) for i in gsel[r] if 0 <= i != j]
        if j not in gsel[r].tolist():
            raise AssertionError(f"row {rows[r]}: own block missing from GPU selection {gsel[r].tolist()}")
        if not O.valid_topk_set(res.scores[r], past, j, min(topk - 1, j), res.score_eps[r]):
            raise AssertionError(f"row {rows[r]}: GPU selection {gsel[r].tolist()} is not a valid top-k")
        redo.append(r)
    ref_out = res.out.copy()
    if redo:
        sub = O.decode_rows(q32, k32, v32, lens, block_size, topk, rows=[rows[r] for r in redo],
                            given_sel=[gsel[r] for r in redo])
        for x, r in enumerate(redo):
            ref_out[r] = sub.out[x]
    secs = time.perf_counter() - t0
    gout = np.stack([outh[bb, h].numpy() for (bb, h) in rows]).astype(np.float64)
    if not np.all(np.isfinite(gout)):
        raise AssertionError("non-finite GPU decode output")
    err = np.abs(gout - ref_out).max(axis=1)
    worst = int(np.argmax(err))
    if err[worst] > tol:
        raise AssertionError(f"max |out - oracle| = {err[worst]:.3e} > {tol} at row {rows[worst]} "
                             f"(sel gpu {gsel[worst].tolist()} oracle {res.sel[worst].tolist()})")
    return ParityReport(len(rows), int(ties.sum()), len(redo), float(err[worst]), rows[worst], secs)
