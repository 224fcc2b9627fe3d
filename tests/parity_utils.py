"""Comparison of the HIP forward against the fp64 oracle, row by row.

Selection protocol (the gate check): a row's chosen blocks must equal the
oracle's exactly, unless the oracle's fp64 gap between the last chosen and the
first unchosen candidate score is a near tie, i.e. at most 1e-4 of the larger
of the two scores' magnitudes.  A differing row that is a near tie is counted;
the GPU's set must then still be a valid top-k within that same 1e-4 relative
tolerance, and the row's output is compared with the oracle evaluated on the
GPU's set.  Any other difference fails.

The report counts near-tie rows (whatever the GPU chose) and, separately, the
rows where the GPU's selection differs from the oracle's.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
import time
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle.moba_oracle as O

REL_TIE = 1e-4


class RowSource:
    """Read-only (b, t, h) row access to a host tensor without an fp64 copy of
    all of it; presents the numpy-like surface the oracle uses."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)
        self.ndim = t.ndim

    def __getitem__(self, idx):
        return self.t[idx].to(torch.float64).numpy()


class GatheredRows:
    """Rows (b, t, h) of a [b, S, H, D] tensor gathered on the device, with
    the shape of the whole tensor: the oracle reads q one row at a time."""

    def __init__(self, shape, rows: Sequence[Tuple[int, int, int]], data: np.ndarray):
        self.shape = tuple(shape)
        self.ndim = len(self.shape)
        self.index: Dict[Tuple[int, int, int], np.ndarray] = {r: data[i] for i, r in enumerate(rows)}

    def __getitem__(self, idx):
        return self.index[tuple(int(x) for x in idx)]


def to_np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy()


def gather_rows(x_dev: torch.Tensor, rows: Sequence[Tuple[int, int, int]], layout: str = "bthd") -> np.ndarray:
    """x[b, t, h] (layout "bthd") or x[b, h, t] (layout "bhtd") for each row,
    gathered on the device and copied to the host."""
    idx = torch.tensor(rows, dtype=torch.long, device=x_dev.device)
    b, t, h = idx[:, 0], idx[:, 1], idx[:, 2]
    g = x_dev[b, t, h] if layout == "bthd" else x_dev[b, h, t]
    return g.detach().cpu()


@dataclasses.dataclass
class ParityReport:
    rows: int
    near_ties: int              # rows whose fp64 gap is a near tie (1e-4 relative)
    sel_mismatch: int           # rows where the GPU's selection differs from the oracle's
    max_abs_err: float
    worst_row: Optional[Tuple[int, int, int]]
    oracle_seconds: float

    def as_dict(self):
        return dataclasses.asdict(self)


def _oracle_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_rows(q, k32: np.ndarray, v32: np.ndarray, block_size: int, topk: int, causal: bool,
                rows: Sequence[Tuple[int, int, int]], mu=None, gate: str = "mean", minmax=None,
                given_sel: Optional[Sequence[Sequence[int]]] = None, threads: Optional[int] = None
                ) -> O.RowResult:
    """O.moba_rows on `rows`, run per (batch, KV head) on that head's fp64
    K and V (converted once) and split over threads.  The per-row arithmetic
    is the oracle's own; this only decides which rows each call gets."""
    b, S, Hq, D = q.shape
    Hkv = k32.shape[2]
    g = Hq // Hkv
    rows = list(rows)
    res = O.RowResult(len(rows), D, topk)
    groups: Dict[Tuple[int, int], List[int]] = {}
    for r, (bb, t, h) in enumerate(rows):
        groups.setdefault((bb, h // g), []).append(r)
    nthr = threads or _oracle_threads()
    for (bb, hk), idx in sorted(groups.items()):
        kh = np.ascontiguousarray(k32[bb:bb + 1, :, hk:hk + 1, :], dtype=np.float64)
        vh = np.ascontiguousarray(v32[bb:bb + 1, :, hk:hk + 1, :], dtype=np.float64)
        muh = mu[bb:bb + 1, hk:hk + 1] if mu is not None else None
        mmh = (minmax[0][bb:bb + 1, hk:hk + 1], minmax[1][bb:bb + 1, hk:hk + 1]) if minmax is not None else None

        class _QView:  # rows of this (batch, KV head) group, renumbered to one KV head
            shape = (1, S, g, D)
            ndim = 4

            def __getitem__(self, i, _bb=bb, _hk=hk):
                _, t, hl = i
                return q[_bb, t, _hk * g + hl]

        qv = _QView()
        parts = [idx[i::nthr] for i in range(min(nthr, len(idx)))]

        def work(part):
            sub_rows = [(0, rows[r][1], rows[r][2] - hk * g) for r in part]
            sub_sel = [given_sel[r] for r in part] if given_sel is not None else None
            return part, O.moba_rows(qv, kh, vh, block_size, topk, causal, sub_rows, mu=muh, given_sel=sub_sel,
                                     keep_scores=True, gate=gate, minmax=mmh)

        with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
            for part, sub in ex.map(work, parts):
                for x, r in enumerate(part):
                    res.out[r] = sub.out[x]
                    res.sel[r] = sub.sel[x]
                    res.gap[r] = sub.gap[x]
                    res.boundary[r] = sub.boundary[x]
                    res.score_eps[r] = sub.score_eps[x]
                    res.scores[r] = sub.scores[x]
    return res


def check_selection(rows, gsel: np.ndarray, res: O.RowResult, block_size: int, topk: int, causal: bool,
                    n_blocks: int, own_of=None) -> Tuple[np.ndarray, List[int]]:
    """Apply the selection protocol.  Returns (near-tie mask, indices of rows
    whose GPU selection differs; each of them is a near tie with a valid
    GPU set).  own_of(r) gives row r's own block (causal)."""
    ties = O.near_tie_rows(res, rel=REL_TIE)
    scale = O.near_tie_scale(res)
    differ: List[int] = []
    for r in range(len(rows)):
        if np.array_equal(gsel[r], res.sel[r]):
            continue
        if not ties[r]:
            raise AssertionError(f"row {rows[r]}: GPU chose {gsel[r].tolist()}, oracle {res.sel[r].tolist()}, "
                                 f"fp64 gap {res.gap[r]:.3e} is not a near tie (scores {res.boundary[r].tolist()})")
        j = own_of(r)
        past = [int(i) for i in gsel[r] if i >= 0 and (not causal or i != j)]
        m = min(topk - 1, j) if causal else min(topk, n_blocks)
        cand = j if causal else n_blocks
        if causal and j not in gsel[r].tolist():
            raise AssertionError(f"row {rows[r]}: own block missing from GPU selection {gsel[r].tolist()}")
        if not O.valid_topk_set(res.scores[r], past, cand, m, REL_TIE * scale[r]):
            raise AssertionError(f"row {rows[r]}: GPU selection {gsel[r].tolist()} is not a valid top-k")
        differ.append(r)
    return ties, differ


def compare(q_dev, k_dev, v_dev, out_dev, sel_dev, block_size: int, topk: int, causal: bool,
            rows: Optional[Sequence[Tuple[int, int, int]]] = None, tol: float = 2e-2,
            mu: Optional[np.ndarray] = None, gate: str = "mean") -> ParityReport:
    """Compare GPU out / sel_idx with the oracle on `rows` (all rows if None),
    the oracle scoring blocks with `gate` ("mean" or "minmax").
    Raises AssertionError on any violation."""
    b, S, Hq, D = q_dev.shape
    if rows is None:
        rows = [(bb, t, h) for bb in range(b) for h in range(Hq) for t in range(S)]
    rows = [tuple(int(x) for x in r) for r in rows]
    qg = GatheredRows(q_dev.shape, rows, gather_rows(q_dev, rows).to(torch.float64).numpy())
    gout = gather_rows(out_dev, rows).to(torch.float64).numpy()
    gsel = gather_rows(sel_dev, rows, layout="bhtd").numpy()
    k32, v32 = to_np32(k_dev), to_np32(v_dev)
    t0 = time.perf_counter()
    mm = None
    if gate == "minmax":
        mm = O.block_minmax(k32, block_size)
    elif mu is None:
        mu = O.block_means(k32, block_size)
    res = oracle_rows(qg, k32, v32, block_size, topk, causal, rows, mu=mu, gate=gate, minmax=mm)
    n_blocks = S // block_size
    ties, redo = check_selection(rows, gsel, res, block_size, topk, causal, n_blocks,
                                 own_of=lambda r: rows[r][1] // block_size)
    ref_out = res.out.copy()
    if redo:
        sub_rows = [rows[r] for r in redo]
        sub = oracle_rows(qg, k32, v32, block_size, topk, causal, sub_rows, mu=mu, gate=gate, minmax=mm,
                          given_sel=[gsel[r] for r in redo])
        for x, r in enumerate(redo):
            ref_out[r] = sub.out[x]
    secs = time.perf_counter() - t0
    if not np.all(np.isfinite(gout)):
        bad = int(np.argmax(~np.isfinite(gout).all(axis=1)))
        raise AssertionError(f"non-finite GPU output at row {rows[bad]}")
    err = np.abs(gout - ref_out).max(axis=1)
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
    gsel = np.stack([selh[bb, h].numpy() for (bb, h) in rows])
    ties, redo = check_selection(rows, gsel, res, block_size, topk, True, 0,
                                 own_of=lambda r: (lens[rows[r][0]] - 1) // block_size)
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
