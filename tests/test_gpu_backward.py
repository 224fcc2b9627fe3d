"""GPU parity of the MoBA backward (moba_attn_fwd_train + moba_attn_bwd,
through the C ABI) against the fp64 oracle's moba_backward, run with the
GPU's own selection (selection parity is the forward's test).

Tolerance, element by element: |gpu - oracle| <= 2^-7 |oracle| + 0.015
max|oracle| (per gradient tensor).  The bf16 path rounds P and dS to bf16 for
the MFMAs (relative 2^-9 each, errors that add up over the keys or rows of a
sum and so scale with the tensor's largest values), accumulates in fp32 and
rounds each gradient to bf16 once (2^-9 of the element)."""
import concurrent.futures as cf
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_40_amd as M
import moba_workloads as W
import oracle.moba_oracle as O
from parity_utils import to_np32

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, b, S, Hq, Hkv, B, topk, causal=True, seed=17):
    return W.Workload(name, "bf16", b, Hq, Hkv, S, 128, B, topk, causal=causal, seed=seed)


def dout_for(w, device):
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 1000)
    return torch.randn((w.batch, w.seqlen, w.num_q_heads, w.head_dim), generator=gen).to(torch.bfloat16).to(device)


def check(name, got, ref):
    diff = np.abs(got.astype(np.float64) - ref)
    scale = float(np.abs(ref).max())
    allowed = 2.0 ** -7 * np.abs(ref) + 0.015 * scale
    worst = float((diff / np.maximum(allowed, 1e-300)).max())
    say(f"[grad] {name}: max err {float(diff.max()):.3e} ({float(diff.max()) / max(scale, 1e-300):.2%} of "
        f"max |ref| {scale:.3e}), worst error / allowed {worst:.2f}")
    assert scale > 0 and np.all(diff <= allowed), (name, float(diff.max()), scale)


def run(w):
    say(f"[case] backward {w}")
    q, k, v, _ = W.make_inputs(w, device="cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    do = dout_for(w, DEV)
    out, sel, lse = M.moba_attn_fwd_train(q, k, v, w.block_size, w.topk, w.causal)
    dq, dk, dv = M.moba_attn_bwd(q, k, v, out, do, lse, sel, w.block_size, w.topk, w.causal)
    torch.cuda.synchronize()
    rq, rk, rv, rl = O.moba_backward(to_np32(q), to_np32(k), to_np32(v), to_np32(do), w.block_size, w.topk,
                                     w.causal, sel_idx=sel.cpu().numpy())
    lerr = float(np.abs(lse.cpu().numpy().astype(np.float64) - rl).max())
    say(f"[lse] max err {lerr:.3e}")
    # the forward sums the bf16-rounded weights it multiplies V with (each
    # within 2^-9 relative), so its log-sum-exp is within log(1 + 2^-9) of the
    # exact one, plus fp32 rounding
    assert lerr < 2.5e-3
    check("dq", to_np32(dq), rq)
    check("dk", to_np32(dk), rk)
    check("dv", to_np32(dv), rv)


CASES = [
    small("gqa_b128_k3", 1, 1024, 4, 2, 128, 3),
    small("mha_b64_k5", 1, 1024, 2, 2, 64, 5),
    small("b256_k2", 1, 2048, 4, 1, 256, 2),
    small("b192_k3", 1, 1536, 2, 1, 192, 3),
    small("batch2", 2, 512, 2, 2, 128, 3),
    small("topk1_own_only", 1, 512, 4, 2, 128, 1),
    small("dense_topk_ge_n", 1, 512, 2, 1, 64, 9),
    small("noncausal", 1, 512, 2, 2, 128, 3, causal=False),
    small("g8", 1, 1024, 8, 1, 128, 4),
    small("g3", 1, 1024, 6, 2, 128, 4),
    # more than 32 past slots per row (the forward's gate ranks in rounds)
    small("topk40_gqa", 1, 4096, 4, 2, 64, 40),
    small("topk50_noncausal", 1, 4096, 2, 1, 64, 50, causal=False),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_small(w):
    run(w)


def oracle_backward_per_kv_head(q, k, v, do, w, sel):
    """O.moba_backward run per KV head (a head group's gradients depend on
    its own rows and keys only), the groups in threads."""
    g = w.num_q_heads // w.num_kv_heads

    def one(hk):
        hs = slice(hk * g, (hk + 1) * g)
        return hk, O.moba_backward(q[:, :, hs], k[:, :, hk:hk + 1], v[:, :, hk:hk + 1], do[:, :, hs], w.block_size,
                                   w.topk, w.causal, sel_idx=sel[:, hs])

    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    lse = np.zeros((w.batch, w.num_q_heads, w.seqlen))
    with cf.ThreadPoolExecutor(max_workers=min(16, w.num_kv_heads)) as ex:
        for hk, (a, b, c, l) in ex.map(one, range(w.num_kv_heads)):
            dq[:, :, hk * g:(hk + 1) * g] = a
            dk[:, :, hk:hk + 1] = b
            dv[:, :, hk:hk + 1] = c
            lse[:, hk * g:(hk + 1) * g] = l
    return dq, dk, dv, lse


def test_backward_gqa32x8_top12_full():
    """The training configuration's head layout and top-k (32 query / 8 KV
    heads, top-12) at 2K positions in blocks of 128 (16 blocks, so the gate
    ranks 11 of up to 15 past blocks): every element of dq, dk and dv against
    the oracle's full backward with the GPU's selection."""
    w = small("bwd_gqa32x8_2k_top12", 1, 2048, 32, 8, 128, 12, seed=29)
    say(f"[case] backward full {w}")
    q, k, v, _ = W.make_inputs(w, device=DEV)
    do = dout_for(w, DEV)
    out, sel, lse = M.moba_attn_fwd_train(q, k, v, w.block_size, w.topk, w.causal)
    dq, dk, dv = M.moba_attn_bwd(q, k, v, out, do, lse, sel, w.block_size, w.topk, w.causal)
    torch.cuda.synchronize()
    rq, rk, rv, rl = oracle_backward_per_kv_head(to_np32(q), to_np32(k), to_np32(v), to_np32(do), w,
                                                 sel.cpu().numpy())
    assert float(np.abs(lse.cpu().numpy().astype(np.float64) - rl).max()) < 2.5e-3
    check("dq", to_np32(dq), rq)
    check("dk", to_np32(dk), rk)
    check("dv", to_np32(dv), rv)


def test_backward_workload_128k_sampled_dkdv():
    """dk and dv at the backward's benchmark configuration (128K positions,
    32/8 heads, block 4096, top-12) for sampled keys of two KV heads: the last
    eight keys of block 30 (attended by the rows of block 31 that chose block
    30 and by the own-block rows at or after them) and of block 31 (own-block
    rows only), against the oracle's per-key gradients with the GPU's
    selection; each attending row's log-sum-exp and delta come from the
    oracle's full row, computed in threads."""
    from parity_utils import RowSource
    w = W.WORKLOADS["gqa32x8_128k"]
    say(f"[case] backward sampled dk/dv {w}")
    q, k, v, _ = W.make_inputs(w, device=DEV)
    do = dout_for(w, DEV)
    out, sel, lse = M.moba_attn_fwd_train(q, k, v, w.block_size, w.topk, w.causal)
    dq, dk, dv = M.moba_attn_bwd(q, k, v, out, do, lse, sel, w.block_size, w.topk, w.causal)
    torch.cuda.synchronize()
    B, g = w.block_size, w.num_q_heads // w.num_kv_heads
    keys = [(0, i * B + B - 8 + x, hk) for hk in (0, 7) for i in (30, 31) for x in range(8)]
    selh = sel.cpu().numpy()
    qh, kh, vh, doh = RowSource(q.cpu()), RowSource(k.cpu()), RowSource(v.cpu()), RowSource(do.cpu())
    rows = sorted({r for (bb, s_, hk) in keys for r in O.attending_rows(selh, B, w.causal, bb, s_, hk, g)})
    say(f"[bwd sampled] {len(keys)} keys, {len(rows)} attending rows")
    parts = [rows[i::16] for i in range(16)]

    def stats(part):
        return O.backward_row_stats(qh, kh, vh, doh, B, w.causal, part, [selh[r[0], r[2], r[1]] for r in part])

    row_stats = {}
    with cf.ThreadPoolExecutor(max_workers=16) as ex:
        for st in ex.map(stats, parts):
            row_stats.update(st)
    rk, rv = O.backward_dkdv_keys(qh, kh, vh, doh, B, w.causal, keys, selh, row_stats=row_stats)
    got_k = np.stack([to_np32(dk[bb, s_, hk]) for (bb, s_, hk) in keys])
    got_v = np.stack([to_np32(dv[bb, s_, hk]) for (bb, s_, hk) in keys])
    check("dk (sampled keys)", got_k, rk)
    check("dv (sampled keys)", got_v, rv)


def test_backward_workload_128k_sampled_dq():
    """The backward's benchmark configuration (128K positions, 32/8 heads,
    block 4096, top-12): dq of seeded sample rows against the oracle's per-row
    dq, with the oracle's own selection (rows whose GPU selection differs by a
    near tie are counted and skipped); dk and dv are checked on sampled keys
    below and in full at 2K."""
    from parity_utils import RowSource
    w = W.WORKLOADS["gqa32x8_128k"]
    say(f"[case] backward sampled {w}")
    q, k, v, _ = W.make_inputs(w, device=DEV)
    do = dout_for(w, DEV)
    out, sel, lse = M.moba_attn_fwd_train(q, k, v, w.block_size, w.topk, w.causal)
    dq, dk, dv = M.moba_attn_bwd(q, k, v, out, do, lse, sel, w.block_size, w.topk, w.causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    S = w.seqlen
    pos = [0, 4095, 4096, S - 1] + [int(t) for t in rng.integers(0, S, 12)]
    rows = [(0, t, int(h)) for t in pos for h in rng.integers(0, w.num_q_heads, 3)]
    k32, v32 = RowSource(k.cpu()), RowSource(v.cpu())
    qh, doh = RowSource(q.cpu()), RowSource(do.cpu())
    res = O.moba_rows(qh, k32, v32, w.block_size, w.topk, w.causal, rows, keep_scores=True)
    ties = O.near_tie_rows(res)
    selh = sel.cpu().numpy()
    keep = []
    for r, (bb, t, h) in enumerate(rows):
        if np.array_equal(selh[bb, h, t], res.sel[r]):
            keep.append(r)
        else:
            assert ties[r], f"row {rows[r]}: selection differs and is not a near tie"
    say(f"[bwd sampled] {len(keep)} of {len(rows)} rows compared ({len(rows) - len(keep)} near ties skipped)")
    kr = [rows[r] for r in keep]
    rq, rl = O.backward_dq_rows(qh, k32, v32, doh, w.block_size, w.causal, kr, [res.sel[r] for r in keep])
    got = np.stack([to_np32(dq[bb, t, h]) for (bb, t, h) in kr]).astype(np.float64)
    gl = np.array([float(lse[bb, h, t]) for (bb, t, h) in kr])
    check("dq (sampled rows)", got, rq)
    assert float(np.abs(gl - rl).max()) < 2.5e-3
    assert torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()


def test_backward_many_blocks_sampled():
    """The backward beyond 8192 blocks (8320 blocks of 64 keys, 532K
    positions, 2/1 heads, top-3): the dispatch counts its row lists per range
    of 8192 blocks.  dq of sampled rows (the oracle's own selection, near ties
    skipped) and dk, dv of sampled keys (the last eight of blocks 100 and 8300,
    the GPU's selection, the attending rows' statistics from the oracle)."""
    from parity_utils import RowSource
    w = small("bwd_n8320", 1, 8320 * 64, 2, 1, 64, 3, seed=87)
    say(f"[case] backward many blocks {w}")
    q, k, v, _ = W.make_inputs(w, device=DEV)
    do = dout_for(w, DEV)
    out, sel, lse = M.moba_attn_fwd_train(q, k, v, w.block_size, w.topk, w.causal)
    dq, dk, dv = M.moba_attn_bwd(q, k, v, out, do, lse, sel, w.block_size, w.topk, w.causal)
    torch.cuda.synchronize()
    B, g = w.block_size, w.num_q_heads // w.num_kv_heads
    qh, kh, vh, doh = RowSource(q.cpu()), RowSource(k.cpu()), RowSource(v.cpu()), RowSource(do.cpu())
    selh = sel.cpu().numpy()
    rng = np.random.default_rng(88)
    pos = [0, B, 8192 * B - 1, 8192 * B, w.seqlen - 1] + [int(t) for t in rng.integers(0, w.seqlen, 11)]
    rows = [(0, t, h) for t in pos for h in range(w.num_q_heads)]
    res = O.moba_rows(qh, kh, vh, B, w.topk, w.causal, rows, keep_scores=True)
    ties = O.near_tie_rows(res)
    keep = []
    for r, (bb, t, h) in enumerate(rows):
        if np.array_equal(selh[bb, h, t], res.sel[r]):
            keep.append(r)
        else:
            assert ties[r], f"row {rows[r]}: selection differs and is not a near tie"
    kr = [rows[r] for r in keep]
    rq, _ = O.backward_dq_rows(qh, kh, vh, doh, B, w.causal, kr, [res.sel[r] for r in keep])
    check("dq (sampled rows)", np.stack([to_np32(dq[bb, t, h]) for (bb, t, h) in kr]).astype(np.float64), rq)
    keys = [(0, i * B + B - 8 + x, 0) for i in (100, 8300) for x in range(8)]
    arows = sorted({r for (bb, s_, hk) in keys for r in O.attending_rows(selh, B, w.causal, bb, s_, hk, g)})
    say(f"[bwd many blocks] {len(kr)} dq rows, {len(keys)} keys, {len(arows)} attending rows")
    row_stats = O.backward_row_stats(qh, kh, vh, doh, B, w.causal, arows, [selh[r[0], r[2], r[1]] for r in arows])
    rk, rv = O.backward_dkdv_keys(qh, kh, vh, doh, B, w.causal, keys, selh, row_stats=row_stats)
    check("dk (sampled keys)", np.stack([to_np32(dk[bb, s_, hk]) for (bb, s_, hk) in keys]), rk)
    check("dv (sampled keys)", np.stack([to_np32(dv[bb, s_, hk]) for (bb, s_, hk) in keys]), rv)
