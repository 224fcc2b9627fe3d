"""GPU parity of the HIP MoBA forward (through the C ABI) against the fp64 oracle.

Tolerances: out within max-abs 2e-2 for bf16 and 1e-4 for fp32; block
selection exact except counted near ties (see parity_utils).  Block means are
compared with a bound derived from fp32 summation (Higham's gamma_{B+2} times
the mean absolute key)."""
import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_40_amd as M
import moba_workloads as W
import oracle.moba_oracle as O
from parity_utils import compare, to_np32

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, dtype, b, S, Hq, Hkv, D, B, topk, causal=True, seed=7):
    return W.Workload(name, dtype, b, Hq, Hkv, S, D, B, topk, causal=causal, seed=seed)


def run(w: W.Workload, rows=None, device_inputs=False, gate="mean"):
    say(f"[case] {w} gate={gate}")
    q, k, v, _ = W.make_inputs(w, device=DEV if device_inputs else "cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    out, sel = M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, gate=gate)
    torch.cuda.synchronize()
    rep = compare(q, k, v, out, sel, w.block_size, w.topk, w.causal, rows=rows, tol=TOL[w.dtype], gate=gate)
    say(f"[parity] {w.name}: {rep.as_dict()}")
    return rep, (q, k, v, out, sel)


# ----------------------------------------------------------------------------
# stage parity
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,b,S,Hkv,D,B", [
    ("bf16", 1, 2048, 2, 128, 256), ("bf16", 2, 1536, 3, 128, 96), ("f32", 1, 1024, 1, 64, 128),
    ("f32", 1, 512, 2, 128, 16), ("bf16", 1, 8192, 16, 128, 512),
])
def test_meanpool_matches_oracle(dtype, b, S, Hkv, D, B):
    w = small("mp", dtype, b, S, Hkv, Hkv, D, B, 1, seed=3)
    say(f"[case] meanpool {w}")
    _, k, _, _ = W.make_inputs(w, device="cpu")
    mu = M.moba_meanpool(k.to(DEV), B)
    torch.cuda.synchronize()
    k32 = to_np32(k)
    ref = O.block_means(k32, B)
    absmean = np.abs(k32.astype(np.float64)).reshape(b, S // B, B, Hkv, D).mean(axis=2).transpose(0, 2, 1, 3)
    u = 2.0 ** -24
    gam = (B + 2) * u / (1 - (B + 2) * u)
    err = np.abs(mu.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= gam * absmean + 1e-30), float((err - gam * absmean).max())


@pytest.mark.parametrize("dtype,b,S,Hkv,D,B", [
    ("bf16", 1, 2048, 2, 128, 256), ("bf16", 2, 1536, 3, 128, 96), ("f32", 1, 1024, 1, 64, 128),
    ("f32", 1, 512, 2, 128, 16), ("bf16", 1, 8192, 8, 128, 1024),
])
def test_minmaxpool_matches_oracle(dtype, b, S, Hkv, D, B):
    """Element-wise block min / max: input values, so bit-exact."""
    w = small("mm", dtype, b, S, Hkv, Hkv, D, B, 1, seed=5)
    say(f"[case] minmaxpool {w}")
    _, k, _, _ = W.make_inputs(w, device="cpu")
    lohi = M.moba_minmaxpool(k.to(DEV), B)
    torch.cuda.synchronize()
    lo, hi = O.block_minmax(to_np32(k), B)
    got = lohi.cpu().numpy().astype(np.float64)
    assert np.array_equal(got[:, :, :, 0], lo)
    assert np.array_equal(got[:, :, :, 1], hi)


@pytest.mark.parametrize("dtype,S,Hq,Hkv,D,B,topk,causal", [
    ("bf16", 2048, 4, 2, 128, 128, 3, True), ("bf16", 4096, 8, 1, 128, 64, 9, True),
    ("bf16", 2048, 2, 2, 128, 128, 20, True), ("bf16", 1024, 2, 1, 128, 64, 5, False),
    ("f32", 1024, 1, 1, 64, 128, 3, True), ("bf16", 4096, 2, 2, 128, 32, 33, True),
    # more than 32 past blocks to rank: the cut-off score found in rounds
    ("bf16", 4096, 2, 2, 128, 32, 60, True), ("f32", 2048, 2, 1, 64, 16, 90, False),
])
def test_gate_matches_oracle(dtype, S, Hq, Hkv, D, B, topk, causal):
    w = small("gate", dtype, 1, S, Hq, Hkv, D, B, topk, causal, seed=11)
    say(f"[case] gate {w}")
    q, k, v, _ = W.make_inputs(w, device="cpu")
    mu = M.moba_meanpool(k.to(DEV), B)
    sel = M.moba_gate(q.to(DEV), mu, B, topk, causal)
    torch.cuda.synchronize()
    k32 = to_np32(k)
    ref_mu = O.block_means(k32, B)
    from parity_utils import RowSource
    rows = [(0, t, h) for h in range(Hq) for t in range(S)]
    res = O.moba_rows(RowSource(q), k32, to_np32(v), B, topk, causal, rows, mu=ref_mu, keep_scores=True)
    ties = O.near_tie_rows(res)
    selh = sel.cpu()
    bad = 0
    for r, (bb, t, h) in enumerate(rows):
        g = selh[bb, h, t].numpy()
        if not np.array_equal(g, res.sel[r]):
            assert ties[r], f"row {(bb, t, h)}: gpu {g.tolist()} oracle {res.sel[r].tolist()} gap {res.gap[r]}"
            bad += 1
    say(f"[gate] near ties {int(ties.sum())}, differing near-tie rows {bad}")


# ----------------------------------------------------------------------------
# whole forward, small shapes spanning several tiles and ragged tails
# ----------------------------------------------------------------------------
SMALL = [
    small("gqa_s2k", "bf16", 1, 2048, 4, 2, 128, 256, 3),
    small("mha_b128", "bf16", 1, 1536, 2, 2, 128, 128, 4),
    small("ragged_b96", "bf16", 1, 960, 2, 1, 128, 96, 3),
    small("b64_g8", "bf16", 1, 4096, 8, 1, 128, 64, 5),
    small("batch2", "bf16", 2, 1024, 2, 2, 128, 128, 3),
    small("topk1", "bf16", 1, 1024, 2, 2, 128, 128, 1),
    small("dense_eq", "bf16", 1, 1024, 2, 1, 128, 128, 8),
    small("dense_clamp", "bf16", 1, 1024, 2, 1, 128, 128, 20),
    small("noncausal", "bf16", 1, 1024, 2, 2, 128, 128, 3, causal=False),
    small("b16_tiny_blocks", "bf16", 1, 512, 2, 2, 128, 16, 4),
    small("b2048_long", "bf16", 1, 8192, 4, 1, 128, 2048, 2),
    small("single_block", "bf16", 1, 256, 2, 2, 128, 256, 3),
    # groups that do not divide the 256-row own-block tiles (g = 3: 85 positions x 3
    # heads) and a group of 32 (8 positions x 32 heads per tile)
    small("gqa_g3", "bf16", 1, 2048, 6, 2, 128, 128, 4),
    small("gqa_g32", "bf16", 1, 1024, 32, 1, 128, 128, 3),
    # lists of 2304 rows on average: 256-row tiles over blocks that are not a
    # whole number of 64-key slices (direct K/V staging, masked last slice)
    small("ragged_b96_long_lists", "bf16", 1, 3840, 8, 1, 128, 96, 4),
    # bf16 gate on MFMA: several 32-block score tiles with a ragged last one,
    # and each top-k list capacity (kept past blocks 8, 11, 15, 19)
    small("gate_n50_k9", "bf16", 1, 2400, 4, 2, 128, 48, 9),
    small("gate_n96_k12", "bf16", 1, 6144, 4, 1, 128, 64, 12),
    small("gate_n64_k16", "bf16", 1, 4096, 4, 1, 128, 64, 16),
    small("gate_n64_k20", "bf16", 1, 4096, 2, 2, 128, 64, 20),
    small("gate_noncausal_n40", "bf16", 1, 2560, 2, 1, 128, 64, 6, causal=False),
    # blocks of five 32-key slices (not whole 64-key slices) and g = 3: the
    # direct-load row kernels' three-buffer pipeline over an odd slice count,
    # 42-position own tiles with a masked last slice
    small("rows_b160_g3", "bf16", 1, 1920, 6, 2, 128, 160, 4),
    small("f32_d128_gqa", "f32", 1, 1024, 4, 2, 128, 128, 3),
    small("f32_noncausal", "f32", 1, 512, 2, 1, 64, 64, 3, causal=False),
    # more than 32 past blocks to rank (the gate's rounds): 2 and 4 rounds on
    # the MFMA gate, non-causal, and the fp32 VALU gate
    small("topk50_rounds", "bf16", 1, 8192, 4, 2, 128, 64, 50),
    small("topk100_rounds_b32", "bf16", 1, 8192, 2, 1, 128, 32, 100),
    small("noncausal_topk70", "bf16", 1, 4096, 2, 2, 128, 32, 70, causal=False),
    small("f32_topk40_rounds", "f32", 1, 2048, 2, 1, 64, 32, 40),
]


GRAPH_CASES = [
    small("graph_small_tiles", "bf16", 1, 2048, 4, 2, 128, 256, 3, seed=31),
    # 384-row tiles: the K/V slice images are built inside the captured call
    small("graph_images", "bf16", 1, 8192, 4, 1, 128, 2048, 2, seed=32),
]


@pytest.mark.parametrize("w", GRAPH_CASES, ids=[w.name for w in GRAPH_CASES])
def test_forward_graph_replay_matches_eager(w):
    """One forward captured into a HIP graph (torch.cuda.CUDAGraph) and
    replayed three times, with eager forwards on other inputs and host
    synchronisations between the replays: every replay's output and selection
    equal the eager ones bit for bit (the library only launches kernels: no
    allocation, copy, memset or synchronisation inside a call)."""
    say(f"[case] graph replay {w}")
    q, k, v, _ = W.make_inputs(w, device=DEV)
    dt = M.DTYPE_BF16
    ws = torch.empty(M.workspace_bytes(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt,
                                       w.block_size, w.topk, w.causal), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    sel = torch.empty((w.batch, w.num_q_heads, w.seqlen, w.topk), dtype=torch.int32, device=DEV)
    M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws)
    torch.cuda.synchronize()
    out_ref, sel_ref = out.clone(), sel.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, out=out, sel_idx=sel, workspace=ws)
    gen = torch.Generator(device="cpu").manual_seed(77)
    for i in range(3):
        # eager work between the replays, on other inputs and buffers
        q2 = torch.randn(q.shape, generator=gen).to(q.dtype).to(DEV)
        o2, _ = M.moba_attn_fwd(q2, k, v, w.block_size, w.topk, w.causal)
        torch.cuda.synchronize()
        out.zero_()
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), f"replay {i}: output differs from the eager forward"
        assert torch.equal(sel, sel_ref), f"replay {i}: selection differs from the eager forward"
        del o2
    del g


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_forward_small(w):
    run(w)


# min/max gate: the bf16 MFMA gate over several score tiles (ragged last
# tile, each list capacity), non-causal, batch 2, and the fp32 VALU gate
SMALL_MINMAX = [
    small("mm_gqa_s2k", "bf16", 1, 2048, 4, 2, 128, 256, 3),
    small("mm_n50_k9", "bf16", 1, 2400, 4, 2, 128, 48, 9),
    small("mm_n96_k12", "bf16", 1, 6144, 4, 1, 128, 64, 12),
    small("mm_n64_k20", "bf16", 1, 4096, 2, 2, 128, 64, 20),
    small("mm_topk2_b16", "bf16", 1, 512, 2, 2, 128, 16, 2),
    small("mm_batch2", "bf16", 2, 1024, 2, 2, 128, 128, 3),
    small("mm_noncausal_n40", "bf16", 1, 2560, 2, 1, 128, 64, 6, causal=False),
    small("mm_f32_d128_gqa", "f32", 1, 1024, 4, 2, 128, 128, 3),
    small("mm_f32_d64_k20", "f32", 1, 2048, 2, 1, 64, 32, 20),
    small("mm_f32_noncausal", "f32", 1, 512, 2, 1, 64, 64, 3, causal=False),
    small("mm_topk45_rounds", "bf16", 1, 4096, 2, 1, 128, 32, 45),
    small("mm_f32_topk36_rounds", "f32", 1, 2048, 2, 1, 64, 32, 36),
]


@pytest.mark.parametrize("w", SMALL_MINMAX, ids=[w.name for w in SMALL_MINMAX])
def test_forward_minmax_small(w):
    run(w, gate="minmax")


TIE_CASES = [(dtype, topk, gate) for dtype in ("bf16", "f32") for topk in (2, 3, 5, 9, 13, 20, 50)
             for gate in ("mean", "minmax")]


@pytest.mark.parametrize("dtype,topk,gate", TIE_CASES)
def test_forward_exact_ties_go_to_lower_index(dtype, topk, gate):
    """Key blocks repeat with period 4 (block i is a copy of block i % 4), so
    a row's block scores take four values and most rows have exact ties at
    the cut-off: equal blocks get bit-identical summaries and scores on both
    sides, and the report's tie rule (section 2.3: the lower block index
    wins) fixes the selection.  Every row whose oracle gap is exactly 0 must
    match the oracle's selection; only rows with a non-zero gap below the
    near-tie threshold may differ.  Covers each gate list capacity on 128
    blocks (four 32-block score tiles): one pass with lists of 1, 2 and 4
    entries (top-2, top-3, top-5), two passes (8, 12, 32 entries), rounds."""
    D = 128 if dtype == "bf16" else 64
    w = small(f"ties_{dtype}_k{topk}", dtype, 1, 4096, 2, 1, D, 32, topk, seed=43)
    say(f"[case] exact ties {w} gate={gate}")
    q, k, v, _ = W.make_inputs(w, device="cpu")
    B = w.block_size
    for i in range(4, w.num_blocks):
        k[:, i * B:(i + 1) * B] = k[:, (i % 4) * B:(i % 4 + 1) * B]
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    out, sel = M.moba_attn_fwd(q, k, v, B, topk, True, gate=gate)
    torch.cuda.synchronize()
    from parity_utils import RowSource
    rows = [(0, t, h) for h in range(w.num_q_heads) for t in range(w.seqlen)]
    k32 = to_np32(k)
    mm = O.block_minmax(k32, B) if gate == "minmax" else None
    res = O.moba_rows(RowSource(q.cpu()), k32, to_np32(v), B, topk, True, rows, keep_scores=True, gate=gate,
                      minmax=mm)
    selh = sel.cpu().numpy()
    ties = O.near_tie_rows(res)
    exact = 0
    for r, (bb, t, h) in enumerate(rows):
        same = np.array_equal(selh[bb, h, t], res.sel[r])
        if res.gap[r] == 0:
            exact += 1
            assert same, f"exact tie row {(bb, t, h)}: gpu {selh[bb, h, t].tolist()} oracle {res.sel[r].tolist()}"
        elif not same:
            assert ties[r], f"row {(bb, t, h)}: selection differs, gap {res.gap[r]}"
    say(f"[ties] {exact} rows with an exact tie at the cut-off of {len(rows)}")
    assert exact > len(rows) // 4
    rep = compare(q, k, v, out, sel, B, topk, True, tol=TOL[dtype], gate=gate)
    say(f"[parity] {w.name}: {rep.as_dict()}")


def test_forward_minmax_gqa32x8_32k_sampled():
    """Min/max gate at 32K, 32 query / 8 KV heads, 128-key blocks, top-12
    (a selective configuration with 256 candidate blocks)."""
    w = small("mm_32k", "bf16", 1, 32768, 32, 8, 128, 128, 12, seed=21)
    rng = np.random.default_rng(5)
    rows = [(0, int(t), h) for h in range(32) for t in rng.integers(0, 32768, 16)]
    run(w, rows=rows, device_inputs=True, gate="minmax")


def test_forward_minmax_differs_from_mean():
    """The two gates are different selections on the same input (so the
    entry point does not silently run the mean gate)."""
    w = small("mm_vs_mean", "bf16", 1, 4096, 2, 1, 128, 64, 4, seed=9)
    q, k, v, _ = W.make_inputs(w, device="cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    _, s_mean = M.moba_attn_fwd(q, k, v, 64, 4, True, gate="mean")
    _, s_mm = M.moba_attn_fwd(q, k, v, 64, 4, True, gate="minmax")
    torch.cuda.synchronize()
    assert not torch.equal(s_mean, s_mm)


def test_forward_dense_equals_sdpa():
    """topk = n: equal to dense causal attention (course page: with every block
    chosen MoBA is dense attention); checked against torch's fp32 CPU SDPA."""
    w = small("dense_sdpa", "bf16", 1, 1024, 4, 2, 128, 128, 8)
    q, k, v, _ = W.make_inputs(w, device="cpu")
    out, _ = M.moba_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 128, 8, True)
    torch.cuda.synchronize()
    g = 2
    qt = q.float().permute(0, 2, 1, 3)
    kt = k.float().permute(0, 2, 1, 3).repeat_interleave(g, 1)
    vt = v.float().permute(0, 2, 1, 3).repeat_interleave(g, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(0, 2, 1, 3)
    assert (out.cpu().float() - ref).abs().max().item() < 2e-2


def test_forward_deterministic_and_future_invariant():
    w = small("determinism", "bf16", 1, 4096, 4, 2, 128, 256, 3)
    q, k, v, _ = W.make_inputs(w, device=DEV)
    o1, s1 = M.moba_attn_fwd(q, k, v, 256, 3, True)
    o2, s2 = M.moba_attn_fwd(q, k, v, 256, 3, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    # perturb every key and value after position t: rows <= t must not move by one bit
    for t in (700, 1023, 2100):
        k2, v2 = k.clone(), v.clone()
        k2[:, t + 1:] = (torch.randn_like(k2[:, t + 1:], dtype=torch.float32) * 5).to(k2.dtype)
        v2[:, t + 1:] = (torch.randn_like(v2[:, t + 1:], dtype=torch.float32) * 5).to(v2.dtype)
        o3, s3 = M.moba_attn_fwd(q, k2, v2, 256, 3, True)
        torch.cuda.synchronize()
        assert torch.equal(o3[:, :t + 1], o1[:, :t + 1])
        assert torch.equal(s3[:, :, :t + 1], s1[:, :, :t + 1])


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
def test_workload_tiny_f32_1k_both_topk():
    w = W.WORKLOADS["tiny_f32_1k"]
    run(w)
    run(w.with_(topk=8))


def test_forward_batch2_slice_images_sampled():
    """Long per-block row lists at batch 2: 384-row tiles fed from the K/V
    slice images, whose offsets depend on the batch entry."""
    w = small("gqa_b2_images", "bf16", 2, 8192, 32, 8, 128, 256, 8, seed=23)
    run(w, rows=W.sample_rows(w, 48, seed=24), device_inputs=True)


def test_forward_dense_one_block_sampled():
    """block_size = seqlen, topk = 1: dense causal attention through the own-block
    kernel alone (fed from the slice images); the dense baseline of the speedup curve."""
    w = small("dense_one_block", "bf16", 1, 16384, 8, 2, 128, 16384, 1, seed=25)
    run(w, rows=W.sample_rows(w, 48, seed=26), device_inputs=True)


@pytest.mark.slow
def test_forward_curve_dense_1m_sampled():
    """The speedup curve's dense baseline at its longest length: one causal
    block of 1M positions (block_size = seqlen, topk = 1), GQA 32/8; sampled
    rows including the first and last position (up to 1M keys per row)."""
    w = small("dense_1m", "bf16", 1, 1 << 20, 32, 8, 128, 1 << 20, 1, seed=33)
    rows = W.sample_rows(w, 4, seed=34, extra_positions=(1, 63, 64, 65535, 524288))
    run(w, rows=rows, device_inputs=True)


@pytest.mark.slow
def test_forward_block_40960_sampled():
    """The block size of the curve's 10M point (40960 keys: 640 slices per
    block), 16 blocks, top-12, GQA 32/8 (655 360 positions; the 10M point
    itself holds 200 GiB of inputs); sampled rows including every block's
    first and last position for head 0."""
    B = 40960
    w = small("b40960", "bf16", 1, 16 * B, 32, 8, 128, B, 12, seed=35)
    edges = [x for i in range(16) for x in (i * B, i * B + B - 1)]
    rows = W.sample_rows(w, 8, seed=36, extra_positions=edges[:8]) + [(0, t, 0) for t in edges[8:]]
    run(w, rows=sorted(set(rows)), device_inputs=True)


def test_forward_curve_config_32k_sampled():
    """The speedup curve's MoBA configuration at its shortest length: 256 blocks
    of 128, top-12, GQA 32/8."""
    w = small("curve_32k", "bf16", 1, 32768, 32, 8, 128, 128, 12, seed=27)
    run(w, rows=W.sample_rows(w, 24, seed=28), device_inputs=True)


def test_workload_mha16_8k_sampled():
    w = W.WORKLOADS["mha16_8k"]
    run(w, rows=W.sample_rows(w, 256, seed=21), device_inputs=True)


def test_workload_mha32_32k_needle_sampled():
    w = W.WORKLOADS["mha32_32k_needle"]
    rep, _ = run(w, rows=W.sample_rows(w, 256, seed=22), device_inputs=True)
    assert rep.rows >= 32 * 200


def chunk_edges(w: W.Workload, workspace_bytes=None):
    """First and last position of every query chunk the forward runs with the
    default workspace (or one of workspace_bytes)."""
    dt = M.DTYPE_BF16 if w.dtype == "bf16" else M.DTYPE_F32
    if workspace_bytes is None:
        workspace_bytes = M.workspace_bytes(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt,
                                            w.block_size, w.topk, w.causal)
    cb = M.plan_chunk_blocks(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt, w.block_size,
                             w.topk, w.causal, workspace_bytes)
    step = cb * w.block_size
    edges = []
    for t0 in range(0, w.seqlen, step):
        edges += [t0, min(t0 + step, w.seqlen) - 1]
    return cb, edges


@pytest.mark.slow
def test_workload_gqa32x8_128k_sampled():
    """128K positions at 256 seeded rows per head, with the first and last
    position of each query chunk (two chunks: 22 + 10 blocks)."""
    w = W.WORKLOADS["gqa32x8_128k"]
    cb, edges = chunk_edges(w)
    say(f"[chunks] {cb} blocks per chunk, edges {edges}")
    rep, _ = run(w, rows=W.sample_rows(w, 256, seed=23, extra_positions=edges), device_inputs=True)
    assert rep.rows >= 32 * 256


@pytest.mark.slow
def test_workload_gqa32x8_1m_sampled():
    """1M positions at 256 seeded rows per head, with the first and last
    position of each of the twelve query chunks."""
    w = W.WORKLOADS["gqa32x8_1m"]
    cb, edges = chunk_edges(w)
    say(f"[chunks] {cb} blocks per chunk, edges {edges}")
    assert len(edges) == 24
    rep, _ = run(w, rows=W.sample_rows(w, 256, seed=24, extra_positions=edges), device_inputs=True)
    assert rep.rows >= 32 * 256


CHUNKED = [
    # slice-image path (384-row tiles) in four chunks of 8 blocks
    (small("chunks_images", "bf16", 1, 16384, 8, 1, 128, 512, 3, seed=61), 8),
    # direct K/V path over ragged 96-key blocks in six chunks of 7 (+ 5) blocks
    (small("chunks_b96", "bf16", 1, 3840, 4, 2, 128, 96, 4, seed=62), 7),
    # fp32 path in three chunks
    (small("chunks_f32", "f32", 1, 1024, 2, 1, 64, 64, 5, seed=63), 6),
    # the smallest workspace: one block per chunk and no slice images, so the
    # long lists take 256-row tiles on K and V as they are (whole 64-key slices)
    (small("chunks_min_no_images", "bf16", 1, 8192, 4, 1, 128, 2048, 2, seed=64), 1),
]


@pytest.mark.parametrize("w,cap", CHUNKED, ids=[c[0].name for c in CHUNKED])
def test_forward_small_workspace_runs_in_query_chunks(w, cap):
    """A workspace smaller than the default makes the forward run in more
    query chunks (the longest that fit); every row is compared with the
    oracle, across every chunk boundary."""
    dt = M.DTYPE_BF16 if w.dtype == "bf16" else M.DTYPE_F32
    nbytes = M.workspace_bytes(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt, w.block_size,
                               w.topk, w.causal, max_chunk_blocks=cap)
    cb, edges = chunk_edges(w, nbytes)
    assert cb == cap and len(edges) >= 6
    if w.name == "chunks_min_no_images":
        info = M.plan_info(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt, w.block_size, w.topk,
                           w.causal, nbytes)
        assert info["tile_rows"] == 256 and not info["slice_images"], info
    say(f"[case] {w}: {cb} blocks per chunk, {len(edges) // 2} chunks")
    q, k, v, _ = W.make_inputs(w, device=DEV)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out, sel = M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, workspace=ws)
    torch.cuda.synchronize()
    rep = compare(q, k, v, out, sel, w.block_size, w.topk, w.causal, tol=TOL[w.dtype])
    say(f"[parity] {w.name}: {rep.as_dict()}")
    # the same selection as with the default workspace (one chunk here)
    out1, sel1 = M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel1)
    assert (out.float() - out1.float()).abs().max().item() <= 2 * TOL[w.dtype]


@pytest.mark.parametrize("n", [8, 128])
def test_forward_granularity_extremes_32k_sampled(n):
    """The coarsest and the finest of the report's block granularities at 32K
    and 75 % sparsity (8 blocks choosing 2; 128 blocks choosing 32), 32 MHA
    heads, sampled rows per head."""
    w = small(f"gran_n{n}", "bf16", 1, 32768, 32, 32, 128, 32768 // n, n // 4, seed=1200 + n)
    rng = np.random.default_rng(n)
    rows = [(0, int(t), h) for h in range(32) for t in rng.integers(0, 32768, 12)] + \
           [(0, t, 0) for t in (0, 32768 // n - 1, 32768 // n, 32767)]
    run(w, rows=rows, device_inputs=True)


def test_forward_max_blocks_sampled():
    """The largest block count whose rows the gate counts itself (8192
    blocks of 16 keys, 128K positions): the per-block counters fill 32 KiB of
    LDS and the top list ranks up to 8191 candidates."""
    w = small("n8192", "bf16", 1, 131072, 2, 2, 128, 16, 4, seed=77)
    rng = np.random.default_rng(3)
    rows = [(0, int(t), h) for h in range(2) for t in rng.integers(0, 131072, 24)] + \
           [(0, t, 1) for t in (0, 15, 16, 131071)]
    run(w, rows=rows, device_inputs=True)


MANY_BLOCKS = [
    (small("n16384_b4", "bf16", 1, 65536, 2, 1, 128, 4, 8, seed=81), "mean"),
    # 20010 blocks: a ragged last dispatch range and a ragged last score tile
    (small("n20010_b4_gqa", "bf16", 1, 80040, 4, 2, 128, 4, 6, seed=82), "mean"),
    (small("n16384_minmax", "bf16", 1, 65536, 2, 1, 128, 4, 5, seed=83), "minmax"),
    (small("n16384_noncausal", "bf16", 1, 65536, 2, 2, 128, 4, 5, causal=False, seed=84), "mean"),
    (small("n16384_f32", "f32", 1, 65536, 2, 1, 64, 4, 5, seed=85), "mean"),
]


@pytest.mark.parametrize("w,gate", MANY_BLOCKS, ids=[w.name for w, _ in MANY_BLOCKS])
def test_forward_many_blocks_sampled(w, gate):
    """More blocks than one pass of LDS counters holds (16384 and 20010
    blocks of 4 keys): the gate leaves the counting to the dispatch, which
    counts and ranks the rows per range of 8192 blocks; sampled rows across
    the sequence, the range boundary (block 8192) included."""
    rng = np.random.default_rng(w.seed)
    B = w.block_size
    edges = (0, B - 1, B, 8191 * B, 8192 * B - 1, 8192 * B, 8193 * B + 1, w.seqlen - 1)
    rows = [(0, int(t), h) for h in range(w.num_q_heads) for t in rng.integers(0, w.seqlen, 48)] + \
           [(0, t, h) for h in range(w.num_q_heads) for t in edges]
    run(w, rows=rows, device_inputs=True, gate=gate)


@pytest.mark.slow
def test_forward_many_blocks_1m_count_table_chunks_sampled():
    """1M positions in blocks of 16 keys (65536 blocks, 32/8 heads, top-3):
    the per-(list, work-group) count table would exceed its cap in one
    chunk, so the forward runs in chunks of 4096 blocks, each counted by the
    dispatch in eight ranges of 8192 blocks.  Sampled rows, with the first
    and last position of every chunk."""
    w = small("n65536_1m", "bf16", 1, 1 << 20, 32, 8, 128, 16, 3, seed=91)
    cb, edges = chunk_edges(w)
    say(f"[chunks] {cb} blocks per chunk, {len(edges) // 2} chunks")
    assert cb == 4096
    rng = np.random.default_rng(92)
    rows = [(0, int(t), int(h)) for t, h in zip(rng.integers(0, w.seqlen, 192), rng.integers(0, 32, 192))] + \
           [(0, t, int(h)) for t in edges for h in (0, 31)]
    run(w, rows=rows, device_inputs=True)
