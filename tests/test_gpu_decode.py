"""GPU parity of decode-time MoBA (moba_decode_fwd / moba_decode_means, through
the C ABI) against the fp64 oracle's decode_rows.

Tolerances: outputs within max-abs 2e-2 (bf16) and 1e-4 (fp32) of the oracle;
selections exact except counted near ties (parity_utils.compare_decode); block
means within Higham's gamma_{B+2} times the mean absolute key."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_40_amd as M
import moba_workloads as W
import oracle.moba_oracle as O
from parity_utils import compare, compare_decode, to_np32

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def wl(name, dtype, Hq, Hkv, Lmax, D, B, topk, lens, seed=3):
    return W.DecodeWorkload(name, dtype, Hq, Hkv, Lmax, D, B, topk, tuple(lens), seed=seed)


def mean_bound_ok(mu_gpu, kc, lens, B, blocks_of):
    """mu_gpu[b, hk, i] against the fp64 mean of block i for i in blocks_of(b)."""
    k32 = to_np32(kc)
    u = 2.0 ** -24
    gam = (B + 2) * u / (1 - (B + 2) * u)
    mu = mu_gpu.cpu().numpy().astype(np.float64)
    for bb, L in enumerate(lens):
        for i in blocks_of(bb, L):
            blk = k32[bb, i * B:(i + 1) * B].astype(np.float64)  # [B, Hkv, D]
            ref = blk.mean(axis=0)
            bound = gam * np.abs(blk).mean(axis=0)
            assert np.all(np.abs(mu[bb, :, i] - ref) <= bound + 1e-30), (bb, i)


def run(w, rows=None, check_means=True):
    say(f"[case] {w}")
    q, kc, vc, lens = W.make_decode_inputs(w, device="cpu")
    q, kc, vc, lens_d = q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)
    B = w.block_size
    mu = M.moba_decode_means(kc, lens_d, B)
    out, sel = M.moba_decode_fwd(q, kc, vc, mu, lens_d, B, w.topk)
    torch.cuda.synchronize()
    if check_means:
        # every complete block, including one the step itself completed
        mean_bound_ok(mu, kc, w.lens, B, lambda bb, L: range(L // B))
    rep = compare_decode(q, kc, vc, w.lens, out, sel, B, w.topk, rows=rows, tol=TOL[w.dtype])
    say(f"[parity] {w.name}: {rep.as_dict()}")
    return rep, (q, kc, vc, lens_d, mu, out, sel)


CASES = [
    # several score chunks per head, ragged own blocks, L = 1, L = B, L = B + 1
    wl("gqa4_b128", "bf16", 8, 2, 2048, 128, 128, 4, [2048, 1000, 129, 128, 1, 1537]),
    wl("mha_b64_k9", "bf16", 4, 4, 4096, 128, 64, 9, [4096, 4033, 2111]),
    wl("g16_b256", "bf16", 16, 1, 8192, 128, 256, 6, [8192, 5000]),
    wl("topk1_own_only", "bf16", 8, 2, 2048, 128, 128, 1, [2048, 700]),
    wl("dense_topk_ge_n", "bf16", 4, 2, 1024, 128, 128, 9, [1024, 555]),
    wl("topk64", "bf16", 4, 1, 16384, 128, 64, 64, [16384, 9000]),
    wl("b2048_long_blocks", "bf16", 4, 1, 16384, 128, 2048, 3, [16384, 12289]),
    wl("b16_small_blocks", "bf16", 4, 2, 1024, 128, 16, 5, [1024, 17, 999]),
    wl("f32_d64", "f32", 4, 2, 1024, 64, 64, 4, [1024, 300, 65]),
    wl("f32_d128", "f32", 4, 1, 2048, 128, 128, 3, [2048, 1500]),
    # a group of 3 query heads per KV head
    wl("g3_b128", "bf16", 6, 2, 2048, 128, 128, 4, [2048, 1111, 300]),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_decode_small(w):
    run(w)


def test_decode_mean_update_for_the_completed_block():
    """A step whose token completes block j (L % B == 0) writes mean j; no
    other entry changes."""
    w = wl("mean_update", "bf16", 8, 2, 2048, 128, 128, 3, [1024, 1000, 2048])
    q, kc, vc, lens = W.make_decode_inputs(w, device="cpu")
    q, kc, vc, lens_d = q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)
    B = w.block_size
    # cached means of the blocks before each own block only
    lens_before = torch.tensor([((L - 1) // B) * B for L in w.lens], dtype=torch.int32, device=DEV)
    mu = torch.full((3, 2, 2048 // B, 128), 7.0, dtype=torch.float32, device=DEV)
    M.moba_decode_means(kc, lens_before, B, mu)
    before = mu.clone()
    M.moba_decode_fwd(q, kc, vc, mu, lens_d, B, w.topk)
    torch.cuda.synchronize()
    changed = (mu != before).any(dim=-1).any(dim=1).cpu()  # [b, n]
    for bb, L in enumerate(w.lens):
        want = [L // B - 1] if L % B == 0 else []
        assert [int(i) for i in torch.nonzero(changed[bb]).flatten()] == want
    mean_bound_ok(mu, kc, w.lens, B, lambda bb, L: range(L // B))
    assert torch.all(mu[1, :, 1000 // B:] == 7.0)  # sequence 1 has no complete block there


def test_decode_out_of_range_lengths_give_zero_rows():
    w = wl("bad_len", "bf16", 4, 2, 1024, 128, 128, 3, [1024, 512, 700])
    q, kc, vc, _ = W.make_decode_inputs(w, device="cpu")
    q, kc, vc = q.to(DEV), kc.to(DEV), vc.to(DEV)
    lens_d = torch.tensor([0, 1025, 700], dtype=torch.int32, device=DEV)
    mu = M.moba_decode_means(kc, lens_d, 128)
    out, sel = M.moba_decode_fwd(q, kc, vc, mu, lens_d, 128, 3)
    torch.cuda.synchronize()
    assert torch.all(out[:2] == 0) and torch.all(sel[:2] == -1)
    rep = compare_decode(q, kc, vc, [1, 1, 700], out, sel, 128, 3, rows=[(2, h) for h in range(4)])
    say(f"[parity] bad_len valid row: {rep.as_dict()}")


def test_decode_equals_prefill_last_row_on_the_gpu():
    """At L = S the decode step is prefill row S - 1 (both HIP paths; same
    selection, outputs within the bf16 tolerance)."""
    pw = W.Workload("pre", "bf16", 1, 8, 2, 4096, 128, 256, 5, seed=31)
    q, k, v, _ = W.make_inputs(pw, device="cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    out_p, sel_p = M.moba_attn_fwd(q, k, v, 256, 5, True)
    lens_d = torch.tensor([4096], dtype=torch.int32, device=DEV)
    mu = M.moba_decode_means(k, lens_d, 256)
    qd = q[:, -1].contiguous()
    out_d, sel_d = M.moba_decode_fwd(qd, k, v, mu, lens_d, 256, 5)
    torch.cuda.synchronize()
    assert torch.equal(sel_d[0], sel_p[0, :, -1])
    err = (out_d[0].float() - out_p[0, -1].float()).abs().max().item()
    say(f"[decode vs prefill] max err {err:.3e}")
    assert err < 2e-2


def test_decode_workload_1m_sampled():
    """The bench's decode layout (32/8 heads, D 128, block 4096, top-12) at
    1M cached positions, two sequences (one at a block boundary), every row."""
    w = wl("d1m", "bf16", 32, 8, 1 << 20, 128, 4096, 12, [(1 << 20) - 4096, (1 << 20) - 70001], seed=2001)
    say(f"[case] {w}")
    q, kc, vc, lens = W.make_decode_inputs(w, device=DEV)
    B = w.block_size
    mu = M.moba_decode_means(kc, lens, B)
    out, sel = M.moba_decode_fwd(q, kc, vc, mu, lens, B, w.topk)
    torch.cuda.synchronize()
    rep = compare_decode(q, kc, vc, w.lens, out, sel, B, w.topk, tol=TOL["bf16"])
    say(f"[parity] {w.name}: {rep.as_dict()}")
