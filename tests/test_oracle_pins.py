"""Pins for the fp64 oracle: checks against things other than the oracle itself.

- printed figures (sparsity, block counts) from the pages, under tests/golden;
- dense causal / non-causal attention from torch's scaled_dot_product_attention
  in fp64 when every block is selected (course summary: all blocks selected is
  exactly dense attention);
- textbook masked attention for the special cases the report names
  (own block only; sliding window = previous block + own, report §2.4);
- brute force over all block subsets and an explicit S x S mask on tiny inputs;
- invariants that hold exactly in exact arithmetic (future keys never matter,
  report §2.3; key shifts, value affine maps, in-block permutations);
- planted mistakes in a copy of the oracle, which the pins must catch.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.moba_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(rng, b, S, Hq, Hkv, D, scale=1.0):
    q = rng.standard_normal((b, S, Hq, D)) * scale
    k = rng.standard_normal((b, S, Hkv, D)) * scale
    v = rng.standard_normal((b, S, Hkv, D))
    return q, k, v


def sdpa_fp64(q, k, v, mask=None, causal=False):
    """torch SDPA in fp64 on [b, S, H, D] numpy arrays; KV heads are expanded
    with repeat_interleave (query head h reads KV head h // g)."""
    Hq, Hkv = q.shape[2], k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal)
    return o.permute(0, 2, 1, 3).numpy()


# ----------------------------------------------------------------------------
# printed figures
# ----------------------------------------------------------------------------
def test_printed_sparsity_pins_topk_counts_own_block():
    cases = json.load(open(os.path.join(GOLDEN, "sparsity_figures.json")))["cases"]
    rng = np.random.default_rng(0)
    for c in cases:
        n = O.num_blocks(c["seqlen"], c["block_size"])
        assert n == c["num_blocks"]
        # a late query (own block n-1): how many blocks does the gate keep?
        scores = rng.standard_normal(n)
        sel = O.select_blocks(scores, n - 1, c["topk"], True)
        sparsity = 100.0 * (1.0 - len(sel) / n)
        assert round(sparsity, 2) == c["sparsity_percent_printed"]


def test_count_selected_keys_matches_rule():
    # keys per head = sum over rows of min(k-1, j) B + (r+1)
    S, B, k = 1024, 128, 3
    n = S // B
    want = sum(min(k - 1, j) * B * B + B * (B + 1) // 2 for j in range(n))
    assert O.count_selected_keys(S, B, k, True) == want
    # dense: topk >= n gives S(S+1)/2 keys
    assert O.count_selected_keys(S, B, n, True) == S * (S + 1) // 2
    assert O.count_selected_keys(S, B, 2 * n, True) == S * (S + 1) // 2


# ----------------------------------------------------------------------------
# dense equality and textbook special cases
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 64, 2, 2, 16, 8), (2, 96, 4, 2, 8, 16), (1, 128, 3, 1, 32, 32)])
@pytest.mark.parametrize("extra", [0, 3])
def test_dense_equality_causal(shape, extra):
    b, S, Hq, Hkv, D, B = shape
    rng = np.random.default_rng(1)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    n = S // B
    out, sel = O.moba_forward(q, k, v, B, n + extra, causal=True)
    ref = sdpa_fp64(q, k, v, causal=True)
    assert np.max(np.abs(out - ref)) < 1e-12
    # every causal block is chosen
    for t in range(S):
        assert list(sel[0, 0, t][sel[0, 0, t] >= 0]) == list(range(t // B + 1))


def test_dense_equality_noncausal():
    b, S, Hq, Hkv, D, B = 1, 64, 2, 1, 16, 16
    rng = np.random.default_rng(2)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    out, sel = O.moba_forward(q, k, v, B, S // B, causal=False)
    ref = sdpa_fp64(q, k, v, causal=False)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_topk1_is_block_local_causal_attention():
    b, S, Hq, Hkv, D, B = 1, 96, 2, 2, 16, 16
    rng = np.random.default_rng(3)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    out, _ = O.moba_forward(q, k, v, B, 1, causal=True)
    t = np.arange(S)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] // B == t[:, None] // B)
    ref = sdpa_fp64(q, k, v, mask=mask)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_sliding_window_construction():
    """report §2.4: SWA = always routing to the most recent block.  Plant a
    strong alignment between each query and its previous block's keys; with
    topk = 2 the gate must pick exactly {j-1, j}, and the output must equal
    attention over the window [(j-1)B, t]."""
    b, S, Hq, Hkv, D, B = 1, 128, 1, 1, 16, 16
    rng = np.random.default_rng(4)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D, scale=0.1)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q[0, :, 0, :] += 3.0 * u
    # every block's keys carry a rising multiple of u, so the newest past
    # block always has the largest mean-key score
    for i in range(S // B):
        k[0, i * B:(i + 1) * B, 0, :] += (0.5 * i) * u
    out, sel = O.moba_forward(q, k, v, B, 2, causal=True)
    t = np.arange(S)
    j = t // B
    lo = np.maximum(j - 1, 0) * B
    mask = (t[None, :] <= t[:, None]) & (t[None, :] >= lo[:, None])
    ref = sdpa_fp64(q, k, v, mask=mask)
    for tt in range(S):
        jj = tt // B
        want = [jj - 1, jj] if jj >= 1 else [0, -1]
        assert list(sel[0, 0, tt]) == want
    assert np.max(np.abs(out - ref)) < 1e-12


def test_gqa_head_mapping_dense():
    b, S, Hq, Hkv, D, B = 1, 64, 6, 2, 8, 16
    rng = np.random.default_rng(5)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    out, _ = O.moba_forward(q, k, v, B, 100, causal=True)
    ref = sdpa_fp64(q, k, v, causal=True)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_gqa_routing_equals_expanded_mha():
    """Sparse case: a GQA call equals the MHA call on explicitly expanded K/V
    (query head h reads KV head h // g, per-head routing)."""
    b, S, Hq, Hkv, D, B = 1, 128, 4, 2, 8, 16
    rng = np.random.default_rng(6)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    out, sel = O.moba_forward(q, k, v, B, 3, causal=True)
    ke = np.repeat(k, Hq // Hkv, axis=2)
    ve = np.repeat(v, Hq // Hkv, axis=2)
    out2, sel2 = O.moba_forward(q, ke, ve, B, 3, causal=True)
    assert np.array_equal(sel, sel2)
    assert np.max(np.abs(out - out2)) == 0.0


# ----------------------------------------------------------------------------
# brute force on tiny inputs
# ----------------------------------------------------------------------------
def brute_force(q, k, v, B, topk, causal):
    """Enumerate every admissible block subset of the right size, take the one
    with the largest score sum (ties: lexicographically smallest index tuple),
    build the S x S mask element by element and run a per-query masked
    softmax with explicit loops."""
    b, S, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    n = S // B
    out = np.zeros_like(q)
    sels = np.full((b, Hq, S, topk), -1, dtype=np.int32)
    for bb in range(b):
        for h in range(Hq):
            hk = h // g
            mu = [[sum(k[bb, s, hk, d] for s in range(i * B, (i + 1) * B)) / B for d in range(D)]
                  for i in range(n)]
            for t in range(S):
                j = t // B
                score = [sum(q[bb, t, h, d] * mu[i][d] for d in range(D)) for i in range(n)]
                if causal:
                    m = min(topk - 1, j)
                    best = None
                    for sub in itertools.combinations(range(j), m):
                        key = (sum(score[i] for i in sub), tuple(-i for i in sub))
                        if best is None or key > best[0]:
                            best = (key, sub)
                    chosen = sorted(best[1] + (j,))
                else:
                    m = min(topk, n)
                    best = None
                    for sub in itertools.combinations(range(n), m):
                        key = (sum(score[i] for i in sub), tuple(-i for i in sub))
                        if best is None or key > best[0]:
                            best = (key, sub)
                    chosen = sorted(best[1])
                sels[bb, h, t, :len(chosen)] = chosen
                mask = [False] * S
                for s in range(S):
                    i = s // B
                    if i in chosen and (not causal or s <= t):
                        mask[s] = True
                logits = [sum(q[bb, t, h, d] * k[bb, s, hk, d] for d in range(D)) / math.sqrt(D)
                          if mask[s] else -math.inf for s in range(S)]
                mx = max(logits)
                w = [math.exp(x - mx) if x != -math.inf else 0.0 for x in logits]
                z = sum(w)
                for d in range(D):
                    out[bb, t, h, d] = sum(w[s] * v[bb, s, hk, d] for s in range(S)) / z
    return out, sels


@pytest.mark.parametrize("S,B,topk,causal,Hq,Hkv", [
    (32, 8, 2, True, 1, 1), (32, 4, 3, True, 2, 1), (24, 4, 4, True, 2, 2),
    (32, 8, 1, True, 1, 1), (16, 4, 2, False, 1, 1), (24, 8, 9, True, 2, 1),
])
def test_bruteforce_tiny(S, B, topk, causal, Hq, Hkv):
    rng = np.random.default_rng(7 + S + B + topk)
    q, k, v = rand_qkv(rng, 1, S, Hq, Hkv, 4)
    out, sel = O.moba_forward(q, k, v, B, topk, causal)
    bout, bsel = brute_force(q, k, v, B, topk, causal)
    assert np.array_equal(sel, bsel)
    assert np.max(np.abs(out - bout)) < 1e-12


def test_bruteforce_exact_ties_go_to_lower_index():
    """Integer-valued keys make several block means (and scores) exactly
    equal; the chosen set must be the lowest-indexed among the tied ones."""
    S, B, D = 32, 4, 2
    rng = np.random.default_rng(8)
    q = rng.integers(-2, 3, size=(1, S, 1, D)).astype(np.float64)
    base = rng.integers(-2, 3, size=(B, D)).astype(np.float64)
    k = np.zeros((1, S, 1, D))
    for i in range(S // B):
        k[0, i * B:(i + 1) * B, 0] = base if i % 2 == 0 else base[::-1]  # equal means
    v = rng.standard_normal((1, S, 1, D))
    for topk in (2, 3):
        out, sel = O.moba_forward(q, k, v, B, topk, True)
        bout, bsel = brute_force(q, k, v, B, topk, True)
        assert np.array_equal(sel, bsel)
        assert np.max(np.abs(out - bout)) < 1e-12
        # all past means are equal: the gate must take the lowest past blocks
        for t in range(S):
            j = t // B
            m = min(topk - 1, j)
            assert list(sel[0, 0, t][:m]) == list(range(m))


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_future_keys_never_matter():
    b, S, Hq, Hkv, D, B = 1, 96, 2, 1, 8, 16
    rng = np.random.default_rng(9)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    out, sel = O.moba_forward(q, k, v, B, 3, True)
    for t in [0, 5, 15, 16, 40, 63, 64, 80, 94]:
        k2, v2 = k.copy(), v.copy()
        k2[:, t + 1:] = rng.standard_normal(k2[:, t + 1:].shape) * 7.0
        v2[:, t + 1:] = rng.standard_normal(v2[:, t + 1:].shape) * 7.0
        res = O.moba_rows(q, k2, v2, B, 3, True, [(0, t, h) for h in range(Hq)])
        for h in range(Hq):
            assert np.array_equal(res.out[h], out[0, t, h])  # bit-exact
            assert np.array_equal(res.sel[h], sel[0, h, t])


def test_own_block_always_selected_and_padding():
    b, S, Hq, Hkv, D, B = 1, 128, 2, 2, 8, 16
    rng = np.random.default_rng(10)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    for topk in (1, 2, 3, 5, 8, 12):
        _, sel = O.moba_forward(q, k, v, B, topk, True)
        for h in range(Hq):
            for t in range(S):
                j = t // B
                row = sel[0, h, t]
                valid = row[row >= 0]
                assert j in valid
                assert len(valid) == min(topk, j + 1)
                assert np.all(valid <= j)
                assert list(valid) == sorted(valid)
                assert np.all(row[len(valid):] == -1)


def test_key_shift_and_value_affine_invariance():
    b, S, Hq, Hkv, D, B = 1, 128, 2, 1, 8, 16
    rng = np.random.default_rng(11)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    out, sel = O.moba_forward(q, k, v, B, 3, True)
    c = rng.standard_normal(D)
    out_k, sel_k = O.moba_forward(q, k + c, v, B, 3, True)
    assert np.array_equal(sel, sel_k)
    assert np.max(np.abs(out - out_k)) < 1e-12
    a, cv = 1.7, rng.standard_normal(D)
    out_v, sel_v = O.moba_forward(q, k, a * v + cv, B, 3, True)
    assert np.array_equal(sel, sel_v)
    assert np.max(np.abs(a * out + cv - out_v)) < 1e-12


def test_permuting_keys_inside_a_past_block():
    b, S, Hq, Hkv, D, B = 1, 128, 1, 1, 8, 16
    rng = np.random.default_rng(12)
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    out, sel = O.moba_forward(q, k, v, B, 3, True)
    perm = rng.permutation(B)
    k2, v2 = k.copy(), v.copy()
    blk = 2
    k2[0, blk * B:(blk + 1) * B] = k[0, blk * B + perm]
    v2[0, blk * B:(blk + 1) * B] = v[0, blk * B + perm]
    out2, sel2 = O.moba_forward(q, k2, v2, B, 3, True)
    assert np.array_equal(sel, sel2)
    # rows past block 2 see a permuted but equal key set
    assert np.max(np.abs(out[0, (blk + 1) * B:] - out2[0, (blk + 1) * B:])) < 1e-12


def test_block_means_definition():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((2, 32, 3, 4))
    mu = O.block_means(k, 8)
    assert mu.shape == (2, 3, 4, 4)
    for bb in range(2):
        for hk in range(3):
            for i in range(4):
                want = [math.fsum(k[bb, s, hk, d] for s in range(8 * i, 8 * i + 8)) / 8 for d in range(4)]
                assert np.max(np.abs(mu[bb, hk, i] - want)) < 1e-15
    with pytest.raises(ValueError):
        O.block_means(k, 5)


# ----------------------------------------------------------------------------
# near-tie protocol: the relative-gap rule, and the fp32 score error bounds
# ----------------------------------------------------------------------------
def _tie_case(delta):
    """One query row (t = 63, B = 16, topk = 2: one past slot among blocks
    0..2) whose block 1 mean is block 0's scaled by (1 + delta), with block 2
    far below both: the top-1 boundary lies between blocks 1 and 0 and their
    fp64 gap is delta / (1 + delta) of the larger score."""
    rng = np.random.default_rng(14)
    q, k, v = rand_qkv(rng, 1, 64, 1, 1, 8)
    t = 63
    qd = q[0, t, 0] / np.linalg.norm(q[0, t, 0])
    k[0, 0:16, 0] = rng.standard_normal((16, 8)) + 2.0 * qd  # block 0 scores well above 0
    k[0, 16:32] = k[0, 0:16] * (1.0 + delta)
    k[0, 32:48, 0] = k[0, 0:16, 0] - 6.0 * qd
    return O.moba_rows(q, k, v, 16, 2, True, [(0, t, 0)], keep_scores=True)


def test_near_tie_rule_is_the_relative_gap():
    # an almost exact tie, gap 1e-9 relative: a near tie
    res = _tie_case(1e-9)
    assert res.sel[0].tolist()[:1] == [1] and O.near_tie_rows(res)[0]
    # just inside and just outside 1e-4 relative
    assert O.near_tie_rows(_tie_case(0.9e-4))[0]
    assert not O.near_tie_rows(_tie_case(1.2e-4))[0]
    # a clear separation is not a near tie; the valid-set check uses the
    # relative tolerance on the candidates' scores
    res2 = _tie_case(0.5)
    assert not O.near_tie_rows(res2)[0]
    s2 = res2.scores[0]
    tol = 1e-4 * O.near_tie_scale(res2)[0]
    assert O.valid_topk_set(s2, [1], 3, 1, tol)
    assert not O.valid_topk_set(s2, [0], 3, 1, tol)
    assert not O.valid_topk_set(s2, [2], 3, 1, tol)
    # at the near tie either of the two tied blocks is a valid choice
    res3 = _tie_case(1e-9)
    tol3 = 1e-4 * O.near_tie_scale(res3)[0]
    assert O.valid_topk_set(res3.scores[0], [0], 3, 1, tol3)
    assert O.valid_topk_set(res3.scores[0], [1], 3, 1, tol3)
    assert not O.valid_topk_set(res3.scores[0], [2], 3, 1, tol3)


F32 = np.float32


def _fp32_sum(x, order, groups=4):
    """Sum the rows of x [n, ...] in fp32, rounding after every addition, in
    the given order: sequential, reverse, pairwise (recursive halves), or
    `groups` interleaved partial sums (rows r, r + groups, ...) added at the
    end."""
    x = np.asarray(x, dtype=F32)

    def seq(rows):
        acc = rows[0].copy()
        for row in rows[1:]:
            acc = (acc + row).astype(F32)
        return acc

    def pw(rows):
        if len(rows) == 1:
            return rows[0].copy()
        h = len(rows) // 2
        return (pw(rows[:h]) + pw(rows[h:])).astype(F32)

    if order == "sequential":
        return seq(x)
    if order == "reverse":
        return seq(x[::-1])
    if order == "pairwise":
        return pw(x)
    if order == "interleaved":
        g = min(groups, len(x))
        return seq(np.stack([seq(x[r::g]) for r in range(g)]))
    raise ValueError(order)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


ORDERS = ("sequential", "reverse", "pairwise", "interleaved")


def _fp32_mean_gate_scores(q, kb, mean_order, dot_order, split):
    """fp32 emulation of one row's gate scores: the block means summed in fp32
    in `mean_order` and divided by B in fp32, then q . mu in fp32 in
    `dot_order`, either from fp32-rounded products (fp32 inputs) or with each
    mean split exactly into three bf16 parts (q in bf16, exact products).
    q: [D]; kb: [n, B, D] fp32 values.  Returns [n]."""
    n, B, D = kb.shape
    mu = np.stack([(_fp32_sum(kb[i], mean_order) / F32(B)).astype(F32) for i in range(n)])  # [n, D]
    if split:
        hi = _bf16(mu)
        mid = _bf16((mu - hi).astype(F32))
        lo = _bf16((mu - hi - mid).astype(F32))
        assert np.array_equal((hi.astype(np.float64) + mid + lo), mu.astype(np.float64))
        terms = np.concatenate([q * hi, q * mid, q * lo], axis=1).astype(F32)  # exact products
    else:
        terms = (q.astype(F32) * mu).astype(F32)
    return _fp32_sum(terms.T, dot_order)


def _mean_bound_worst_ratio():
    """Largest |emulated fp32 score - exact score| / score_error_bound over
    random inputs (bf16 and fp32, several B) and inputs built to make every
    fp32 addition lose half an ulp, in every summation order."""
    u = 2.0 ** -24
    worst = 0.0
    cases = []
    rng = np.random.default_rng(40)
    for B, D, split in ((16, 128, True), (256, 128, True), (4096, 128, True), (128, 64, False), (64, 128, False)):
        kb = rng.standard_normal((3, B, D)).astype(F32)
        q = rng.standard_normal(D).astype(F32)
        if split:
            kb, q = _bf16(kb), _bf16(q)
        cases.append((q, kb, split))
    # adversarial mean: one coordinate holds [1, u, u, ...]; 1 + u rounds back
    # to 1 at every step of a sequential sum
    B = 4096
    kb = np.zeros((1, B, 128), dtype=F32)
    kb[0, 0, 0] = 1.0
    kb[0, 1:, 0] = u
    q = np.zeros(128, dtype=F32)
    q[0] = 1.0
    cases.append((q, kb, True))
    # adversarial dot product: mean [1, u, ..., u] (every key equal to it),
    # q all ones: the products 1, u, u, ... lose every u
    B = 16
    kb = np.zeros((1, B, 128), dtype=F32)
    kb[0, :, 0] = 1.0
    kb[0, :, 1:] = u
    cases.append((np.ones(128, dtype=F32), kb, True))
    for q, kb, split in cases:
        n, B, D = kb.shape
        q64 = q.astype(np.float64)
        k64 = kb.astype(np.float64)
        mu64 = k64.mean(axis=1)
        exact = mu64 @ q64
        bound = O.score_error_bound(q64, mu64, np.abs(k64).mean(axis=1), B)
        for mo in ORDERS:
            for do in ORDERS:
                got = _fp32_mean_gate_scores(q, kb, mo, do, split).astype(np.float64)
                worst = max(worst, float(np.max(np.abs(got - exact))) / bound)
    return worst


def _minmax_bound_worst_ratio():
    """The same for the min/max gate: the score sum_d max(q_d lo_d, q_d hi_d)
    formed in fp32 as the larger of two rounded products per d (fp32 inputs)
    or as the 2 D exact products q+ . hi + q- . lo (bf16 inputs), summed in
    every order."""
    u = 2.0 ** -24
    rng = np.random.default_rng(41)
    cases = []
    for D, split in ((128, True), (64, False)):
        kb = rng.standard_normal((3, 64, D)).astype(F32)
        q = rng.standard_normal(D).astype(F32)
        if split:
            kb, q = _bf16(kb), _bf16(q)
        cases.append((q, kb.min(axis=1), kb.max(axis=1), split))
    hi = np.full((1, 128), u, dtype=F32)
    hi[0, 0] = 1.0
    cases.append((np.ones(128, dtype=F32), hi.copy(), hi, True))
    worst = 0.0
    for q, lo, hi, split in cases:
        q64 = q.astype(np.float64)
        exact = np.maximum(lo.astype(np.float64) * q64, hi.astype(np.float64) * q64).sum(axis=1)
        bound = O.score_error_bound_minmax(q64, lo.astype(np.float64), hi.astype(np.float64))
        if split:
            qp, qm = np.maximum(q, F32(0)), np.minimum(q, F32(0))
            terms = np.concatenate([qp * hi, qm * lo], axis=1).astype(F32)
        else:
            terms = np.maximum((q * lo).astype(F32), (q * hi).astype(F32))
        for o in ORDERS:
            got = _fp32_sum(terms.T, o).astype(np.float64)
            worst = max(worst, float(np.max(np.abs(got - exact))) / bound)
    return worst


def test_score_error_bound_holds_and_is_attained():
    """The worst-case fp32 error bound of a mean-gate score holds for every
    summation order, and inputs built so that each addition loses half an ulp
    reach more than a tenth of it (so a bound ten times too small fails)."""
    r = _mean_bound_worst_ratio()
    assert 0.1 < r <= 1.0, r


def test_score_error_bound_minmax_holds_and_is_attained():
    r = _minmax_bound_worst_ratio()
    assert 0.1 < r <= 1.0, r


def test_planted_small_error_bounds_are_caught(monkeypatch):
    """Both bounds planted ten times too small: the emulated errors exceed them."""
    gamma = O._gamma
    monkeypatch.setattr(O, "_gamma", lambda n, u=2.0 ** -24: 0.1 * gamma(n, u))
    assert _mean_bound_worst_ratio() > 1.0
    assert _minmax_bound_worst_ratio() > 1.0


# ----------------------------------------------------------------------------
# planted mistakes: each variant must fail at least one pin above
# ----------------------------------------------------------------------------
def _mutant_select(kind):
    orig = O.select_blocks

    def sel(scores, j, topk, causal):
        if kind == "no_forced_own":
            past = list(range(j + 1))
            ranked = sorted(past, key=lambda i: (-float(scores[i]), i))
            return sorted(ranked[:min(topk, j + 1)])
        if kind == "k_excludes_own":
            ranked = sorted(range(j), key=lambda i: (-float(scores[i]), i))
            return sorted(ranked[:min(topk, j)] + [j])
        if kind == "ties_to_higher":
            ranked = sorted(range(j), key=lambda i: (-float(scores[i]), -i))
            return sorted(ranked[:min(topk - 1, j)] + [j])
        if kind == "future_leak":
            cand = list(range(min(j + 2, len(scores))))
            cand.remove(j)
            ranked = sorted(cand, key=lambda i: (-float(scores[i]), i))
            return sorted(ranked[:min(topk - 1, len(cand))] + [j])
        return orig(scores, j, topk, causal)
    return sel


@pytest.mark.parametrize("kind", ["no_forced_own", "k_excludes_own", "ties_to_higher", "future_leak"])
def test_planted_selection_mistakes_are_caught(kind, monkeypatch):
    rng = np.random.default_rng(15)
    S, B = 32, 4
    q, k, v = rand_qkv(rng, 1, S, 1, 1, 3)
    # exact ties as in the tie test so the tie rule is exercised
    base = rng.integers(-2, 3, size=(B, 3)).astype(np.float64)
    kt = np.zeros((1, S, 1, 3))
    for i in range(S // B):
        kt[0, i * B:(i + 1) * B, 0] = base if i % 2 == 0 else base[::-1]
    qt = rng.integers(-2, 3, size=(1, S, 1, 3)).astype(np.float64)
    monkeypatch.setattr(O, "select_blocks", _mutant_select(kind))
    caught = False
    for (qq, kk) in ((q, k), (qt, kt)):
        bout, bsel = brute_force(qq, kk, v, B, 2, True)
        try:
            out, sel = O.moba_forward(qq, kk, v, B, 2, True)
        except ValueError:  # more blocks than slots: the mutant cannot even fill sel_idx
            caught = True
            continue
        if not np.array_equal(sel, bsel) or np.max(np.abs(out - bout)) > 1e-12:
            caught = True
    # the printed sparsity figures catch a wrong slot count on their own
    try:
        test_printed_sparsity_pins_topk_counts_own_block()
    except AssertionError:
        caught = True
    assert caught


def test_planted_missing_scale_is_caught(monkeypatch):
    rng = np.random.default_rng(16)
    q, k, v = rand_qkv(rng, 1, 64, 1, 1, 16)
    orig = O._attend_blocks

    def no_scale(q64, kh, vh, sel, t, B, causal, scale):
        return orig(q64, kh, vh, sel, t, B, causal, 1.0)
    monkeypatch.setattr(O, "_attend_blocks", no_scale)
    out, _ = O.moba_forward(q, k, v, 16, 4, True)
    assert np.max(np.abs(out - sdpa_fp64(q, k, v, causal=True))) > 1e-6


def test_planted_own_block_off_by_one_is_caught(monkeypatch):
    """Letting the own block see one key past the query breaks future
    invariance and dense equality."""
    rng = np.random.default_rng(17)
    q, k, v = rand_qkv(rng, 1, 64, 1, 1, 8)
    orig = O._attend_blocks

    def leak(q64, kh, vh, sel, t, B, causal, scale):
        return orig(q64, kh, vh, sel, min(t + 1, kh.shape[0] - 1), B, causal, scale) if (t + 1) % B else \
            orig(q64, kh, vh, sel, t, B, causal, scale)
    monkeypatch.setattr(O, "_attend_blocks", leak)
    out, _ = O.moba_forward(q, k, v, 16, 4, True)
    assert np.max(np.abs(out - sdpa_fp64(q, k, v, causal=True))) > 1e-6


# ----------------------------------------------------------------------------
# the Quest-style min/max gate (report §1.3: MoBA with min/max pooling)
# ----------------------------------------------------------------------------
def test_minmax_score_is_the_largest_logit_over_the_box():
    """The min/max score bounds q.k from above for every key of the block,
    equals it when the block has one key, and is attained at the box corner
    that takes the upper bound where q_d >= 0 and the lower one elsewhere."""
    rng = np.random.default_rng(31)
    D, B, n = 6, 5, 7
    keys = rng.standard_normal((n, B, D))
    lo = np.array([[min(keys[i, s, d] for s in range(B)) for d in range(D)] for i in range(n)])
    hi = np.array([[max(keys[i, s, d] for s in range(B)) for d in range(D)] for i in range(n)])
    for _ in range(20):
        q = rng.standard_normal(D)
        sc = O.gate_scores_minmax(q, lo, hi)
        for i in range(n):
            best_key = max(float(keys[i, s] @ q) for s in range(B))
            assert sc[i] >= best_key - 1e-12
            corner = np.array([hi[i, d] if q[d] >= 0 else lo[i, d] for d in range(D)])
            assert abs(sc[i] - float(corner @ q)) < 1e-12
    # one key per block: the box is a point and the score is the logit itself
    one = rng.standard_normal((n, D))
    q = rng.standard_normal(D)
    assert np.max(np.abs(O.gate_scores_minmax(q, one, one) - one @ q)) < 1e-12


def test_block_minmax_definition():
    rng = np.random.default_rng(32)
    k = rng.standard_normal((2, 24, 3, 4))
    lo, hi = O.block_minmax(k, 8)
    for bb in range(2):
        for hk in range(3):
            for i in range(3):
                for d in range(4):
                    vals = [k[bb, s, hk, d] for s in range(i * 8, (i + 1) * 8)]
                    assert lo[bb, hk, i, d] == min(vals) and hi[bb, hk, i, d] == max(vals)


def brute_force_minmax_selection(q, k, B, topk):
    """Causal selection with the min/max gate, by explicit loops and subset
    enumeration (max score sum, ties to the lexicographically smallest)."""
    b, S, Hq, D = q.shape
    g = Hq // k.shape[2]
    n = S // B
    sels = np.full((b, Hq, S, topk), -1, dtype=np.int32)
    for bb in range(b):
        for h in range(Hq):
            hk = h // g
            for t in range(S):
                j = t // B
                score = []
                for i in range(n):
                    tot = 0.0
                    for d in range(D):
                        col = [k[bb, s, hk, d] for s in range(i * B, (i + 1) * B)]
                        tot += q[bb, t, h, d] * (max(col) if q[bb, t, h, d] >= 0 else min(col))
                    score.append(tot)
                m = min(topk - 1, j)
                best = None
                for sub in itertools.combinations(range(j), m):
                    key = (sum(score[i] for i in sub), tuple(-i for i in sub))
                    if best is None or key > best[0]:
                        best = (key, sub)
                chosen = sorted(best[1] + (j,))
                sels[bb, h, t, :len(chosen)] = chosen
    return sels


@pytest.mark.parametrize("S,B,topk,Hq,Hkv", [(32, 4, 3, 2, 1), (24, 4, 4, 1, 1), (32, 8, 2, 2, 2)])
def test_minmax_gate_bruteforce_tiny(S, B, topk, Hq, Hkv):
    rng = np.random.default_rng(33 + S + B)
    q, k, v = rand_qkv(rng, 1, S, Hq, Hkv, 4)
    out, sel = O.moba_forward(q, k, v, B, topk, True, gate="minmax")
    assert np.array_equal(sel, brute_force_minmax_selection(q, k, B, topk))
    # the attention itself is the method's, given the selection
    ref = O.moba_rows(q, k, v, B, topk, True, [(0, t, h) for h in range(Hq) for t in range(S)],
                      given_sel=[sel[0, h, t] for h in range(Hq) for t in range(S)])
    got = np.stack([out[0, t, h] for h in range(Hq) for t in range(S)])
    assert np.max(np.abs(got - ref.out)) == 0.0


def test_minmax_gate_dense_and_shift_invariance():
    """With topk >= n the gate does not matter: dense causal attention; and
    K + c leaves every min/max score shifted by q.c, so nothing changes."""
    rng = np.random.default_rng(34)
    q, k, v = rand_qkv(rng, 1, 64, 2, 1, 8)
    out, _ = O.moba_forward(q, k, v, 16, 4, True, gate="minmax")
    dense, _ = O.moba_forward(q, k, v, 64, 1, True)
    assert np.max(np.abs(out - dense)) < 1e-12
    q, k, v = rand_qkv(rng, 1, 96, 2, 1, 8)
    out, sel = O.moba_forward(q, k, v, 16, 3, True, gate="minmax")
    c = rng.standard_normal(8)
    out2, sel2 = O.moba_forward(q, k + c, v, 16, 3, True, gate="minmax")
    assert np.array_equal(sel, sel2)
    assert np.max(np.abs(out - out2)) < 1e-9


def test_minmax_gate_finds_the_block_the_mean_hides():
    """One key of block 1 points along q while the rest cancel it (its mean
    is ~0); block 2 has a small positive mean.  The mean gate takes block 2,
    the min/max gate block 1."""
    D, B = 4, 4
    q = np.zeros((1, 4 * B, 1, D)); q[0, :, 0, 0] = 1.0
    k = np.zeros((1, 4 * B, 1, D))
    k[0, B + 0, 0, 0] = 3.0
    k[0, B + 1:2 * B, 0, 0] = -1.0
    k[0, 2 * B:3 * B, 0, 0] = 0.1
    v = np.random.default_rng(35).standard_normal((1, 4 * B, 1, D))
    t = 4 * B - 1  # own block 3; one past slot
    _, sel_mean = O.moba_forward(q, k, v, B, 2, True)
    _, sel_mm = O.moba_forward(q, k, v, B, 2, True, gate="minmax")
    assert list(sel_mean[0, 0, t]) == [2, 3]
    assert list(sel_mm[0, 0, t]) == [1, 3]


def test_planted_swapped_minmax_bounds_are_caught(monkeypatch):
    """A gate that takes the smaller product per dimension is a lower bound:
    the upper-bound pin must fail for it."""
    monkeypatch.setattr(O, "gate_scores_minmax",
                        lambda q, lo, hi: np.minimum(lo * q, hi * q).sum(axis=1))
    with pytest.raises(AssertionError):
        test_minmax_score_is_the_largest_logit_over_the_box()


# ----------------------------------------------------------------------------
# decode: one new query per sequence against its cache (prefill rule at t = L-1)
# ----------------------------------------------------------------------------
def _decode_case(rng, b, Lmax, Hq, Hkv, D):
    q = rng.standard_normal((b, Hq, D))
    kc = rng.standard_normal((b, Lmax, Hkv, D))
    vc = rng.standard_normal((b, Lmax, Hkv, D))
    return q, kc, vc


@pytest.mark.parametrize("lens,B,topk,Hq,Hkv", [
    ([1, 7, 16, 17], 16, 3, 2, 1), ([64, 63, 48, 33], 16, 2, 4, 2), ([80, 95, 96, 5], 16, 4, 2, 2),
    ([40, 41], 8, 20, 2, 1),
])
def test_decode_equals_prefill_last_row_with_any_future(lens, B, topk, Hq, Hkv):
    """Decode at cache length L is prefill row L-1 of a sequence padded to a
    whole number of blocks with arbitrary keys and values after L-1."""
    rng = np.random.default_rng(sum(lens) + B)
    b, D, Lmax = len(lens), 8, 96
    q, kc, vc = _decode_case(rng, b, Lmax, Hq, Hkv, D)
    res = O.decode_rows(q, kc, vc, lens, B, topk)
    for bb, L in enumerate(lens):
        S = -(-L // B) * B
        qp = rng.standard_normal((1, S, Hq, D))
        qp[0, L - 1] = q[bb]
        kp = rng.standard_normal((1, S, Hkv, D)) * 5.0
        vp = rng.standard_normal((1, S, Hkv, D)) * 5.0
        kp[0, :L], vp[0, :L] = kc[bb, :L], vc[bb, :L]
        pre = O.moba_rows(qp, kp, vp, B, topk, True, [(0, L - 1, h) for h in range(Hq)])
        for h in range(Hq):
            r = bb * Hq + h
            assert np.array_equal(res.sel[r], pre.sel[h])
            np.testing.assert_allclose(res.out[r], pre.out[h], rtol=0, atol=1e-12)


def test_decode_dense_and_own_block_only_match_sdpa():
    """topk >= number of blocks: softmax over all L cached keys; topk = 1: over
    the own block's keys jB..L-1 only (torch fp64 SDPA, one query)."""
    rng = np.random.default_rng(4)
    b, Lmax, Hq, Hkv, D, B = 3, 64, 4, 2, 8, 8
    q, kc, vc = _decode_case(rng, b, Lmax, Hq, Hkv, D)
    lens = [64, 37, 9]
    dense = O.decode_rows(q, kc, vc, lens, B, 8)
    own = O.decode_rows(q, kc, vc, lens, B, 1)
    for bb, L in enumerate(lens):
        j = (L - 1) // B
        for res, lo in ((dense, 0), (own, j * B)):
            ref = sdpa_fp64(q[bb][None, None], kc[bb, lo:L][None], vc[bb, lo:L][None])[0, 0]
            np.testing.assert_allclose(res.out[bb * Hq:(bb + 1) * Hq], ref, rtol=0, atol=1e-12)
        assert all(own.sel[bb * Hq + h].tolist() == [j] for h in range(Hq))


def test_decode_never_reads_past_the_cache_length():
    """Cache entries at positions >= L (stale or unwritten) never change the
    result: a decode that attended the own block in full would fail this."""
    rng = np.random.default_rng(12)
    b, Lmax, Hq, Hkv, D, B = 2, 48, 2, 1, 8, 16
    q, kc, vc = _decode_case(rng, b, Lmax, Hq, Hkv, D)
    lens = [21, 40]
    ref = O.decode_rows(q, kc, vc, lens, B, 2)
    kc2, vc2 = kc.copy(), vc.copy()
    for bb, L in enumerate(lens):
        kc2[bb, L:] = 100.0
        vc2[bb, L:] = -100.0
    got = O.decode_rows(q, kc2, vc2, lens, B, 2)
    assert np.array_equal(got.out, ref.out) and np.array_equal(got.sel, ref.sel)


def test_decode_selection_by_brute_force():
    """The chosen past blocks maximise the summed mean-key score among all
    min(k-1, j)-subsets of the complete blocks (explicit loops), ties to the
    lexicographically smallest subset."""
    rng = np.random.default_rng(21)
    b, Lmax, Hq, Hkv, D, B, topk = 2, 80, 2, 1, 4, 8, 4
    q, kc, vc = _decode_case(rng, b, Lmax, Hq, Hkv, D)
    lens = [80, 53]
    res = O.decode_rows(q, kc, vc, lens, B, topk)
    for bb, L in enumerate(lens):
        j = (L - 1) // B
        for h in range(Hq):
            score = []
            for i in range(j):
                s = 0.0
                for d in range(D):
                    tot = 0.0
                    for x in range(B):
                        tot += kc[bb, i * B + x, 0, d]
                    s += q[bb, h, d] * (tot / B)
                score.append(s)
            best, best_set = None, None
            for sub in itertools.combinations(range(j), min(topk - 1, j)):
                val = sum(score[i] for i in sub)
                if best is None or val > best + 1e-12:
                    best, best_set = val, sub
            want = list(best_set) + [j] + [-1] * (topk - 1 - len(best_set))
            assert res.sel[bb * Hq + h].tolist() == want


def test_decode_rejects_bad_lengths():
    rng = np.random.default_rng(1)
    q, kc, vc = _decode_case(rng, 1, 32, 2, 1, 4)
    for L in (0, 33):
        with pytest.raises(ValueError):
            O.decode_rows(q, kc, vc, [L], 8, 2)


# ----------------------------------------------------------------------------
# backward: gradients with the gate's choice held fixed
# ----------------------------------------------------------------------------
def _autograd_masked(q, k, v, dout, mask):
    """torch fp64 autograd of softmax(q k^T / sqrt(D) + log mask) v, with the
    KV heads expanded (query head h reads KV head h // g)."""
    Hq, Hkv = q.shape[2], k.shape[2]
    g = Hq // Hkv
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    qh = qt.permute(0, 2, 1, 3)
    kh = kt.permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    vh = vt.permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    logits = (qh @ kh.transpose(-1, -2)) / math.sqrt(q.shape[3])
    logits = logits.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.softmax(logits, dim=-1) @ vh
    (o.permute(0, 2, 1, 3) * torch.from_numpy(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _mask_from_sel(sel, S, B, causal):
    """[b, Hq, S, S] boolean mask of the keys each row attends, element by
    element from the chosen blocks (own block cut at the row itself)."""
    b, Hq = sel.shape[0], sel.shape[1]
    mask = np.zeros((b, Hq, S, S), dtype=bool)
    for bb in range(b):
        for h in range(Hq):
            for t in range(S):
                for i in sel[bb, h, t]:
                    if i < 0:
                        continue
                    for s in range(i * B, (i + 1) * B):
                        if not causal or s <= t:
                            mask[bb, h, t, s] = True
    return mask


@pytest.mark.parametrize("S,B,topk,Hq,Hkv,causal", [
    (64, 16, 2, 2, 1, True), (96, 16, 3, 4, 2, True), (48, 8, 4, 2, 2, True), (64, 16, 2, 2, 1, False),
])
def test_backward_equals_autograd_of_masked_attention(S, B, topk, Hq, Hkv, causal):
    rng = np.random.default_rng(S + B + topk)
    D = 8
    q, k, v = rand_qkv(rng, 1, S, Hq, Hkv, D)
    dout = rng.standard_normal(q.shape)
    _, sel = O.moba_forward(q, k, v, B, topk, causal)
    dq, dk, dv, lse = O.moba_backward(q, k, v, dout, B, topk, causal)
    mask = _mask_from_sel(sel, S, B, causal)
    rq, rk, rv = _autograd_masked(q, k, v, dout, mask)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)
    # lse: log-sum-exp of the row's scaled logits over the same mask
    logits = np.einsum("bthd,bshd->bhts", q, np.repeat(k, Hq // Hkv, axis=2)) / math.sqrt(D)
    ref_lse = np.log(np.where(mask, np.exp(logits), 0.0).sum(-1))
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_backward_dense_equals_sdpa_autograd():
    """Every block chosen: the gradients of dense causal attention (torch fp64
    SDPA autograd)."""
    rng = np.random.default_rng(77)
    b, S, Hq, Hkv, D, B = 2, 48, 4, 2, 8, 16
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    dout = rng.standard_normal(q.shape)
    dq, dk, dv, _ = O.moba_backward(q, k, v, dout, B, 3, True)
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    o = F.scaled_dot_product_attention(qt.permute(0, 2, 1, 3), kt.permute(0, 2, 1, 3).repeat_interleave(2, 1),
                                       vt.permute(0, 2, 1, 3).repeat_interleave(2, 1), is_causal=True)
    (o.permute(0, 2, 1, 3) * torch.from_numpy(dout)).sum().backward()
    for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-10)


def test_backward_matches_finite_differences():
    """Central differences of sum(dout * out) along random directions, with
    the selection held fixed (it is piecewise constant: checked unchanged)."""
    rng = np.random.default_rng(5)
    b, S, Hq, Hkv, D, B, topk = 1, 48, 2, 1, 8, 8, 3
    q, k, v = rand_qkv(rng, b, S, Hq, Hkv, D)
    dout = rng.standard_normal(q.shape)
    out0, sel0 = O.moba_forward(q, k, v, B, topk, True)
    dq, dk, dv, _ = O.moba_backward(q, k, v, dout, B, topk, True)
    eps = 1e-6
    for which in range(3):
        dirn = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
        dirn[which] = rng.standard_normal(dirn[which].shape)
        plus = [x + eps * d for x, d in zip((q, k, v), dirn)]
        minus = [x - eps * d for x, d in zip((q, k, v), dirn)]
        op, sp = O.moba_forward(*plus, B, topk, True)
        om, sm = O.moba_forward(*minus, B, topk, True)
        assert np.array_equal(sp, sel0) and np.array_equal(sm, sel0)
        fd = ((op - om) * dout).sum() / (2 * eps)
        an = (dq * dirn[0]).sum() + (dk * dirn[1]).sum() + (dv * dirn[2]).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def test_planted_backward_mistakes_are_caught(monkeypatch):
    """A backward without the delta term, or with the own block uncut, must
    fail the masked-autograd pin."""
    rng = np.random.default_rng(8)
    S, B, topk, D = 48, 16, 2, 8
    q, k, v = rand_qkv(rng, 1, S, 2, 1, D)
    dout = rng.standard_normal(q.shape)
    _, sel = O.moba_forward(q, k, v, B, topk, True)
    rq, rk, rv = _autograd_masked(q, k, v, dout, _mask_from_sel(sel, S, B, True))
    real = O.key_ranges

    def own_uncut(sel_, t, B_, causal):
        return real(sel_, (t // B_) * B_ + B_ - 1, B_, causal) if causal else real(sel_, t, B_, causal)

    monkeypatch.setattr(O, "key_ranges", own_uncut)
    dq, dk, dv, _ = O.moba_backward(q, k, v, dout, B, topk, True, sel_idx=sel)
    assert not np.allclose(dv, rv, atol=1e-6)
    monkeypatch.setattr(O, "key_ranges", real)
    dq, dk, dv, _ = O.moba_backward(q, k, v, dout, B, topk, True, sel_idx=sel)
    np.testing.assert_allclose(dv, rv, rtol=0, atol=1e-10)


def test_backward_dq_rows_equal_the_full_backward():
    """The per-row dq (for sampled checks at large sizes) is the full
    backward's dq, row by row, bit for bit up to summation order."""
    rng = np.random.default_rng(31)
    S, B, topk, D = 64, 16, 3, 8
    q, k, v = rand_qkv(rng, 2, S, 4, 2, D)
    dout = rng.standard_normal(q.shape)
    _, sel = O.moba_forward(q, k, v, B, topk, True)
    dq, _, _, lse = O.moba_backward(q, k, v, dout, B, topk, True, sel_idx=sel)
    rows = [(bb, t, h) for bb in range(2) for t in (0, 15, 16, 40, 63) for h in range(4)]
    got, gl = O.backward_dq_rows(q, k, v, dout, B, True, rows, [sel[bb, h, t] for (bb, t, h) in rows])
    for x, (bb, t, h) in enumerate(rows):
        np.testing.assert_allclose(got[x], dq[bb, t, h], rtol=0, atol=1e-12)
        assert abs(gl[x] - lse[bb, h, t]) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_backward_dkdv_keys_equal_the_full_backward(causal):
    """The per-key dk / dv (for sampled checks at large sizes) is the full
    backward's, key by key, up to summation order: keys in own blocks, in
    blocks chosen as past blocks, and in blocks nobody chose."""
    rng = np.random.default_rng(32)
    S, B, topk, D = 64, 16, 2, 8
    q, k, v = rand_qkv(rng, 2, S, 4, 2, D)
    dout = rng.standard_normal(q.shape)
    _, sel = O.moba_forward(q, k, v, B, topk, causal)
    _, dk, dv, _ = O.moba_backward(q, k, v, dout, B, topk, causal, sel_idx=sel)
    keys = [(bb, s, hk) for bb in range(2) for s in (0, 7, 15, 16, 31, 40, 47, 48, 63) for hk in range(2)]
    gk, gv = O.backward_dkdv_keys(q, k, v, dout, B, causal, keys, sel)
    for x, (bb, s, hk) in enumerate(keys):
        np.testing.assert_allclose(gk[x], dk[bb, s, hk], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gv[x], dv[bb, s, hk], rtol=0, atol=1e-12)
    # a key of the last block is attended only by its own rows at or after it
    assert np.abs(dk[:, 63]).max() > 0
