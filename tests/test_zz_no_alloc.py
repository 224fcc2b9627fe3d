"""moba_attn_fwd_noalloc (the forward on the library's fixed per-GPU scratch,
for callers that cannot allocate) through the C ABI, against moba_attn_fwd.

With a caller workspace of the scratch's size, moba_attn_fwd plans the same
query chunks and runs the same kernels, so the two agree bit for bit; with
its default workspace the selection is the same and the outputs agree within
the bf16 tolerance of the forward's parity tests (2e-2)."""
import sys

import pytest
import torch

import block_sparse_attention_40_amd as M
import moba_workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_against_fwd(w):
    dt = M.DTYPE_BF16 if w.dtype == "bf16" else M.DTYPE_F32
    cb = M.plan_chunk_blocks(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, dt, w.block_size,
                             w.topk, w.causal, M.NOALLOC_SCRATCH_BYTES)
    say(f"[case] noalloc {w}: {cb} of {w.num_blocks} blocks per chunk")
    q, k, v, _ = W.make_inputs(w, device=DEV)
    out_n, sel_n = M.moba_attn_fwd_noalloc(q, k, v, w.block_size, w.topk, w.causal)
    ws = torch.empty(M.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=DEV)
    out_w, sel_w = M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal, workspace=ws)
    del ws
    out_d, sel_d = M.moba_attn_fwd(q, k, v, w.block_size, w.topk, w.causal)
    torch.cuda.synchronize()
    assert torch.equal(sel_n, sel_w), "selection differs from moba_attn_fwd on an equal workspace"
    assert torch.equal(out_n, out_w), "output differs from moba_attn_fwd on an equal workspace"
    assert torch.equal(sel_n, sel_d), "selection differs from moba_attn_fwd"
    err = (out_n.float() - out_d.float()).abs().max().item()
    say(f"[noalloc] {w.name}: bit-exact against the equal workspace; max |diff| {err:.3e} against the default")
    assert err <= (2e-2 if w.dtype == "bf16" else 1e-4)


def test_noalloc_matches_fwd_on_two_calls_the_second_smaller():
    # 32K positions, 32 heads, block 512, top-3: the default workspace (546
    # MiB) exceeds the scratch, so the fixed-scratch call runs in two chunks
    check_against_fwd(W.WORKLOADS["mha32_32k_needle"])
    # then a smaller call on the scratch the first one left behind
    check_against_fwd(W.Workload("noalloc_small", "bf16", 1, 4, 2, 2048, 128, 256, 3, seed=5))


def test_noalloc_one_block_chunks_without_slice_images():
    # 128K positions, 32/8 heads, block 4096, top-12: only one query block per
    # chunk fits, and only with K and V read as they are (no slice images)
    w = W.WORKLOADS["gqa32x8_128k"]
    assert M.plan_chunk_blocks(w.batch, w.seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, M.DTYPE_BF16,
                               w.block_size, w.topk, w.causal, M.NOALLOC_SCRATCH_BYTES) == 1
    check_against_fwd(w)
    # and an fp32 call after it
    check_against_fwd(W.WORKLOADS["tiny_f32_1k"])
