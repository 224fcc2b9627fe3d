"""The C-ABI library without a GPU: it loads, exports every function that
include/moba.h declares, and rejects invalid arguments on the host with the
documented status codes before anything is launched."""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_attention_40_amd as M
from block_sparse_attention_40_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moba.h")

OK, NULL, DTYPE, HEAD_DIM, SEQ, TOPK, GQA, WS, HIP, SHAPE, ALIGN = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10
BF16, F32 = 1, 0


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moba_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert "moba_attn_fwd" in names and "moba_workspace_bytes" in names
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in moba.h but not exported"
        assert n in _lib.SIGNATURES, f"{n} has no Python binding"
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings_and_version():
    assert M.version() >= 100
    for st in (OK, NULL, DTYPE, HEAD_DIM, SEQ, TOPK, GQA, WS, HIP, SHAPE, ALIGN):
        assert M.status_string(st) and M.status_string(st) != "unknown status"
    assert M.status_string(12345) == "unknown status"


def ws(b=1, S=1024, Hq=4, Hkv=2, D=128, dt=BF16, B=128, k=3, causal=1):
    out = ctypes.c_size_t(0)
    st = _lib.lib.moba_workspace_bytes(b, S, Hq, Hkv, D, dt, B, k, causal, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,want", [
    (dict(), OK),
    (dict(S=1000, B=128), SEQ),
    (dict(k=0), TOPK),
    (dict(k=-3), TOPK),
    (dict(Hq=6, Hkv=4), GQA),
    (dict(Hq=256, Hkv=1), GQA),
    (dict(dt=7), DTYPE),
    (dict(D=64), HEAD_DIM),          # bf16 needs 128
    (dict(dt=F32, D=96), HEAD_DIM),
    (dict(dt=F32, D=64), OK),
    (dict(b=0), SHAPE),
    (dict(S=0), SHAPE),
    (dict(B=0), SHAPE),
    (dict(S=1 << 20, B=64), SHAPE),  # 16384 blocks: more than the gate's LDS counters
    (dict(S=8192, B=64, k=40), TOPK),  # 127 past candidates, 39 to choose: above the maximum
    (dict(S=8192, B=64, k=33), OK),
    (dict(S=8192, B=64, k=128), OK),  # every causal block: no ranking needed
    (dict(S=8192, B=64, k=500), OK),  # clamped
])
def test_workspace_validation(kw, want):
    st, nbytes = ws(**kw)
    assert st == want
    if st == OK:
        assert nbytes > 0


def test_workspace_grows_with_work_and_chunks_the_partials():
    _, small = ws(S=1024)
    _, big = ws(S=8192)
    assert big > small
    # 1M tokens, 32/8 heads, block 4096, top-12: the partial buffer is chunked
    # so the workspace stays far below the unchunked ~190 GB
    st, w1m = ws(S=1 << 20, Hq=32, Hkv=8, B=4096, k=12)
    assert st == OK and w1m < 12 * (1 << 30)
    # top-1: no partials at all
    _, w_top1 = ws(S=1 << 20, Hq=32, Hkv=8, B=4096, k=1)
    assert w_top1 < w1m


FAKE = 1 << 20  # 16-byte aligned fake device addresses: never dereferenced on an error path


def call_fwd(q=FAKE, k=FAKE, v=FAKE, out=FAKE, sel=None, wsp=FAKE, wsb=None, **kw):
    a = dict(b=1, S=1024, Hq=4, Hkv=2, D=128, dt=BF16, B=128, topk=3, causal=1)
    a.update(kw)
    if wsb is None:
        st, wsb = ws(a["b"], a["S"], a["Hq"], a["Hkv"], a["D"], a["dt"], a["B"], a["topk"], a["causal"])
    return _lib.lib.moba_attn_fwd(q, k, v, a["b"], a["S"], a["Hq"], a["Hkv"], a["D"], a["dt"], a["B"],
                                  a["topk"], a["causal"], out, sel, wsp, wsb, None)


def test_fwd_rejects_bad_arguments_before_launching():
    assert call_fwd(q=None) == NULL
    assert call_fwd(out=None) == NULL
    assert call_fwd(wsp=None) == WS
    assert call_fwd(wsb=16) == WS
    assert call_fwd(q=FAKE + 8) == ALIGN
    assert call_fwd(sel=FAKE + 2) == ALIGN
    assert call_fwd(S=1000) == SEQ
    assert call_fwd(topk=0) == TOPK
    assert call_fwd(Hq=3) == GQA
    assert call_fwd(D=64) == HEAD_DIM
    assert call_fwd(dt=5) == DTYPE


def test_stage_entry_points_reject_bad_arguments():
    L = _lib.lib
    assert L.moba_meanpool(None, 1, 1024, 2, 128, BF16, 128, FAKE, None) == NULL
    assert L.moba_meanpool(FAKE, 1, 1000, 2, 128, BF16, 128, FAKE, None) == SEQ
    assert L.moba_meanpool(FAKE + 4, 1, 1024, 2, 128, BF16, 128, FAKE, None) == ALIGN
    assert L.moba_gate(FAKE, None, 1, 1024, 4, 2, 128, BF16, 128, 3, 1, FAKE, None) == NULL
    assert L.moba_gate(FAKE, FAKE, 1, 1024, 4, 2, 128, BF16, 128, 0, 1, FAKE, None) == TOPK
    assert L.moba_gate(FAKE, FAKE, 1, 1024, 4, 3, 128, BF16, 128, 3, 1, FAKE, None) == GQA


def call_fwd_gate(gate_kind, q=FAKE, out=FAKE, **kw):
    a = dict(b=1, S=1024, Hq=4, Hkv=2, D=128, dt=BF16, B=128, topk=3, causal=1)
    a.update(kw)
    st, wsb = ws(a["b"], a["S"], a["Hq"], a["Hkv"], a["D"], a["dt"], a["B"], a["topk"], a["causal"])
    return _lib.lib.moba_attn_fwd_gate(q, FAKE, FAKE, a["b"], a["S"], a["Hq"], a["Hkv"], a["D"], a["dt"], a["B"],
                                       a["topk"], a["causal"], gate_kind, out, None, FAKE, wsb, None)


def test_gate_kind_entry_point_rejects_bad_arguments():
    assert _lib.GATE_KINDS == {"mean": 0, "minmax": 1}
    assert call_fwd_gate(2) == SHAPE
    assert call_fwd_gate(-1) == SHAPE
    for kind in (0, 1):
        assert call_fwd_gate(kind, q=None) == NULL
        assert call_fwd_gate(kind, out=FAKE + 4) == ALIGN
        assert call_fwd_gate(kind, S=1000) == SEQ
        assert call_fwd_gate(kind, topk=0) == TOPK
    L = _lib.lib
    assert L.moba_minmaxpool(None, 1, 1024, 2, 128, BF16, 128, FAKE, None) == NULL
    assert L.moba_minmaxpool(FAKE, 1, 1000, 2, 128, BF16, 128, FAKE, None) == SEQ
    assert L.moba_minmaxpool(FAKE, 1, 1024, 2, 128, BF16, 128, FAKE + 4, None) == ALIGN


def test_python_binding_rejects_unknown_gate():
    with pytest.raises(ValueError):
        M.moba_attn_fwd(torch.zeros(1), torch.zeros(1), torch.zeros(1), 128, 3, gate="max")


def dws(b=2, L=4096, Hq=8, Hkv=2, D=128, dt=BF16, B=128, k=4):
    out = ctypes.c_size_t(0)
    st = _lib.lib.moba_decode_workspace_bytes(b, L, Hq, Hkv, D, dt, B, k, ctypes.byref(out))
    return st, out.value


def test_decode_workspace_validation():
    st, n = dws()
    assert st == OK and n > 0
    assert dws(dt=7)[0] == DTYPE
    assert dws(D=64)[0] == HEAD_DIM
    assert dws(dt=0, D=64)[0] == OK
    assert dws(Hq=6, Hkv=4)[0] == GQA
    assert dws(Hq=34, Hkv=2)[0] == GQA  # group of 17 > 16
    assert dws(k=0)[0] == TOPK and dws(k=65)[0] == TOPK and dws(k=64)[0] == OK
    assert dws(L=4000)[0] == SEQ
    assert dws(L=16385 * 64, B=64)[0] == SHAPE  # more than 16384 blocks
    # partials grow with topk and the block size; scores with the capacity
    assert dws(k=12)[1] > dws(k=4)[1]
    assert dws(L=1 << 20, B=4096, k=12)[1] < 64 << 20


def test_decode_entry_points_reject_bad_arguments():
    L = _lib.lib
    st, n = dws()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4096, 8, 2, 128, BF16, 128, 4, FAKE, None, FAKE, n, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.moba_decode_fwd(*a)

    assert call(a0=None) == NULL
    assert call(a3=None) == NULL  # mu_cache
    assert call(a4=None) == NULL  # cache_lens
    assert call(a15=None) == WS
    assert call(a16=n - 1) == WS
    assert call(a1=FAKE + 8) == ALIGN
    assert call(a4=FAKE + 2) == ALIGN
    assert call(a12=0) == TOPK
    assert call(a6=4000) == SEQ
    assert L.moba_decode_means(None, FAKE, 2, 4096, 2, 128, BF16, 128, FAKE, None) == NULL
    assert L.moba_decode_means(FAKE, FAKE, 2, 4000, 2, 128, BF16, 128, FAKE, None) == SEQ
    assert L.moba_decode_means(FAKE, FAKE, 2, 4096, 2, 128, BF16, 128, FAKE + 4, None) == ALIGN
