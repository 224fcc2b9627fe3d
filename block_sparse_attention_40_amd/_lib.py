"""ctypes binding of the MoBA C ABI (include/moba.h).

Argument marshalling only: every step of the forward runs in the HIP kernels
of libmoba.so.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoba.so")

MOBA_OK = 0
DTYPE_F32 = 0
DTYPE_BF16 = 1
NOALLOC_SCRATCH_BYTES = 512 << 20  # MOBA_NOALLOC_SCRATCH_BYTES

_c_i64, _c_i32, _c_p, _c_sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes), one entry per function declared in include/moba.h
SIGNATURES = {
    "moba_version": (ctypes.c_int, []),
    "moba_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moba_workspace_bytes": (ctypes.c_int, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                            _c_i32, ctypes.POINTER(_c_sz)]),
    "moba_workspace_bytes_chunked": (ctypes.c_int, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                    _c_i32, _c_i32, _c_i64, ctypes.POINTER(_c_sz)]),
    "moba_plan_info": (ctypes.c_int, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_sz,
                                      ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32)]),
    "moba_attn_fwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                     _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "moba_attn_fwd_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                             _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
    "moba_attn_fwd_gate": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                          _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "moba_minmaxpool": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p]),
    "moba_meanpool": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p]),
    "moba_gate": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                 _c_i32, _c_p, _c_p]),
    "moba_decode_workspace_bytes": (ctypes.c_int, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                   _c_i32, ctypes.POINTER(_c_sz)]),
    "moba_decode_fwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                       _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "moba_decode_means": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p]),
    "moba_attn_fwd_train": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "moba_bwd_workspace_bytes": (ctypes.c_int, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                _c_i32, ctypes.POINTER(_c_sz)]),
    "moba_attn_bwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32,
                                     _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "moba_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "moba_profile_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_i64),
                                         ctypes.POINTER(ctypes.c_double), _c_i32]),
}

# gate kinds (enum moba_gate_kind)
GATE_KINDS = {"mean": 0, "minmax": 1}

STAGES = ("meanpool", "gate", "dispatch", "attn_past", "attn_own", "attn_f32", "kv_layout",
          "decode_gate", "decode_attn", "decode_merge", "bwd_prep", "bwd_dkdv", "bwd_dq")


class MobaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run block_sparse_attention_40_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.moba_status_string(int(status)).decode()


def version() -> int:
    return int(lib.moba_version())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_dev(*ts: torch.Tensor):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_shape(t: torch.Tensor, name: str, shape, dtype: torch.dtype):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _check_on(t: torch.Tensor, name: str, device: torch.device):
    _check_dev(t)
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_like(t: torch.Tensor, name: str, shape, dtype: torch.dtype, device: torch.device):
    """t must be a contiguous GPU tensor of exactly this shape and dtype on
    `device` (the C ABI derives every extent from q, so a mismatched tensor
    would be read or written out of bounds)."""
    _check_shape(t, name, shape, dtype)
    _check_on(t, name, device)


def _check_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    """q [b, S, Hq, D]; k, v [b, S, Hkv, D] with Hq a multiple of Hkv, one
    dtype and one device.  Returns (b, S, Hq, Hkv, D)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [batch, seqlen, heads, head_dim]")
    b, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"num_q_heads {Hq} must be a multiple of num_kv_heads {Hkv}")
    _check_shape(k, "k", (b, S, Hkv, D), q.dtype)
    _check_shape(v, "v", (b, S, Hkv, D), q.dtype)
    _check_dev(q)
    _check_on(k, "k", q.device)
    _check_on(v, "v", q.device)
    return b, S, Hq, Hkv, D


def workspace_bytes(batch: int, seqlen: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    dtype: int, block_size: int, topk: int, causal: bool = True, max_chunk_blocks: int = 0) -> int:
    """Forward workspace bytes; max_chunk_blocks > 0 limits the query blocks
    per chunk (1 gives the smallest workspace the forward accepts)."""
    out = _c_sz(0)
    st = lib.moba_workspace_bytes_chunked(batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size,
                                          topk, int(bool(causal)), int(max_chunk_blocks), ctypes.byref(out))
    if st != MOBA_OK:
        raise MobaError(st, "moba_workspace_bytes_chunked")
    return int(out.value)


def plan_info(batch: int, seqlen: int, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: int,
              block_size: int, topk: int, causal: bool, workspace_bytes_: int) -> dict:
    """The forward's plan with a workspace of that size: query blocks per
    chunk, rows per past-block tile, whether K/V slice images are built."""
    cb, tr, img = _c_i64(0), _c_i32(0), _c_i32(0)
    st = lib.moba_plan_info(batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk,
                            int(bool(causal)), int(workspace_bytes_), ctypes.byref(cb), ctypes.byref(tr),
                            ctypes.byref(img))
    if st != MOBA_OK:
        raise MobaError(st, "moba_plan_info")
    return {"chunk_blocks": int(cb.value), "tile_rows": int(tr.value), "slice_images": bool(img.value)}


def plan_chunk_blocks(*args) -> int:
    """Query blocks per chunk the forward runs with a workspace of that size
    (same arguments as plan_info)."""
    return plan_info(*args)["chunk_blocks"]


def _workspace(workspace: Optional[torch.Tensor], nbytes, device: torch.device) -> torch.Tensor:
    """The caller's workspace (checked to be on `device`), or a new one of
    nbytes() bytes.  The C ABI checks its size."""
    if workspace is None:
        return torch.empty(nbytes(), dtype=torch.uint8, device=device)
    _check_dev(workspace)
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}")
    return workspace


def moba_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_size: int, topk: int,
                  causal: bool = True, out: Optional[torch.Tensor] = None,
                  sel_idx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  return_sel: bool = True, gate: str = "mean") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """MoBA prefill forward.  q [b, S, Hq, D], k/v [b, S, Hkv, D] (bf16 with
    D = 128, or fp32 with D in {64, 128}).  Returns (out, sel_idx) where
    sel_idx is [b, Hq, S, topk] int32 (None if return_sel is False and no
    sel_idx tensor was passed).  gate: "mean" (block means) or "minmax"
    (element-wise key min / max per block, score = largest q.k over the box);
    "mean" calls moba_attn_fwd, "minmax" moba_attn_fwd_gate."""
    if gate not in GATE_KINDS:
        raise ValueError(f"gate must be one of {sorted(GATE_KINDS)}")
    b, S, Hq, Hkv, D = _check_qkv(q, k, v)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _check_like(out, "out", q.shape, q.dtype, q.device)
    if sel_idx is None and return_sel:
        sel_idx = torch.empty((b, Hq, S, topk), dtype=torch.int32, device=q.device)
    if sel_idx is not None:
        _check_like(sel_idx, "sel_idx", (b, Hq, S, topk), torch.int32, q.device)
    # a caller's workspace may be smaller than the default: the forward then
    # runs in more query chunks
    workspace = _workspace(workspace, lambda: workspace_bytes(b, S, Hq, Hkv, D, dt, block_size, topk, causal),
                           q.device)
    sel_ptr = sel_idx.data_ptr() if sel_idx is not None else None
    ws_len = workspace.numel() * workspace.element_size()
    if gate == "mean":
        st = lib.moba_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, S, Hq, Hkv, D, dt, block_size, topk,
                               int(bool(causal)), out.data_ptr(), sel_ptr, workspace.data_ptr(), ws_len,
                               _stream_ptr(q.device))
        where = "moba_attn_fwd"
    else:
        st = lib.moba_attn_fwd_gate(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, S, Hq, Hkv, D, dt, block_size,
                                    topk, int(bool(causal)), GATE_KINDS[gate], out.data_ptr(), sel_ptr,
                                    workspace.data_ptr(), ws_len, _stream_ptr(q.device))
        where = "moba_attn_fwd_gate"
    if st != MOBA_OK:
        raise MobaError(st, where)
    return out, sel_idx


def moba_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_size: int, topk: int,
                          causal: bool = True, out: Optional[torch.Tensor] = None,
                          sel_idx: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """moba_attn_fwd_noalloc: the forward on the library's fixed per-GPU
    scratch (no workspace; the C call allocates nothing).  Pass out and
    sel_idx to allocate nothing here either."""
    b, S, Hq, Hkv, D = _check_qkv(q, k, v)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _check_like(out, "out", q.shape, q.dtype, q.device)
    if sel_idx is None:
        sel_idx = torch.empty((b, Hq, S, topk), dtype=torch.int32, device=q.device)
    _check_like(sel_idx, "sel_idx", (b, Hq, S, topk), torch.int32, q.device)
    st = lib.moba_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, S, Hq, Hkv, D, dt, block_size, topk,
                                   int(bool(causal)), out.data_ptr(), sel_idx.data_ptr(), _stream_ptr(q.device))
    if st != MOBA_OK:
        raise MobaError(st, "moba_attn_fwd_noalloc")
    return out, sel_idx


def profile_enable(on: bool = True) -> None:
    lib.moba_profile_enable(int(bool(on)))


def profile_read() -> dict:
    """Per stage: summed kernel ms (HIP events on the launch stream), number
    of launches and summed algorithmic work (FLOPs or bytes); clears them."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    launches = (_c_i64 * n)()
    work = (ctypes.c_double * n)()
    st = lib.moba_profile_read(ms, launches, work, n)
    if st != MOBA_OK:
        raise MobaError(st, "moba_profile_read")
    return {name: {"ms": ms[i], "launches": int(launches[i]), "work": work[i]} for i, name in enumerate(STAGES)}


def moba_meanpool(k: torch.Tensor, block_size: int, mu: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block means of the keys: mu [b, Hkv, S / block_size, D] fp32."""
    b, S, Hkv, D = k.shape
    shape = (b, Hkv, S // max(block_size, 1), D)
    if mu is not None:
        _check_shape(mu, "mu", shape, torch.float32)
    _check_dev(k)
    if mu is None:
        mu = torch.empty(shape, dtype=torch.float32, device=k.device)
    _check_on(mu, "mu", k.device)
    st = lib.moba_meanpool(k.data_ptr(), b, S, Hkv, D, _dtype_code(k), block_size, mu.data_ptr(),
                           _stream_ptr(k.device))
    if st != MOBA_OK:
        raise MobaError(st, "moba_meanpool")
    return mu


def moba_minmaxpool(k: torch.Tensor, block_size: int, lohi: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Element-wise key min and max per block: lohi [b, Hkv, S / block_size,
    2, D] fp32 (index 0 the min, 1 the max)."""
    b, S, Hkv, D = k.shape
    shape = (b, Hkv, S // max(block_size, 1), 2, D)
    if lohi is not None:
        _check_shape(lohi, "lohi", shape, torch.float32)
    _check_dev(k)
    if lohi is None:
        lohi = torch.empty(shape, dtype=torch.float32, device=k.device)
    _check_on(lohi, "lohi", k.device)
    st = lib.moba_minmaxpool(k.data_ptr(), b, S, Hkv, D, _dtype_code(k), block_size, lohi.data_ptr(),
                             _stream_ptr(k.device))
    if st != MOBA_OK:
        raise MobaError(st, "moba_minmaxpool")
    return lohi


def moba_gate(q: torch.Tensor, mu: torch.Tensor, block_size: int, topk: int, causal: bool = True,
              sel_idx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gate and top-k: sel_idx [b, Hq, S, topk] int32 from q and block means."""
    if q.dim() != 4 or mu.dim() != 4:
        raise ValueError("q must be [b, S, Hq, D] and mu [b, Hkv, S / block_size, D]")
    b, S, Hq, D = q.shape
    Hkv = mu.shape[1]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"num_q_heads {Hq} must be a multiple of mu's num_kv_heads {Hkv}")
    _check_like(mu, "mu", (b, Hkv, S // max(block_size, 1), D), torch.float32, q.device)
    _check_dev(q)
    if sel_idx is None:
        sel_idx = torch.empty((b, Hq, S, topk), dtype=torch.int32, device=q.device)
    _check_like(sel_idx, "sel_idx", (b, Hq, S, topk), torch.int32, q.device)
    st = lib.moba_gate(q.data_ptr(), mu.data_ptr(), b, S, Hq, Hkv, D, _dtype_code(q), block_size, topk,
                       int(bool(causal)), sel_idx.data_ptr(), _stream_ptr(q.device))
    if st != MOBA_OK:
        raise MobaError(st, "moba_gate")
    return sel_idx


MAX_DECODE_TOPK = 64
MAX_DECODE_GROUP = 16
DECODE_CHUNK = 512  # keys per decode attention work-group (one partial per head, slot and chunk)


def decode_workspace_bytes(batch: int, max_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           dtype: int, block_size: int, topk: int) -> int:
    out = _c_sz(0)
    st = lib.moba_decode_workspace_bytes(batch, max_len, num_q_heads, num_kv_heads, head_dim, dtype, block_size,
                                         topk, ctypes.byref(out))
    if st != MOBA_OK:
        raise MobaError(st, "moba_decode_workspace_bytes")
    return int(out.value)


def moba_decode_means(k_cache: torch.Tensor, cache_lens: torch.Tensor, block_size: int,
                      mu_cache: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mean key of every complete block of every cached sequence:
    mu_cache [b, Hkv, max_len / block_size, D] fp32 (entries of incomplete or
    unused blocks are left as they are; a new tensor starts at zero)."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [batch, max_len, Hkv, D]")
    b, Lmax, Hkv, D = k_cache.shape
    dt = _dtype_code(k_cache)
    shape = (b, Hkv, Lmax // max(block_size, 1), D)
    _check_shape(cache_lens, "cache_lens", (b,), torch.int32)
    if mu_cache is not None:
        _check_shape(mu_cache, "mu_cache", shape, torch.float32)
    _check_dev(k_cache)
    _check_on(cache_lens, "cache_lens", k_cache.device)
    if mu_cache is None:
        mu_cache = torch.zeros(shape, dtype=torch.float32, device=k_cache.device)
    _check_on(mu_cache, "mu_cache", k_cache.device)
    st = lib.moba_decode_means(k_cache.data_ptr(), cache_lens.data_ptr(), b, Lmax, Hkv, D, dt,
                               block_size, mu_cache.data_ptr(), _stream_ptr(k_cache.device))
    if st != MOBA_OK:
        raise MobaError(st, "moba_decode_means")
    return mu_cache


def moba_decode_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, mu_cache: torch.Tensor,
                    cache_lens: torch.Tensor, block_size: int, topk: int, out: Optional[torch.Tensor] = None,
                    sel_idx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    return_sel: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One MoBA decode step.  q [b, Hq, D]; k_cache / v_cache [b, max_len,
    Hkv, D]; mu_cache fp32 [b, Hkv, max_len / block_size, D] (moba_decode_means,
    kept current by this call); cache_lens int32 [b] (the new token included).
    Returns (out [b, Hq, D], sel_idx [b, Hq, topk] int32 or None)."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [batch, Hq, D] and k_cache [batch, max_len, Hkv, D]")
    b, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"num_q_heads {Hq} must be a multiple of num_kv_heads {Hkv}")
    dt = _dtype_code(q)
    # every extent the C ABI uses comes from q and k_cache: check the rest
    _check_shape(k_cache, "k_cache", (b, Lmax, Hkv, D), q.dtype)
    _check_shape(v_cache, "v_cache", (b, Lmax, Hkv, D), q.dtype)
    _check_shape(mu_cache, "mu_cache", (b, Hkv, Lmax // max(block_size, 1), D), torch.float32)
    _check_shape(cache_lens, "cache_lens", (b,), torch.int32)
    _check_dev(q)
    for t_, name in ((k_cache, "k_cache"), (v_cache, "v_cache"), (mu_cache, "mu_cache"), (cache_lens, "cache_lens")):
        _check_on(t_, name, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_like(out, "out", q.shape, q.dtype, q.device)
    if sel_idx is None and return_sel:
        sel_idx = torch.empty((b, Hq, topk), dtype=torch.int32, device=q.device)
    if sel_idx is not None:
        _check_like(sel_idx, "sel_idx", (b, Hq, topk), torch.int32, q.device)
    workspace = _workspace(workspace, lambda: decode_workspace_bytes(b, Lmax, Hq, Hkv, D, dt, block_size, topk),
                           q.device)
    st = lib.moba_decode_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), mu_cache.data_ptr(),
                             cache_lens.data_ptr(), b, Lmax, Hq, Hkv, D, dt, block_size, topk, out.data_ptr(),
                             sel_idx.data_ptr() if sel_idx is not None else None, workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _stream_ptr(q.device))
    if st != MOBA_OK:
        raise MobaError(st, "moba_decode_fwd")
    return out, sel_idx


def moba_attn_fwd_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_size: int, topk: int,
                        causal: bool = True, workspace: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Forward for training: (out, sel_idx [b, Hq, S, topk] int32, lse [b, Hq,
    S] fp32, natural log of the row's sum of exp of the scaled logits)."""
    b, S, Hq, Hkv, D = _check_qkv(q, k, v)
    dt = _dtype_code(q)
    out = torch.empty_like(q)
    sel = torch.empty((b, Hq, S, topk), dtype=torch.int32, device=q.device)
    lse = torch.empty((b, Hq, S), dtype=torch.float32, device=q.device)
    workspace = _workspace(workspace, lambda: workspace_bytes(b, S, Hq, Hkv, D, dt, block_size, topk, causal),
                           q.device)
    st = lib.moba_attn_fwd_train(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, S, Hq, Hkv, D, dt, block_size, topk,
                                 int(bool(causal)), out.data_ptr(), sel.data_ptr(), lse.data_ptr(),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream_ptr(q.device))
    if st != MOBA_OK:
        raise MobaError(st, "moba_attn_fwd_train")
    return out, sel, lse


def bwd_workspace_bytes(batch: int, seqlen: int, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: int,
                        block_size: int, topk: int, causal: bool = True) -> int:
    out = _c_sz(0)
    st = lib.moba_bwd_workspace_bytes(batch, seqlen, num_q_heads, num_kv_heads, head_dim, dtype, block_size, topk,
                                      int(bool(causal)), ctypes.byref(out))
    if st != MOBA_OK:
        raise MobaError(st, "moba_bwd_workspace_bytes")
    return int(out.value)


def moba_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                  lse: torch.Tensor, sel_idx: torch.Tensor, block_size: int, topk: int, causal: bool = True,
                  workspace: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward with the forward's selection held fixed: (dq, dk, dv)."""
    b, S, Hq, Hkv, D = _check_qkv(q, k, v)
    _check_like(out, "out", q.shape, q.dtype, q.device)
    _check_like(dout, "dout", q.shape, q.dtype, q.device)
    _check_like(lse, "lse", (b, Hq, S), torch.float32, q.device)
    _check_like(sel_idx, "sel_idx", (b, Hq, S, topk), torch.int32, q.device)
    dt = _dtype_code(q)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    workspace = _workspace(workspace, lambda: bwd_workspace_bytes(b, S, Hq, Hkv, D, dt, block_size, topk, causal),
                           q.device)
    st = lib.moba_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                           lse.data_ptr(), sel_idx.data_ptr(), b, S, Hq, Hkv, D, dt, block_size, topk,
                           int(bool(causal)), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), _stream_ptr(q.device))
    if st != MOBA_OK:
        raise MobaError(st, "moba_attn_bwd")
    return dq, dk, dv
