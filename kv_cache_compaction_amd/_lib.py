"""ctypes binding of libks.so.

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  torch provides device memory (outputs and workspaces) and the
current stream.  If libks.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libks.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "ks.h")

KS_OK = 0
KS_F32 = 0
KS_BF16 = 1
KS_NEVER = 0x7FFFFFFF
KS_BLOCK = 16

_STATUS = {1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "HIP_ERROR", 4: "WORKSPACE_TOO_SMALL"}


class KSError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "ks_last_error": ([], ctypes.c_char_p),
    "ks_version": ([], ctypes.c_char_p),
    "ks_rope_logical": ([_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp], _i),
    "ks_evict_attn_fwd_workspace": ([_i, _i, _i, _i, _i, _i], _sz),
    "ks_evict_attn_fwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _sz,
                           _vp], _i),
    "ks_evict_attn_bwd_workspace": ([_i, _i, _i, _i, _i, _i], _sz),
    "ks_evict_attn_bwd": ([_vp] * 10 + [_i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp], _i),
    "ks_evict_attn_fwd_rope_workspace": ([_i, _i, _i, _i, _i, _i], _sz),
    "ks_evict_attn_fwd_rope": ([_vp] * 9 + [_i, _i, _i, _i, _i, _i, _f, _f, _vp, _sz, _vp], _i),
    "ks_evict_attn_bwd_rope_workspace": ([_i, _i, _i, _i, _i, _i], _sz),
    "ks_evict_attn_bwd_rope": ([_vp] * 11 + [_i, _i, _i, _i, _i, _i, _f, _f, _vp, _sz, _vp], _i),
    "ks_compact_block_table": ([_vp] * 7 + [_i, _i, _vp], _i),
    "ks_compact_block_table_rounds": ([_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _vp], _i),
    "ks_paged_decode_workspace": ([_i, _i, _i, _i], _sz),
    "ks_paged_decode": ([_vp] * 7 + [_i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp], _i),
    "ks_paged_decode_noalloc_max_scratch": ([], _sz),
    "ks_paged_decode_noalloc": ([_vp] * 7 + [_i, _i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "ks_append_kv": ([_vp] * 7 + [_i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "ks_paged_decode_bs1_workspace": ([_i, _i, _i, _i], _sz),
    "ks_paged_decode_bs1": ([_vp] * 7 + [_i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp], _i),
    "ks_append_kv_bs1": ([_vp] * 7 + [_i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "ks_paged_decode_rope": ([_vp] * 8 + [_i] * 8 + [_f, _f, _vp, _sz, _vp], _i),
    "ks_check_eviction_record": ([_vp, _i, _i, _vp, _vp], _i),
    "ks_check_block_table": ([_vp, _vp, _i, _i, _i, _i, _vp, _vp], _i),
    # measurement aid (include/ks_measure.h)
    "ks_measure_mfma_flops": ([_i, _i], ctypes.c_double),
    "ks_measure_mfma_bf16": ([_vp, _vp, _i, _i, _vp], _i),
    "ks_measure_dq_atomics": ([_vp, _vp, _i, _i, _i, _i, _vp], _i),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libks.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build it with `python -m kv_cache_compaction_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions declared in include/ks.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ks_[a-z0-9_]+)\s*\(", text)))


def _check(fn, st):
    if st != KS_OK:
        msg = load_library().ks_last_error().decode(errors="replace")
        raise KSError(fn, st, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return KS_F32
    if t.dtype == torch.bfloat16:
        return KS_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _cuda_contig(name, t, dtype=None):
    _need(t.is_cuda, f"{name} must be a GPU tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")


def _given(name, t, shape, dtype):
    """A caller-supplied output: a contiguous GPU tensor of exactly this shape
    and dtype (the library writes through the raw pointer, so a smaller or
    strided buffer would be written past its end)."""
    _cuda_contig(name, t, dtype)
    _need(tuple(t.shape) == tuple(shape), f"{name} must be {list(shape)}, got {list(t.shape)}")
    return t


def _workspace(nbytes, device, ws):
    if ws is None:
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    _cuda_contig("ws", ws)
    _need(ws.numel() * ws.element_size() >= nbytes, "workspace too small")
    return ws


# ---------------------------------------------------------------------------
def ks_rope_logical(q, k, pos, base=10000.0, inverse=False, stream=None):
    """Rotate q [B,N,Hq,D] and/or k [B,N,Hkv,D] in place at positions pos [B,N]."""
    lib = load_library()
    ref = q if q is not None else k
    _need(ref is not None, "q or k required")
    B, N, _, D = ref.shape
    for name, t in (("q", q), ("k", k)):
        if t is not None:
            _cuda_contig(name, t, ref.dtype)
            _need(t.shape[0] == B and t.shape[1] == N and t.shape[3] == D, f"{name} shape")
    _cuda_contig("pos", pos, torch.int32)
    _need(tuple(pos.shape) == (B, N), "pos must be [B, N]")
    Hq = q.shape[2] if q is not None else 0
    Hkv = k.shape[2] if k is not None else 0
    st = lib.ks_rope_logical(_ptr(q), _ptr(k), _ptr(pos), B, N, Hq, Hkv, D, _dtype_code(ref),
                             float(base), int(bool(inverse)), _stream(stream))
    _check("ks_rope_logical", st)
    return q, k


def ks_evict_attn_fwd_workspace(B, N, Hq, Hkv, D, dtype_code):
    return load_library().ks_evict_attn_fwd_workspace(B, N, Hq, Hkv, D, dtype_code)


def ks_evict_attn_fwd(q, k, v, e, scale=None, out=None, lse=None, ws=None, stream=None):
    """Eviction-masked attention forward.  Returns (o, lse)."""
    lib = load_library()
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    _cuda_contig("q", q)
    _cuda_contig("k", k, q.dtype)
    _cuda_contig("v", v, q.dtype)
    _cuda_contig("e", e, torch.int32)
    _need(tuple(k.shape) == (B, N, Hkv, D) and tuple(v.shape) == (B, N, Hkv, D), "k/v shape")
    _need(tuple(e.shape) == (B, N), "e must be [B, N]")
    out = torch.empty_like(q) if out is None else _given("out", out, q.shape, q.dtype)
    lse = (torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None
           else _given("lse", lse, (B, Hq, N), torch.float32))
    code = _dtype_code(q)
    nbytes = lib.ks_evict_attn_fwd_workspace(B, N, Hq, Hkv, D, code)
    ws = _workspace(nbytes, q.device, ws)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.ks_evict_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(e), _ptr(out), _ptr(lse), B, N, Hq,
                               Hkv, D, code, sc, _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream))
    _check("ks_evict_attn_fwd", st)
    return out, lse


def ks_evict_attn_bwd_workspace(B, N, Hq, Hkv, D, dtype_code):
    return load_library().ks_evict_attn_bwd_workspace(B, N, Hq, Hkv, D, dtype_code)


def ks_evict_attn_bwd(q, k, v, e, o, lse, dout, scale=None, dq=None, dk=None, dv=None, ws=None,
                      stream=None):
    """Gradients of the masked forward.  Returns (dq, dk, dv)."""
    lib = load_library()
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _cuda_contig(name, t, q.dtype)
    _cuda_contig("e", e, torch.int32)
    _cuda_contig("lse", lse, torch.float32)
    _need(tuple(k.shape) == (B, N, Hkv, D) and tuple(v.shape) == (B, N, Hkv, D), "k/v shape")
    _need(tuple(e.shape) == (B, N), "e must be [B, N]")
    _need(tuple(o.shape) == tuple(q.shape) and tuple(dout.shape) == tuple(q.shape), "o/dout")
    _need(tuple(lse.shape) == (B, Hq, N), "lse must be [B, Hq, N]")
    dq = torch.empty_like(q) if dq is None else _given("dq", dq, q.shape, q.dtype)
    dk = torch.empty_like(k) if dk is None else _given("dk", dk, k.shape, q.dtype)
    dv = torch.empty_like(v) if dv is None else _given("dv", dv, v.shape, q.dtype)
    code = _dtype_code(q)
    nbytes = lib.ks_evict_attn_bwd_workspace(B, N, Hq, Hkv, D, code)
    ws = _workspace(nbytes, q.device, ws)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.ks_evict_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(e), _ptr(o), _ptr(lse),
                               _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, N, Hq, Hkv, D, code,
                               sc, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("ks_evict_attn_bwd", st)
    return dq, dk, dv


def ks_evict_attn_fwd_rope(q, k, v, e, pos, base=10000.0, scale=None, q_rot=None, k_rot=None,
                           out=None, lse=None, ws=None, stream=None):
    """RoPE at logical positions fused into the masked forward; q and k are
    unrotated and left unchanged.  Returns (o, lse, q_rot, k_rot)."""
    lib = load_library()
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    _cuda_contig("q", q)
    _cuda_contig("k", k, q.dtype)
    _cuda_contig("v", v, q.dtype)
    _cuda_contig("e", e, torch.int32)
    _cuda_contig("pos", pos, torch.int32)
    _need(tuple(k.shape) == (B, N, Hkv, D) and tuple(v.shape) == (B, N, Hkv, D), "k/v shape")
    _need(tuple(e.shape) == (B, N) and tuple(pos.shape) == (B, N), "e/pos must be [B, N]")
    q_rot = torch.empty_like(q) if q_rot is None else _given("q_rot", q_rot, q.shape, q.dtype)
    k_rot = torch.empty_like(k) if k_rot is None else _given("k_rot", k_rot, k.shape, q.dtype)
    out = torch.empty_like(q) if out is None else _given("out", out, q.shape, q.dtype)
    lse = (torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None
           else _given("lse", lse, (B, Hq, N), torch.float32))
    code = _dtype_code(q)
    nbytes = lib.ks_evict_attn_fwd_rope_workspace(B, N, Hq, Hkv, D, code)
    ws = _workspace(nbytes, q.device, ws)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.ks_evict_attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(e), _ptr(pos), _ptr(q_rot),
                                    _ptr(k_rot), _ptr(out), _ptr(lse), B, N, Hq, Hkv, D, code, sc,
                                    float(base), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream))
    _check("ks_evict_attn_fwd_rope", st)
    return out, lse, q_rot, k_rot


def ks_evict_attn_bwd_rope(q_rot, k_rot, v, e, pos, o, lse, dout, base=10000.0, scale=None,
                           dq=None, dk=None, dv=None, ws=None, stream=None):
    """Gradients of ks_evict_attn_fwd_rope with respect to the unrotated q and
    k (and v).  Returns (dq, dk, dv)."""
    lib = load_library()
    B, N, Hq, D = q_rot.shape
    Hkv = k_rot.shape[2]
    for name, t in (("q_rot", q_rot), ("k_rot", k_rot), ("v", v), ("o", o), ("dout", dout)):
        _cuda_contig(name, t, q_rot.dtype)
    _cuda_contig("e", e, torch.int32)
    _cuda_contig("pos", pos, torch.int32)
    _cuda_contig("lse", lse, torch.float32)
    _need(tuple(k_rot.shape) == (B, N, Hkv, D) and tuple(v.shape) == (B, N, Hkv, D),
          "k/v shape")
    _need(tuple(e.shape) == (B, N) and tuple(pos.shape) == (B, N), "e/pos must be [B, N]")
    _need(tuple(o.shape) == tuple(q_rot.shape) and tuple(dout.shape) == tuple(q_rot.shape),
          "o/dout")
    _need(tuple(lse.shape) == (B, Hq, N), "lse must be [B, Hq, N]")
    dq = torch.empty_like(q_rot) if dq is None else _given("dq", dq, q_rot.shape, q_rot.dtype)
    dk = torch.empty_like(k_rot) if dk is None else _given("dk", dk, k_rot.shape, q_rot.dtype)
    dv = torch.empty_like(v) if dv is None else _given("dv", dv, v.shape, q_rot.dtype)
    code = _dtype_code(q_rot)
    nbytes = lib.ks_evict_attn_bwd_rope_workspace(B, N, Hq, Hkv, D, code)
    ws = _workspace(nbytes, q_rot.device, ws)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.ks_evict_attn_bwd_rope(_ptr(q_rot), _ptr(k_rot), _ptr(v), _ptr(e), _ptr(pos),
                                    _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                    B, N, Hq, Hkv, D, code, sc, float(base), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream))
    _check("ks_evict_attn_bwd_rope", st)
    return dq, dk, dv


def ks_compact_block_table(table_in, nblk_in, keep, table_out=None, nblk_out=None, pos_in=None,
                           pos_out=None, stream=None):
    """Splice dropped blocks out of each table row.  Returns (table_out, nblk_out, pos_out)."""
    lib = load_library()
    B, MB = table_in.shape
    _cuda_contig("table_in", table_in, torch.int32)
    _cuda_contig("nblk_in", nblk_in, torch.int32)
    _cuda_contig("keep", keep, torch.uint8)
    _need(tuple(keep.shape) == (B, MB) and tuple(nblk_in.shape) == (B,), "keep/nblk shape")
    table_out = (torch.empty_like(table_in) if table_out is None
                 else _given("table_out", table_out, (B, MB), torch.int32))
    nblk_out = (torch.empty_like(nblk_in) if nblk_out is None
                else _given("nblk_out", nblk_out, (B,), torch.int32))
    if pos_in is not None:
        _given("pos_in", pos_in, (B, MB), torch.int32)
        pos_out = (torch.empty_like(pos_in) if pos_out is None
                   else _given("pos_out", pos_out, (B, MB), torch.int32))
    else:
        _need(pos_out is None, "pos_out given without pos_in")
    st = lib.ks_compact_block_table(_ptr(table_in), _ptr(nblk_in), _ptr(keep), _ptr(table_out),
                                    _ptr(nblk_out), _ptr(pos_in), _ptr(pos_out), B, MB,
                                    _stream(stream))
    _check("ks_compact_block_table", st)
    return table_out, nblk_out, pos_out


def ks_compact_block_table_rounds(table_in, nblk_in, keeps, table_out=None, nblk_out=None,
                                  pos_in=None, pos_out=None, stream=None):
    """Apply R compaction events at once; keeps is uint8 [R, B, max_blocks], event r
    indexing the table left by events 0..r-1.  Returns (table_out, nblk_out, pos_out)."""
    lib = load_library()
    B, MB = table_in.shape
    _cuda_contig("table_in", table_in, torch.int32)
    _cuda_contig("nblk_in", nblk_in, torch.int32)
    _cuda_contig("keeps", keeps, torch.uint8)
    _need(keeps.dim() == 3 and tuple(keeps.shape[1:]) == (B, MB) and
          tuple(nblk_in.shape) == (B,), "keeps/nblk shape")
    table_out = (torch.empty_like(table_in) if table_out is None
                 else _given("table_out", table_out, (B, MB), torch.int32))
    nblk_out = (torch.empty_like(nblk_in) if nblk_out is None
                else _given("nblk_out", nblk_out, (B,), torch.int32))
    if pos_in is not None:
        _given("pos_in", pos_in, (B, MB), torch.int32)
        pos_out = (torch.empty_like(pos_in) if pos_out is None
                   else _given("pos_out", pos_out, (B, MB), torch.int32))
    else:
        _need(pos_out is None, "pos_out given without pos_in")
    st = lib.ks_compact_block_table_rounds(_ptr(table_in), _ptr(nblk_in), _ptr(keeps),
                                           keeps.shape[0], _ptr(table_out), _ptr(nblk_out),
                                           _ptr(pos_in), _ptr(pos_out), B, MB, _stream(stream))
    _check("ks_compact_block_table_rounds", st)
    return table_out, nblk_out, pos_out


def ks_paged_decode_workspace(B, Hq, D, max_blocks):
    return load_library().ks_paged_decode_workspace(B, Hq, D, max_blocks)


def ks_paged_decode(q, k_pool, v_pool, table, seq_lens, scale=None, out=None, lse=None, ws=None,
                    stream=None):
    """One GQA decode step over paged caches.  Returns (out, lse)."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(k_pool.dim() == 4, "pool must be [NB, Hkv, 16, D]")
    NB, Hkv, BS, Dp = k_pool.shape
    _need(BS == KS_BLOCK and Dp == D, "pool must be [NB, Hkv, 16, D] with q's D")
    _cuda_contig("q", q)
    _cuda_contig("k_pool", k_pool, q.dtype)
    _cuda_contig("v_pool", v_pool, q.dtype)
    _cuda_contig("table", table, torch.int32)
    _cuda_contig("seq_lens", seq_lens, torch.int32)
    _need(tuple(v_pool.shape) == tuple(k_pool.shape), "v_pool shape")
    _need(table.shape[0] == B and tuple(seq_lens.shape) == (B,), "table/seq_lens shape")
    MB = table.shape[1]
    out = torch.empty_like(q) if out is None else _given("out", out, q.shape, q.dtype)
    lse = (torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None
           else _given("lse", lse, (B, Hq), torch.float32))
    nbytes = lib.ks_paged_decode_workspace(B, Hq, D, MB)
    ws = _workspace(nbytes, q.device, ws)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.ks_paged_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(table), _ptr(seq_lens),
                             _ptr(out), _ptr(lse), B, Hq, Hkv, D, MB, NB, _dtype_code(q), sc,
                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("ks_paged_decode", st)
    return out, lse


def ks_paged_decode_noalloc_max_scratch():
    return load_library().ks_paged_decode_noalloc_max_scratch()


def ks_paged_decode_noalloc(q, k_pool, v_pool, table, seq_lens, scale=None, out=None, lse=None,
                            stream=None):
    """ks_paged_decode with the library's own per-GPU scratch (no workspace).
    Returns (out, lse); pass out and lse to keep the call allocation-free."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(k_pool.dim() == 4, "pool must be [NB, Hkv, 16, D]")
    NB, Hkv, BS, Dp = k_pool.shape
    _need(BS == KS_BLOCK and Dp == D, "pool must be [NB, Hkv, 16, D] with q's D")
    _cuda_contig("q", q)
    _cuda_contig("k_pool", k_pool, q.dtype)
    _cuda_contig("v_pool", v_pool, q.dtype)
    _cuda_contig("table", table, torch.int32)
    _cuda_contig("seq_lens", seq_lens, torch.int32)
    _need(tuple(v_pool.shape) == tuple(k_pool.shape), "v_pool shape")
    _need(table.shape[0] == B and tuple(seq_lens.shape) == (B,), "table/seq_lens shape")
    MB = table.shape[1]
    out = torch.empty_like(q) if out is None else _given("out", out, q.shape, q.dtype)
    lse = (torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None
           else _given("lse", lse, (B, Hq), torch.float32))
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.ks_paged_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(table),
                                     _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, D, MB, NB,
                                     _dtype_code(q), sc, _stream(stream))
    _check("ks_paged_decode_noalloc", st)
    return out, lse


def ks_append_kv(k_new, v_new, pos, table, seq_lens, k_pool, v_pool, base=10000.0,
                 stream=None):
    """Rotate k_new [B, Hkv, D] at pos [B] and write it and v_new into pool
    slot seq_lens[b] - 1 of every sequence (in place on the pools)."""
    lib = load_library()
    B, Hkv, D = k_new.shape
    NB = k_pool.shape[0]
    _cuda_contig("k_new", k_new)
    _cuda_contig("v_new", v_new, k_new.dtype)
    _cuda_contig("k_pool", k_pool, k_new.dtype)
    _cuda_contig("v_pool", v_pool, k_new.dtype)
    _cuda_contig("pos", pos, torch.int32)
    _cuda_contig("table", table, torch.int32)
    _cuda_contig("seq_lens", seq_lens, torch.int32)
    _need(tuple(v_new.shape) == (B, Hkv, D), "v_new shape")
    _need(tuple(k_pool.shape) == (NB, Hkv, KS_BLOCK, D) and v_pool.shape == k_pool.shape,
          "pool shape")
    _need(tuple(pos.shape) == (B,) and tuple(seq_lens.shape) == (B,) and table.shape[0] == B,
          "pos/seq_lens/table shape")
    st = lib.ks_append_kv(_ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(table), _ptr(seq_lens),
                          _ptr(k_pool), _ptr(v_pool), B, Hkv, D, table.shape[1], NB,
                          _dtype_code(k_new), float(base), _stream(stream))
    _check("ks_append_kv", st)


def ks_paged_decode_bs1_workspace(B, Hq, D, max_tokens):
    return load_library().ks_paged_decode_bs1_workspace(B, Hq, D, max_tokens)


def ks_paged_decode_bs1(q, k_pool, v_pool, token_table, seq_lens, scale=None, out=None,
                        lse=None, ws=None, stream=None):
    """One GQA decode step over single-token-block caches: pools
    [slots, Hkv, D], token_table [B, max_tokens].  Returns (out, lse)."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(k_pool.dim() == 3 and k_pool.shape[2] == D, "pool must be [slots, Hkv, D] with q's D")
    NT, Hkv, _ = k_pool.shape
    _cuda_contig("q", q)
    _cuda_contig("k_pool", k_pool, q.dtype)
    _cuda_contig("v_pool", v_pool, q.dtype)
    _cuda_contig("token_table", token_table, torch.int32)
    _cuda_contig("seq_lens", seq_lens, torch.int32)
    _need(tuple(v_pool.shape) == tuple(k_pool.shape), "v_pool shape")
    _need(token_table.shape[0] == B and tuple(seq_lens.shape) == (B,),
          "token_table/seq_lens shape")
    MT = token_table.shape[1]
    out = torch.empty_like(q) if out is None else _given("out", out, q.shape, q.dtype)
    lse = (torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None
           else _given("lse", lse, (B, Hq), torch.float32))
    nbytes = lib.ks_paged_decode_bs1_workspace(B, Hq, D, MT)
    ws = _workspace(nbytes, q.device, ws)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.ks_paged_decode_bs1(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(token_table),
                                 _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, D, MT, NT,
                                 _dtype_code(q), sc, _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check("ks_paged_decode_bs1", st)
    return out, lse


def ks_append_kv_bs1(k_new, v_new, pos, token_table, seq_lens, k_pool, v_pool, base=10000.0,
                     stream=None):
    """Rotate k_new [B, Hkv, D] at pos [B] and write it and v_new into slot
    token_table[b, seq_lens[b] - 1] of the single-token-block pools."""
    lib = load_library()
    B, Hkv, D = k_new.shape
    NT = k_pool.shape[0]
    _cuda_contig("k_new", k_new)
    _cuda_contig("v_new", v_new, k_new.dtype)
    _cuda_contig("k_pool", k_pool, k_new.dtype)
    _cuda_contig("v_pool", v_pool, k_new.dtype)
    _cuda_contig("pos", pos, torch.int32)
    _cuda_contig("token_table", token_table, torch.int32)
    _cuda_contig("seq_lens", seq_lens, torch.int32)
    _need(tuple(v_new.shape) == (B, Hkv, D), "v_new shape")
    _need(tuple(k_pool.shape) == (NT, Hkv, D) and v_pool.shape == k_pool.shape, "pool shape")
    _need(tuple(pos.shape) == (B,) and tuple(seq_lens.shape) == (B,)
          and token_table.shape[0] == B, "pos/seq_lens/token_table shape")
    st = lib.ks_append_kv_bs1(_ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(token_table),
                              _ptr(seq_lens), _ptr(k_pool), _ptr(v_pool), B, Hkv, D,
                              token_table.shape[1], NT, _dtype_code(k_new), float(base),
                              _stream(stream))
    _check("ks_append_kv_bs1", st)


def ks_check_eviction_record(e, bad=None, stream=None):
    """Per trace, the number of tokens j with e[b, j] <= j (int32 [B] on the device)."""
    lib = load_library()
    _cuda_contig("e", e, torch.int32)
    _need(e.dim() == 2, "e must be [B, N]")
    B, N = e.shape
    bad = (torch.empty(B, dtype=torch.int32, device=e.device) if bad is None
           else _given("bad", bad, (B,), torch.int32))
    _check("ks_check_eviction_record",
           lib.ks_check_eviction_record(_ptr(e), B, N, _ptr(bad), _stream(stream)))
    return bad


def ks_check_block_table(table, seq_lens, num_pool_blocks, block_size=KS_BLOCK, bad=None,
                         stream=None):
    """Per sequence, the number of table entries a decode would reach that are not
    pool indices, plus one if seq_lens[b] is negative or past the row."""
    lib = load_library()
    _cuda_contig("table", table, torch.int32)
    _cuda_contig("seq_lens", seq_lens, torch.int32)
    B, MB = table.shape
    _need(tuple(seq_lens.shape) == (B,), "seq_lens shape")
    bad = (torch.empty(B, dtype=torch.int32, device=table.device) if bad is None
           else _given("bad", bad, (B,), torch.int32))
    _check("ks_check_block_table",
           lib.ks_check_block_table(_ptr(table), _ptr(seq_lens), B, MB, int(num_pool_blocks),
                                    int(block_size), _ptr(bad), _stream(stream)))
    return bad


def ks_paged_decode_rope(q, pos, k_pool, v_pool, table, seq_lens, base=10000.0, scale=None,
                         out=None, lse=None, ws=None, stream=None):
    """Paged decode of the UNROTATED query q [B, Hq, D], rotated inside the kernel
    at pos [B].  Pools [NB, Hkv, 16, D] (16-token blocks) or [slots, Hkv, D]
    (single-token blocks).  Returns (out, lse); q is not modified."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(k_pool.shape[-1] == D, "pool head dim must equal q's D")
    if k_pool.dim() == 4:
        NP, Hkv, BS, _ = k_pool.shape
        _need(BS == KS_BLOCK, "pool block size must be 16")
    else:
        _need(k_pool.dim() == 3, "pool must be [NB, Hkv, 16, D] or [slots, Hkv, D]")
        NP, Hkv, _ = k_pool.shape
        BS = 1
    _cuda_contig("q", q)
    _cuda_contig("pos", pos, torch.int32)
    _cuda_contig("k_pool", k_pool, q.dtype)
    _cuda_contig("v_pool", v_pool, q.dtype)
    _cuda_contig("table", table, torch.int32)
    _cuda_contig("seq_lens", seq_lens, torch.int32)
    _need(tuple(v_pool.shape) == tuple(k_pool.shape), "v_pool shape")
    _need(table.shape[0] == B and tuple(seq_lens.shape) == (B,) and tuple(pos.shape) == (B,),
          "table/seq_lens/pos shape")
    ME = table.shape[1]
    out = torch.empty_like(q) if out is None else _given("out", out, q.shape, q.dtype)
    lse = (torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None
           else _given("lse", lse, (B, Hq), torch.float32))
    nbytes = (lib.ks_paged_decode_workspace(B, Hq, D, ME) if BS == KS_BLOCK
              else lib.ks_paged_decode_bs1_workspace(B, Hq, D, ME))
    ws = _workspace(nbytes, q.device, ws)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib.ks_paged_decode_rope(_ptr(q), _ptr(pos), _ptr(k_pool), _ptr(v_pool), _ptr(table),
                                  _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, D, ME, NP,
                                  BS, _dtype_code(q), sc, float(base), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check("ks_paged_decode_rope", st)
    return out, lse



def ks_measure_mfma_flops(workgroups, iters):
    return load_library().ks_measure_mfma_flops(workgroups, iters)


def ks_measure_mfma_bf16(seed, sink, workgroups, iters, stream=None):
    """Measurement aid: a loop of bf16 MFMAs only (include/ks_measure.h).
    seed: >= 1024 bf16 values; sink: >= workgroups * 512 floats."""
    lib = load_library()
    _cuda_contig("seed", seed, torch.bfloat16)
    _cuda_contig("sink", sink, torch.float32)
    _need(seed.numel() >= 1024 and sink.numel() >= workgroups * 512, "seed/sink too small")
    _check("ks_measure_mfma_bf16",
           lib.ks_measure_mfma_bf16(_ptr(seed), _ptr(sink), workgroups, iters, _stream(stream)))


def ks_measure_dq_atomics(acc, cend, Hkv, stream=None):
    """Measurement aid: the fp32 atomic dQ adds of a single-pass backward
    (include/ks_measure.h).  acc: fp32 [B, N, Hq, 128]; cend: int32
    [B, ceil(N / 256)]."""
    lib = load_library()
    B, N, Hq, Dd = acc.shape
    _need(Dd == 128 and Hq % Hkv == 0, "acc must be [B, N, Hq, 128]")
    _cuda_contig("acc", acc, torch.float32)
    _cuda_contig("cend", cend, torch.int32)
    _need(tuple(cend.shape) == (B, (N + 255) // 256), "cend shape")
    _check("ks_measure_dq_atomics",
           lib.ks_measure_dq_atomics(_ptr(acc), _ptr(cend), B, N, Hq, Hkv, _stream(stream)))
