"""Python binding of the C ABI in ``include/nsa.h`` (``libnsa.so``).

Argument marshalling only: every function checks tensor dtypes, devices and shapes,
allocates outputs and workspaces with PyTorch (device memory and streams are all PyTorch
is used for), and calls the library on the current stream.  No computation happens
here, and there is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .configs import NSAConfig

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnsa.so")

(OP_COMPRESS, OP_SCORE_SELECT, OP_SPARSE_ATTN, OP_DECODE, OP_FULL_ATTN, OP_SPARSE_BWD, OP_COMPRESS_BWD,
 OP_PREFILL) = range(8)
STATUS = {0: "ok", 1: "null", 2: "shape", 3: "unsupported", 4: "workspace", 5: "hip"}


class NSAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"nsa status {status} ({STATUS.get(status, '?')}): {detail}")
        self.status = status
        self.detail = detail


class CConfig(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32)] + [(n, ctypes.c_int32) for n in (
        "batch", "seq_len", "num_kv_heads", "heads_per_group", "d_k", "d_v", "cmp_block", "cmp_stride",
        "slc_block", "top_n", "n_init", "n_local", "window", "phi", "score_mode", "branches")] + [
        ("softmax_scale", ctypes.c_float)]


def c_config(cfg: NSAConfig, **over) -> CConfig:
    c = CConfig()
    c.struct_size = over.get("struct_size", ctypes.sizeof(CConfig))
    for f, _ in CConfig._fields_[1:]:
        setattr(c, f, over.get(f, getattr(cfg, f)))
    return c


_lib = None
_P = ctypes.c_void_p


def lib(build_if_missing: bool = True):
    """Load libnsa.so (building it first if it is absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            if not build_if_missing:
                raise RuntimeError(f"{LIB_PATH} is not built")
            from .build import build
            build()
        L = ctypes.CDLL(LIB_PATH)
        cp = ctypes.POINTER(CConfig)
        L.nsa_workspace_size.argtypes = [cp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        L.nsa_compress.argtypes = [cp] + [_P] * 9 + [ctypes.c_size_t, _P]
        L.nsa_score_select.argtypes = [cp] + [_P] * 7 + [ctypes.c_size_t, _P]
        L.nsa_select_from_scores.argtypes = [cp, _P, _P, _P]
        L.nsa_sparse_attn_fwd.argtypes = [cp] + [_P] * 8 + [ctypes.c_size_t, _P]
        L.nsa_decode.argtypes = [cp] + [_P] * 10 + [ctypes.c_size_t, _P]
        L.nsa_decode_noalloc.argtypes = [cp] + [_P] * 10
        L.nsa_prefill_fwd.argtypes = [cp] + [_P] * 11 + [ctypes.c_size_t, _P]
        L.nsa_full_attn_fwd.argtypes = [cp] + [_P] * 5 + [ctypes.c_size_t, _P]
        L.nsa_compress_prepare.argtypes = [cp] + [_P] * 5 + [ctypes.c_size_t, _P]
        L.nsa_cache_append.argtypes = [cp, _P, _P, ctypes.c_int32] + [_P] * 6 + [ctypes.c_size_t, _P]
        L.nsa_sparse_attn_bwd.argtypes = [cp] + [_P] * 19 + [ctypes.c_size_t, _P]
        L.nsa_sparse_attn_fwd_train.argtypes = [cp] + [_P] * 10 + [ctypes.c_size_t, _P]
        L.nsa_compress_bwd.argtypes = [cp] + [_P] * 15 + [ctypes.c_size_t, _P]
        for f in ("nsa_workspace_size", "nsa_compress", "nsa_score_select", "nsa_select_from_scores",
                  "nsa_sparse_attn_fwd", "nsa_decode", "nsa_decode_noalloc", "nsa_full_attn_fwd", "nsa_compress_prepare",
                  "nsa_prefill_fwd",
                  "nsa_cache_append"):
            getattr(L, f).restype = ctypes.c_int
        L.nsa_status_string.argtypes = [ctypes.c_int]
        L.nsa_status_string.restype = ctypes.c_char_p
        L.nsa_last_error_detail.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise NSAError(rc, lib().nsa_last_error_detail().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def workspace_size(cfg: NSAConfig, op: int, **over) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().nsa_workspace_size(ctypes.byref(c_config(cfg, **over)), op, ctypes.byref(n)))
    return int(n.value)


def _workspace(cfg, op, device, workspace=None, **over):
    need = workspace_size(cfg, op, **over)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return workspace, workspace.numel()


# ---------------------------------------------------------------------------
def compress(cfg: NSAConfig, K, V=None, w_k=None, w_v=None, pe_k=None, pe_v=None, *, seq_len=None,
             out_k=None, out_v=None, workspace=None, stream=None):
    """nsa_compress.  K [B,Hkv,T,dk] bf16 (T = cfg.seq_len unless ``seq_len`` is given).
    Returns (K_cmp, V_cmp) ([B,Hkv,N,d] bf16; V_cmp is None in mean mode)."""
    T = cfg.seq_len if seq_len is None else seq_len
    c = cfg.replace(seq_len=T)
    B, Hkv, dk, dv = c.batch, c.num_kv_heads, c.d_k, c.d_v
    N = c.n_cmp
    _need(K, "K", torch.bfloat16, (B, Hkv, T, dk))
    dev = K.device
    if out_k is None:
        out_k = torch.empty((B, Hkv, N, dk), dtype=torch.bfloat16, device=dev)
    _need(out_k, "out_k", torch.bfloat16, (B, Hkv, N, dk))
    if c.phi == 0:
        _need(V, "V", torch.bfloat16, (B, Hkv, T, dv))
        _need(w_k, "w_k", torch.bfloat16, (c.cmp_block * dk, dk))
        _need(w_v, "w_v", torch.bfloat16, (c.cmp_block * dv, dv))
        _need(pe_k, "pe_k", torch.bfloat16, (c.cmp_block, dk))
        _need(pe_v, "pe_v", torch.bfloat16, (c.cmp_block, dv))
        if out_v is None:
            out_v = torch.empty((B, Hkv, N, dv), dtype=torch.bfloat16, device=dev)
        _need(out_v, "out_v", torch.bfloat16, (B, Hkv, N, dv))
    else:
        out_v = None
    ws, nws = _workspace(c, OP_COMPRESS, dev, workspace)
    _check(lib().nsa_compress(ctypes.byref(c_config(c)), _ptr(K), _ptr(V), _ptr(w_k), _ptr(w_v), _ptr(pe_k),
                              _ptr(pe_v), _ptr(out_k), _ptr(out_v), _ptr(ws), nws, _stream(stream)))
    return out_k, out_v


def score_select(cfg: NSAConfig, Q, K_cmp, V_cmp=None, *, want_lse=False, want_ocmp=True, sel=None, lse=None,
                 o_cmp=None, workspace=None, stream=None):
    """nsa_score_select.  Returns (sel [B,T,Hkv,n] int32, lse [B,T,H] fp32 or None, o_cmp fp32 or None)."""
    B, T, H, Hkv = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads
    _need(Q, "Q", torch.bfloat16, (B, T, H, cfg.d_k))
    _need(K_cmp, "K_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_k))
    dev = Q.device
    mean = cfg.score_mode == 1
    if sel is None:
        sel = torch.empty((B, T, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    _need(sel, "sel", torch.int32, (B, T, Hkv, cfg.top_n))
    if want_lse and not mean and lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    if want_ocmp and not mean:
        _need(V_cmp, "V_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_v))
        if o_cmp is None:
            o_cmp = torch.empty((B, T, H, cfg.d_v), dtype=torch.float32, device=dev)
        _need(o_cmp, "o_cmp", torch.float32, (B, T, H, cfg.d_v))
    else:
        o_cmp = None
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, T, H))
    ws, nws = _workspace(cfg, OP_SCORE_SELECT, dev, workspace)
    _check(lib().nsa_score_select(ctypes.byref(c_config(cfg)), _ptr(Q), _ptr(K_cmp), _ptr(V_cmp if o_cmp is not None else None),
                                  _ptr(sel), _ptr(lse), _ptr(o_cmp), _ptr(ws), nws, _stream(stream)))
    return sel, lse, o_cmp


def select_from_scores(cfg: NSAConfig, scores, *, sel=None, stream=None):
    """nsa_select_from_scores.  scores [B,T,Hkv,N_slc] fp32 -> sel [B,T,Hkv,n] int32."""
    B, T, Hkv = cfg.batch, cfg.seq_len, cfg.num_kv_heads
    _need(scores, "scores", torch.float32, (B, T, Hkv, cfg.n_slc))
    if sel is None:
        sel = torch.empty((B, T, Hkv, cfg.top_n), dtype=torch.int32, device=scores.device)
    _need(sel, "sel", torch.int32, (B, T, Hkv, cfg.top_n))
    _check(lib().nsa_select_from_scores(ctypes.byref(c_config(cfg)), _ptr(scores), _ptr(sel), _stream(stream)))
    return sel


def sparse_attn_fwd(cfg: NSAConfig, Q, K, V, sel=None, o_cmp=None, gates=None, *, out=None, workspace=None,
                    stream=None):
    """nsa_sparse_attn_fwd.  Returns O [B,T,H,dv] bf16."""
    B, T, H, Hkv = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads
    _need(Q, "Q", torch.bfloat16, (B, T, H, cfg.d_k))
    _need(K, "K", torch.bfloat16, (B, Hkv, T, cfg.d_k))
    _need(V, "V", torch.bfloat16, (B, Hkv, T, cfg.d_v))
    if cfg.branches & 2:
        _need(sel, "sel", torch.int32, (B, T, Hkv, cfg.top_n))
    if cfg.branches & 1:
        _need(o_cmp, "o_cmp", torch.float32, (B, T, H, cfg.d_v))
    if gates is not None:
        _need(gates, "gates", torch.float32, (B, T, H, 3))
    if out is None:
        out = torch.empty((B, T, H, cfg.d_v), dtype=torch.bfloat16, device=Q.device)
    _need(out, "out", torch.bfloat16, (B, T, H, cfg.d_v))
    ws, nws = _workspace(cfg, OP_SPARSE_ATTN, Q.device, workspace)
    _check(lib().nsa_sparse_attn_fwd(ctypes.byref(c_config(cfg)), _ptr(Q), _ptr(K), _ptr(V),
                                     _ptr(sel if cfg.branches & 2 else None), _ptr(o_cmp if cfg.branches & 1 else None),
                                     _ptr(gates), _ptr(out), _ptr(ws), nws, _stream(stream)))
    return out


def full_attn_fwd(cfg: NSAConfig, Q, K, V, *, out=None, workspace=None, stream=None):
    """nsa_full_attn_fwd (dense causal attention).  Returns O [B,T,H,dv] bf16."""
    B, T, H, Hkv = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads
    _need(Q, "Q", torch.bfloat16, (B, T, H, cfg.d_k))
    _need(K, "K", torch.bfloat16, (B, Hkv, T, cfg.d_k))
    _need(V, "V", torch.bfloat16, (B, Hkv, T, cfg.d_v))
    if out is None:
        out = torch.empty((B, T, H, cfg.d_v), dtype=torch.bfloat16, device=Q.device)
    _need(out, "out", torch.bfloat16, (B, T, H, cfg.d_v))
    ws, nws = _workspace(cfg, OP_FULL_ATTN, Q.device, workspace)
    _check(lib().nsa_full_attn_fwd(ctypes.byref(c_config(cfg)), _ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(ws), nws,
                                   _stream(stream)))
    return out


def decode(cfg: NSAConfig, q, K_cache, V_cache, cache_len, K_cmp, V_cmp, gates=None, *, out=None, sel=None,
           want_sel=True, workspace=None, stream=None):
    """nsa_decode.  Returns (O [B,H,dv] bf16, sel [B,Hkv,n] int32 or None)."""
    B, L, H, Hkv = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads
    _need(q, "q", torch.bfloat16, (B, H, cfg.d_k))
    _need(K_cache, "K_cache", torch.bfloat16, (B, Hkv, L, cfg.d_k))
    _need(V_cache, "V_cache", torch.bfloat16, (B, Hkv, L, cfg.d_v))
    _need(cache_len, "cache_len", torch.int32, (B,))
    _need(K_cmp, "K_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_k))
    _need(V_cmp, "V_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_v))
    if gates is not None:
        _need(gates, "gates", torch.float32, (B, H, 3))
    if out is None:
        out = torch.empty((B, H, cfg.d_v), dtype=torch.bfloat16, device=q.device)
    if want_sel and sel is None:
        sel = torch.empty((B, Hkv, cfg.top_n), dtype=torch.int32, device=q.device)
    ws, nws = _workspace(cfg, OP_DECODE, q.device, workspace)
    _check(lib().nsa_decode(ctypes.byref(c_config(cfg)), _ptr(q), _ptr(K_cache), _ptr(V_cache), _ptr(cache_len),
                            _ptr(K_cmp), _ptr(V_cmp), _ptr(gates), _ptr(out), _ptr(sel), _ptr(ws), nws,
                            _stream(stream)))
    return out, sel


def decode_noalloc(cfg: NSAConfig, q, K_cache, V_cache, cache_len, K_cmp, V_cmp, gates=None, *, out, sel=None,
                   stream=None):
    """nsa_decode_noalloc: nsa_decode with the library's fixed device scratch instead of a
    workspace.  The caller passes the output ``out`` [B,H,dv] bf16 (and optionally ``sel``
    [B,Hkv,n] int32); nothing is allocated here either.  Returns (out, sel)."""
    B, L, H, Hkv = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads
    _need(q, "q", torch.bfloat16, (B, H, cfg.d_k))
    _need(K_cache, "K_cache", torch.bfloat16, (B, Hkv, L, cfg.d_k))
    _need(V_cache, "V_cache", torch.bfloat16, (B, Hkv, L, cfg.d_v))
    _need(cache_len, "cache_len", torch.int32, (B,))
    _need(K_cmp, "K_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_k))
    _need(V_cmp, "V_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_v))
    if gates is not None:
        _need(gates, "gates", torch.float32, (B, H, 3))
    _need(out, "out", torch.bfloat16, (B, H, cfg.d_v))
    if sel is not None:
        _need(sel, "sel", torch.int32, (B, Hkv, cfg.top_n))
    _check(lib().nsa_decode_noalloc(ctypes.byref(c_config(cfg)), _ptr(q), _ptr(K_cache), _ptr(V_cache),
                                    _ptr(cache_len), _ptr(K_cmp), _ptr(V_cmp), _ptr(gates), _ptr(out), _ptr(sel),
                                    _stream(stream)))
    return out, sel


def compress_prepare(cfg: NSAConfig, w_k, w_v, pe_k, pe_v, *, out=None, stream=None):
    """nsa_compress_prepare: the prepared linear maps (a uint8 device buffer) for cache_append."""
    l, dk, dv = cfg.cmp_block, cfg.d_k, cfg.d_v
    _need(w_k, "w_k", torch.bfloat16, (l * dk, dk))
    _need(w_v, "w_v", torch.bfloat16, (l * dv, dv))
    _need(pe_k, "pe_k", torch.bfloat16, (l, dk))
    _need(pe_v, "pe_v", torch.bfloat16, (l, dv))
    prep, n = _workspace(cfg, OP_COMPRESS, w_k.device, out)
    _check(lib().nsa_compress_prepare(ctypes.byref(c_config(cfg)), _ptr(w_k), _ptr(w_v), _ptr(pe_k), _ptr(pe_v),
                                      _ptr(prep), n, _stream(stream)))
    return prep


def cache_append(cfg: NSAConfig, K_new, V_new, K_cache, V_cache, cache_len, K_cmp, V_cmp, prep, stream=None):
    """nsa_cache_append: K_new/V_new [B,Hkv,n_new,d] into the caches at cache_len, new
    compressed entries into K_cmp/V_cmp, cache_len advanced by n_new (all in place)."""
    B, L, Hkv = cfg.batch, cfg.seq_len, cfg.num_kv_heads
    if K_new is None or K_new.dim() != 4:
        raise ValueError("K_new must be [B, Hkv, n_new, d_k]")
    n_new = int(K_new.shape[2])
    _need(K_new, "K_new", torch.bfloat16, (B, Hkv, n_new, cfg.d_k))
    _need(V_new, "V_new", torch.bfloat16, (B, Hkv, n_new, cfg.d_v))
    _need(K_cache, "K_cache", torch.bfloat16, (B, Hkv, L, cfg.d_k))
    _need(V_cache, "V_cache", torch.bfloat16, (B, Hkv, L, cfg.d_v))
    _need(cache_len, "cache_len", torch.int32, (B,))
    _need(K_cmp, "K_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_k))
    _need(V_cmp, "V_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_v))
    _need(prep, "prep", torch.uint8)
    _check(lib().nsa_cache_append(ctypes.byref(c_config(cfg)), _ptr(K_new), _ptr(V_new), n_new, _ptr(K_cache),
                                  _ptr(V_cache), _ptr(cache_len), _ptr(K_cmp), _ptr(V_cmp), _ptr(prep),
                                  prep.numel(), _stream(stream)))


def prefill_fwd(cfg: NSAConfig, Q, K, V, K_cmp, V_cmp, gates=None, *, out=None, sel=None, lse=None, o_cmp=None,
                want_sel=True, want_lse=False, want_ocmp=False, workspace=None, stream=None):
    """nsa_prefill_fwd: score_select + sparse_attn_fwd in one fused launch.  Returns
    (O [B,T,H,dv] bf16, sel [B,T,Hkv,n] int32 or None, lse [B,T,H] or None, o_cmp
    [B,T,H,dv] fp32 or None)."""
    B, T, H, Hkv = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads
    dev = Q.device
    _need(Q, "Q", torch.bfloat16, (B, T, H, cfg.d_k))
    _need(K, "K", torch.bfloat16, (B, Hkv, T, cfg.d_k))
    _need(V, "V", torch.bfloat16, (B, Hkv, T, cfg.d_v))
    _need(K_cmp, "K_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_k))
    _need(V_cmp, "V_cmp", torch.bfloat16, (B, Hkv, cfg.n_cmp, cfg.d_v))
    if gates is not None:
        _need(gates, "gates", torch.float32, (B, T, H, 3))
    if out is None:
        out = torch.empty((B, T, H, cfg.d_v), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, T, H, cfg.d_v))
    if sel is None and want_sel:
        sel = torch.empty((B, T, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, (B, T, Hkv, cfg.top_n))
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, T, H))
    if o_cmp is None and want_ocmp:
        o_cmp = torch.empty((B, T, H, cfg.d_v), dtype=torch.float32, device=dev)
    if o_cmp is not None:
        _need(o_cmp, "o_cmp", torch.float32, (B, T, H, cfg.d_v))
    ws, nws = _workspace(cfg, OP_PREFILL, dev, workspace)
    _check(lib().nsa_prefill_fwd(ctypes.byref(c_config(cfg)), _ptr(Q), _ptr(K), _ptr(V), _ptr(K_cmp), _ptr(V_cmp),
                                 _ptr(gates), _ptr(out), _ptr(sel), _ptr(lse), _ptr(o_cmp), _ptr(ws), nws,
                                 _stream(stream)))
    return out, sel, lse, o_cmp


def prefill(cfg: NSAConfig, Q, K, V, w_k=None, w_v=None, pe_k=None, pe_v=None, gates=None, stream=None,
            train=False, fused=False):
    """The whole prefill hot path: compress -> score_select -> sparse_attn_fwd (or, with
    ``train``, sparse_attn_fwd_train; with ``fused``, compress -> prefill_fwd).  Returns
    dict(out, sel, o_cmp, lse, k_cmp, v_cmp and, with ``train``, saved_lse, saved_o) (o_cmp
    and lse: compressed branch only)."""
    k_cmp, v_cmp = compress(cfg, K, V, w_k, w_v, pe_k, pe_v, stream=stream)
    if fused:
        use_c = bool(cfg.branches & 1)
        out, sel, lse, o_cmp = prefill_fwd(cfg, Q, K, V, k_cmp, v_cmp, gates, want_lse=use_c, want_ocmp=use_c,
                                           stream=stream)
        return {"out": out, "sel": sel, "o_cmp": o_cmp, "lse": lse, "k_cmp": k_cmp, "v_cmp": v_cmp}
    use_c = bool(cfg.branches & 1)
    sel, lse, o_cmp = score_select(cfg, Q, k_cmp, v_cmp, want_lse=use_c, want_ocmp=use_c, stream=stream)
    r = {"sel": sel, "o_cmp": o_cmp, "lse": lse, "k_cmp": k_cmp, "v_cmp": v_cmp}
    if train:
        r["out"], r["saved_lse"], r["saved_o"] = sparse_attn_fwd_train(cfg, Q, K, V, sel, o_cmp, gates, stream=stream)
    else:
        r["out"] = sparse_attn_fwd(cfg, Q, K, V, sel, o_cmp, gates, stream=stream)
    return r


# ---------------------------------------------------------------------------
def sparse_attn_fwd_train(cfg: NSAConfig, Q, K, V, sel=None, o_cmp=None, gates=None, *, out=None, workspace=None,
                          stream=None):
    """nsa_sparse_attn_fwd_train.  Returns (O [B,T,H,dv] bf16, saved_lse [B,T,H,2] fp32,
    saved_o [B,T,H,2,dv] fp32)."""
    B, T, H, Hkv = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads
    _need(Q, "Q", torch.bfloat16, (B, T, H, cfg.d_k))
    _need(K, "K", torch.bfloat16, (B, Hkv, T, cfg.d_k))
    _need(V, "V", torch.bfloat16, (B, Hkv, T, cfg.d_v))
    if cfg.branches & 2:
        _need(sel, "sel", torch.int32, (B, T, Hkv, cfg.top_n))
    if cfg.branches & 1:
        _need(o_cmp, "o_cmp", torch.float32, (B, T, H, cfg.d_v))
    if gates is not None:
        _need(gates, "gates", torch.float32, (B, T, H, 3))
    if out is None:
        out = torch.empty((B, T, H, cfg.d_v), dtype=torch.bfloat16, device=Q.device)
    saved_lse = torch.empty((B, T, H, 2), dtype=torch.float32, device=Q.device)
    saved_o = torch.empty((B, T, H, 2, cfg.d_v), dtype=torch.float32, device=Q.device)
    ws, nws = _workspace(cfg, OP_SPARSE_ATTN, Q.device, workspace)
    _check(lib().nsa_sparse_attn_fwd_train(ctypes.byref(c_config(cfg)), _ptr(Q), _ptr(K), _ptr(V),
                                           _ptr(sel if cfg.branches & 2 else None),
                                           _ptr(o_cmp if cfg.branches & 1 else None), _ptr(gates), _ptr(out),
                                           _ptr(saved_lse), _ptr(saved_o), _ptr(ws), nws, _stream(stream)))
    return out, saved_lse, saved_o


def sparse_attn_bwd(cfg: NSAConfig, Q, K, V, K_cmp, V_cmp, sel, lse_cmp, o_cmp, gates, dO, *, saved_lse=None,
                    saved_o=None, want_dgates=True, workspace=None, stream=None) -> dict:
    """nsa_sparse_attn_bwd.  Returns dict(dq, dk, dv, dk_cmp, dv_cmp, dgates) of fp32 tensors
    (dk_cmp/dv_cmp None without the compressed branch, dgates None without gates).
    saved_lse/saved_o: from sparse_attn_fwd_train (None: recomputed)."""
    B, T, H, Hkv, N = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads, cfg.n_cmp
    dk, dv = cfg.d_k, cfg.d_v
    _need(Q, "Q", torch.bfloat16, (B, T, H, dk))
    _need(K, "K", torch.bfloat16, (B, Hkv, T, dk))
    _need(V, "V", torch.bfloat16, (B, Hkv, T, dv))
    _need(dO, "dO", torch.bfloat16, (B, T, H, dv))
    use_c = bool(cfg.branches & 1)
    if use_c:
        _need(K_cmp, "K_cmp", torch.bfloat16, (B, Hkv, N, dk))
        _need(V_cmp, "V_cmp", torch.bfloat16, (B, Hkv, N, dv))
        _need(lse_cmp, "lse_cmp", torch.float32, (B, T, H))
        _need(o_cmp, "o_cmp", torch.float32, (B, T, H, dv))
    if cfg.branches & 2:
        _need(sel, "sel", torch.int32, (B, T, Hkv, cfg.top_n))
    if gates is not None:
        _need(gates, "gates", torch.float32, (B, T, H, 3))
    if saved_o is not None:
        _need(saved_lse, "saved_lse", torch.float32, (B, T, H, 2))
        _need(saved_o, "saved_o", torch.float32, (B, T, H, 2, dv))
    dev = Q.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, Hkv, T, dk), **f32),
           "dv": torch.empty((B, Hkv, T, dv), **f32),
           "dk_cmp": torch.empty((B, Hkv, N, dk), **f32) if use_c else None,
           "dv_cmp": torch.empty((B, Hkv, N, dv), **f32) if use_c else None,
           "dgates": torch.empty((B, T, H, 3), **f32) if (gates is not None and want_dgates) else None}
    ws, nws = _workspace(cfg, OP_SPARSE_BWD, dev, workspace)
    _check(lib().nsa_sparse_attn_bwd(
        ctypes.byref(c_config(cfg)), _ptr(Q), _ptr(K), _ptr(V), _ptr(K_cmp if use_c else None),
        _ptr(V_cmp if use_c else None), _ptr(sel if cfg.branches & 2 else None), _ptr(lse_cmp if use_c else None),
        _ptr(o_cmp if use_c else None), _ptr(gates), _ptr(saved_lse), _ptr(saved_o), _ptr(dO), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]),
        _ptr(out["dk_cmp"]), _ptr(out["dv_cmp"]), _ptr(out["dgates"]), _ptr(ws), nws, _stream(stream)))
    return out


def compress_bwd(cfg: NSAConfig, K, V, w_k, w_v, pe_k, pe_v, dK_cmp, dV_cmp, dK, dV, *, workspace=None,
                 stream=None) -> dict:
    """nsa_compress_bwd: adds the block map's share into dK, dV (fp32, in place) and returns
    dict(dw_k, dw_v, dpe_k, dpe_v) (fp32)."""
    B, T, Hkv, N, l = cfg.batch, cfg.seq_len, cfg.num_kv_heads, cfg.n_cmp, cfg.cmp_block
    dk, dv = cfg.d_k, cfg.d_v
    _need(K, "K", torch.bfloat16, (B, Hkv, T, dk))
    _need(V, "V", torch.bfloat16, (B, Hkv, T, dv))
    _need(w_k, "w_k", torch.bfloat16, (l * dk, dk))
    _need(w_v, "w_v", torch.bfloat16, (l * dv, dv))
    _need(pe_k, "pe_k", torch.bfloat16, (l, dk))
    _need(pe_v, "pe_v", torch.bfloat16, (l, dv))
    _need(dK_cmp, "dK_cmp", torch.float32, (B, Hkv, N, dk))
    _need(dV_cmp, "dV_cmp", torch.float32, (B, Hkv, N, dv))
    _need(dK, "dK", torch.float32, (B, Hkv, T, dk))
    _need(dV, "dV", torch.float32, (B, Hkv, T, dv))
    f32 = dict(dtype=torch.float32, device=K.device)
    out = {"dw_k": torch.empty((l * dk, dk), **f32), "dw_v": torch.empty((l * dv, dv), **f32),
           "dpe_k": torch.empty((l, dk), **f32), "dpe_v": torch.empty((l, dv), **f32)}
    ws, nws = _workspace(cfg, OP_COMPRESS_BWD, K.device, workspace)
    _check(lib().nsa_compress_bwd(ctypes.byref(c_config(cfg)), _ptr(K), _ptr(V), _ptr(w_k), _ptr(w_v), _ptr(pe_k),
                                  _ptr(pe_v), _ptr(dK_cmp), _ptr(dV_cmp), _ptr(dK), _ptr(dV), _ptr(out["dw_k"]),
                                  _ptr(out["dw_v"]), _ptr(out["dpe_k"]), _ptr(out["dpe_v"]), _ptr(ws), nws,
                                  _stream(stream)))
    return out


def backward(cfg: NSAConfig, fwd: dict, Q, K, V, w_k, w_v, pe_k, pe_v, gates, dO, stream=None) -> dict:
    """The whole backward of ``prefill`` (its returned dict ``fwd`` plus an LSE of the
    compressed branch in fwd["lse"]): nsa_sparse_attn_bwd then nsa_compress_bwd.  Returns
    dict(dq, dk, dv, dgates, dk_cmp, dv_cmp, dw_k, dw_v, dpe_k, dpe_v)."""
    g = sparse_attn_bwd(cfg, Q, K, V, fwd["k_cmp"], fwd["v_cmp"], fwd["sel"], fwd.get("lse"), fwd["o_cmp"], gates,
                        dO, saved_lse=fwd.get("saved_lse"), saved_o=fwd.get("saved_o"), stream=stream)
    if cfg.branches & 1:
        g.update(compress_bwd(cfg, K, V, w_k, w_v, pe_k, pe_v, g["dk_cmp"], g["dv_cmp"], g["dk"], g["dv"],
                              stream=stream))
    return g
