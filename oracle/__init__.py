"""fp64 CPU oracle of the NSA forward and backward passes (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import
this package.  It loads ``liboracle.so`` built from ``nsa_oracle.c`` with gcc (OpenMP),
and shares no code with the GPU library.  ``bruteforce`` is an independent dense-mask
numpy formulation used to pin the C oracle on tiny shapes.

Every function here is a thin ctypes wrapper: arrays go in as contiguous float64 / int32.
Parity status of each function (what pins it) is listed in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2 -fopenmp).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_compress_linear.argtypes = [ctypes.c_int] * 5 + [_D, _D, _D, _I, ctypes.c_int, _D]
        L.oracle_compress_mean.argtypes = [ctypes.c_int] * 3 + [_D, _I, ctypes.c_int, _D]
        L.oracle_score_select.argtypes = ([ctypes.c_int] * 13 + [ctypes.c_double, _D, _I, ctypes.c_int,
                                          _D, _D, _D, _D, _D, _I, _D])
        L.oracle_score_select.restype = ctypes.c_int
        L.oracle_select_from_scores.argtypes = [ctypes.c_int] * 5 + [_I, _D, _I, _D]
        L.oracle_select_from_scores.restype = ctypes.c_int
        L.oracle_attend.argtypes = ([ctypes.c_int] * 8 + [ctypes.c_double, ctypes.c_int, _D, _I, ctypes.c_int,
                                    _D, _D, _I, _D, _D, _D, _D, _D])
        L.oracle_attend.restype = ctypes.c_int
        L.oracle_causal_attention.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, _D, _D, _D, _D]
        L.oracle_causal_attention_rows.argtypes = [ctypes.c_int, _I, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                                   _D, _D, _D, _D]
        L.oracle_nsa_bwd.argtypes = ([ctypes.c_int] * 11 + [ctypes.c_double, ctypes.c_int] + [_D] * 5 + [_I]
                                     + [_D] * 8)
        L.oracle_nsa_bwd.restype = ctypes.c_int
        L.oracle_compress_linear_bwd.argtypes = [ctypes.c_int] * 6 + [_D] * 7
        L.oracle_nsa_bwd_rows.argtypes = ([ctypes.c_int] * 11 + [ctypes.c_double, ctypes.c_int, _D, _I, ctypes.c_int]
                                          + [_D] * 4 + [_I] + [_D] * 4)
        L.oracle_nsa_bwd_rows.restype = ctypes.c_int
        L.oracle_nsa_bwd_keys.argtypes = ([ctypes.c_int] * 11 + [ctypes.c_double, ctypes.c_int] + [_D] * 5 + [_I]
                                          + [_D] * 2 + [_I, ctypes.c_int, _I, ctypes.c_int] + [_D] * 4)
        L.oracle_nsa_bwd_keys.restype = ctypes.c_int
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _d(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _pd(a):
    return None if a is None else a.ctypes.data_as(_D)


def _pi(a):
    return None if a is None else a.ctypes.data_as(_I)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ---------------------------------------------------------------------------
# step 1
# ---------------------------------------------------------------------------
def compress_linear(X, pe, W, l: int, s: int, blocks=None) -> np.ndarray:
    """Linear phi of the listed blocks of one head's token rows X [n_tok, d] -> [nblk, d_out]."""
    X, W = _d(X), _d(W)
    pe = None if pe is None else _d(pe)
    n_tok, d = X.shape
    d_out = W.shape[1]
    assert W.shape[0] == l * d
    if blocks is None:
        blocks = np.arange((n_tok - l) // s + 1 if n_tok >= l else 0)
    blocks = _i(blocks)
    assert blocks.size == 0 or (blocks.max() * s + l <= n_tok and blocks.min() >= 0)
    out = np.zeros((blocks.size, d_out), dtype=np.float64)
    lib().oracle_compress_linear(n_tok, d, d_out, l, s, _pd(X), _pd(pe), _pd(W), _pi(blocks),
                                 blocks.size, _pd(out))
    return out


def compress_mean(X, l: int, s: int, blocks=None) -> np.ndarray:
    X = _d(X)
    n_tok, d = X.shape
    if blocks is None:
        blocks = np.arange((n_tok - l) // s + 1 if n_tok >= l else 0)
    blocks = _i(blocks)
    assert blocks.size == 0 or (blocks.max() * s + l <= n_tok and blocks.min() >= 0)
    out = np.zeros((blocks.size, d), dtype=np.float64)
    lib().oracle_compress_mean(d, l, s, _pd(X), _pi(blocks), blocks.size, _pd(out))
    return out


# ---------------------------------------------------------------------------
# steps 2-4
# ---------------------------------------------------------------------------
def score_select(cfg, Q_rows, rows, Kc, Vc=None, want_scores=True, want_ocmp=True) -> dict:
    """Compressed attention + block scores + selection for listed rows of one batch element.

    ``cfg`` needs the attributes of an NSA configuration (num_kv_heads, heads_per_group, d_k,
    d_v, cmp_block, cmp_stride, slc_block, top_n, n_init, n_local, score_mode, scale,
    seq_len).  Q_rows [nrows, H, dk]; Kc [Hkv, n_cmp, dk]; Vc [Hkv, n_cmp, dv].
    Returns dict(lse [nrows,H], o_cmp [nrows,H,dv], scores [nrows,Hkv,n_slc],
    sel [nrows,Hkv,top_n] int32, gap [nrows,Hkv]).
    """
    Hkv, G = cfg.num_kv_heads, cfg.heads_per_group
    H = Hkv * G
    Q_rows, Kc = _d(Q_rows), _d(Kc)
    rows = _i(rows)
    nrows = rows.size
    n_cmp = Kc.shape[1]
    n_slc = -(-cfg.seq_len // cfg.slc_block)
    mode = int(cfg.score_mode)
    Vc = None if (Vc is None or mode == 1) else _d(Vc)
    lse = np.zeros((nrows, H))
    ocmp = np.zeros((nrows, H, cfg.d_v)) if (want_ocmp and Vc is not None) else None
    scores = np.zeros((nrows, Hkv, n_slc)) if want_scores else None
    sel = np.zeros((nrows, Hkv, cfg.top_n), dtype=np.int32)
    gap = np.zeros((nrows, Hkv))
    rc = lib().oracle_score_select(mode, Hkv, G, cfg.d_k, cfg.d_v, cfg.cmp_block, cfg.cmp_stride,
                                   n_cmp, cfg.slc_block, n_slc, cfg.top_n, cfg.n_init, cfg.n_local,
                                   float(cfg.scale), _pd(Q_rows), _pi(rows), nrows, _pd(Kc), _pd(Vc),
                                   _pd(lse), _pd(ocmp), _pd(scores), _pi(sel), _pd(gap))
    if rc != 0:
        raise ValueError(f"oracle_score_select failed ({rc})")
    return {"lse": lse, "o_cmp": ocmp, "scores": scores, "sel": sel, "gap": gap}


def select_from_scores(scores, jc, top_n: int, n_init: int, n_local: int):
    """Step 4 alone: scores [nrows, n_slc], own block jc [nrows] -> (sel [nrows, top_n], gap)."""
    scores = _d(scores)
    jc = _i(jc)
    nrows, n_slc = scores.shape
    sel = np.zeros((nrows, top_n), dtype=np.int32)
    gap = np.zeros(nrows)
    rc = lib().oracle_select_from_scores(nrows, n_slc, top_n, n_init, n_local, _pi(jc), _pd(scores),
                                         _pi(sel), _pd(gap))
    if rc != 0:
        raise ValueError("top_n smaller than the number of forced blocks")
    return sel, gap


# ---------------------------------------------------------------------------
# steps 5-7
# ---------------------------------------------------------------------------
def attend(cfg, Q_rows, rows, K, V, sel, o_cmp=None, gates=None, branches=None) -> dict:
    """Selected + window branches and the gated sum for listed rows of one batch element.

    Q_rows [nrows, H, dk]; K [Hkv, n_tok, dk]; V [Hkv, n_tok, dv]; sel [nrows, Hkv, top_n];
    o_cmp [nrows, H, dv]; gates [nrows, H, 3] logits (None -> weights 1).
    Returns dict(out, o_slc, o_win), each [nrows, H, dv].
    """
    Hkv, G = cfg.num_kv_heads, cfg.heads_per_group
    H = Hkv * G
    branches = cfg.branches if branches is None else branches
    Q_rows, K, V = _d(Q_rows), _d(K), _d(V)
    rows, sel = _i(rows), _i(sel)
    nrows = rows.size
    n_tok = K.shape[1]
    if branches & 1:
        assert o_cmp is not None
        o_cmp = _d(o_cmp)
    else:
        o_cmp = None
    gates = None if gates is None else _d(gates)
    out = np.zeros((nrows, H, cfg.d_v))
    oslc = np.zeros_like(out)
    owin = np.zeros_like(out)
    rc = lib().oracle_attend(Hkv, G, cfg.d_k, cfg.d_v, n_tok, cfg.slc_block, sel.shape[-1], cfg.window,
                             float(cfg.scale), branches, _pd(Q_rows), _pi(rows), nrows, _pd(K), _pd(V),
                             _pi(sel), _pd(o_cmp), _pd(gates), _pd(out), _pd(oslc), _pd(owin))
    if rc != 0:
        raise MemoryError("oracle_attend failed")
    return {"out": out, "o_slc": oslc, "o_win": owin}


def causal_attention_rows(Q_rows, rows, K, V, scale: float) -> np.ndarray:
    """Causal attention of one head for listed rows of a sequence: row rows[k] (query
    Q_rows[k]) attends keys 0 .. rows[k] of K [n,dk], V [n,dv].  Returns [nrows, dv]."""
    Q, K, V = _d(Q_rows), _d(K), _d(V)
    rows = _i(rows)
    assert rows.min() >= 0 and rows.max() < K.shape[0]
    out = np.zeros((len(rows), V.shape[1]))
    lib().oracle_causal_attention_rows(len(rows), _pi(rows), Q.shape[1], V.shape[1], float(scale), _pd(Q), _pd(K),
                                       _pd(V), _pd(out))
    return out


def causal_attention(Q, K, V, scale: float, window: int = 0) -> np.ndarray:
    """Textbook causal (optionally sliding-window) attention of one head: Q [n,dk] -> [n,dv]."""
    Q, K, V = _d(Q), _d(K), _d(V)
    n, dk = Q.shape
    dv = V.shape[1]
    out = np.zeros((n, dv))
    lib().oracle_causal_attention(n, dk, dv, window, float(scale), _pd(Q), _pd(K), _pd(V), _pd(out))
    return out


# ---------------------------------------------------------------------------
# backward (the selection held fixed)
# ---------------------------------------------------------------------------
def nsa_bwd(cfg, Q, K, V, Kc, Vc, sel, gates, dO, branches=None) -> dict:
    """Gradients of the gated output of every row of one batch element.

    Q [T,H,dk]; K [Hkv,T,dk]; V [Hkv,T,dv]; Kc [Hkv,N,dk]; Vc [Hkv,N,dv] (None when the
    compressed branch is off); sel [T,Hkv,top_n]; gates [T,H,3] logits or None (weights 1);
    dO [T,H,dv].  Returns dict(dq, dk, dv, dkc, dvc, dgates) shaped like their inputs
    (dgates None without gates; dkc/dvc None without the compressed branch).
    """
    Hkv, G = cfg.num_kv_heads, cfg.heads_per_group
    branches = cfg.branches if branches is None else branches
    Q, K, V, dO = _d(Q), _d(K), _d(V), _d(dO)
    sel = _i(sel)
    T = Q.shape[0]
    use_c = bool(branches & 1)
    Kc = _d(Kc) if use_c else None
    Vc = _d(Vc) if use_c else None
    n_cmp = Kc.shape[1] if use_c else 0
    gates = None if gates is None else _d(gates)
    out = {"dq": np.zeros_like(Q), "dk": np.zeros_like(K), "dv": np.zeros_like(V),
           "dkc": np.zeros_like(Kc) if use_c else None, "dvc": np.zeros_like(Vc) if use_c else None,
           "dgates": np.zeros_like(gates) if gates is not None else None}
    rc = lib().oracle_nsa_bwd(Hkv, G, cfg.d_k, cfg.d_v, T, n_cmp, cfg.cmp_block, cfg.cmp_stride, cfg.slc_block,
                              sel.shape[-1], cfg.window, float(cfg.scale), branches, _pd(Q), _pd(K), _pd(V),
                              _pd(Kc), _pd(Vc), _pi(sel), _pd(gates), _pd(dO), _pd(out["dq"]), _pd(out["dk"]),
                              _pd(out["dv"]), _pd(out["dkc"]), _pd(out["dvc"]), _pd(out["dgates"]))
    if rc != 0:
        raise MemoryError("oracle_nsa_bwd failed")
    return out


def compress_linear_bwd(X, pe, W, dY, l: int, s: int) -> dict:
    """Backward of the linear phi over blocks 0 .. dY.shape[0]-1 of one head's token rows
    X [n_tok, d]: returns dict(dx [n_tok,d], dw [l*d,d_out], dpe [l,d])."""
    X, W, dY = _d(X), _d(W), _d(dY)
    pe = None if pe is None else _d(pe)
    n_tok, d = X.shape
    d_out = W.shape[1]
    nblk = dY.shape[0]
    assert W.shape[0] == l * d and (nblk == 0 or (nblk - 1) * s + l <= n_tok)
    out = {"dx": np.zeros_like(X), "dw": np.zeros_like(W), "dpe": np.zeros((l, d))}
    lib().oracle_compress_linear_bwd(n_tok, d, d_out, l, s, nblk, _pd(X), _pd(pe), _pd(W), _pd(dY),
                                     _pd(out["dx"]), _pd(out["dw"]), _pd(out["dpe"]))
    return out


def nsa_bwd_rows(cfg, Q_rows, rows, K, V, Kc, Vc, sel_rows, gates_rows, dO_rows, branches=None) -> dict:
    """dq and the gate-logit gradients of listed rows of one batch element (the query side of
    nsa_bwd).  Q_rows [nrows,H,dk], sel_rows [nrows,Hkv,top_n], gates_rows [nrows,H,3] or
    None, dO_rows [nrows,H,dv]; K, V, Kc, Vc as for nsa_bwd.  Returns dict(dq, dgates)."""
    Hkv, G = cfg.num_kv_heads, cfg.heads_per_group
    branches = cfg.branches if branches is None else branches
    Q_rows, K, V, dO_rows = _d(Q_rows), _d(K), _d(V), _d(dO_rows)
    rows, sel_rows = _i(rows), _i(sel_rows)
    use_c = bool(branches & 1)
    Kc = _d(Kc) if use_c else None
    Vc = _d(Vc) if use_c else None
    gates_rows = None if gates_rows is None else _d(gates_rows)
    out = {"dq": np.zeros_like(Q_rows),
           "dgates": None if gates_rows is None else np.zeros_like(gates_rows)}
    rc = lib().oracle_nsa_bwd_rows(Hkv, G, cfg.d_k, cfg.d_v, K.shape[1], Kc.shape[1] if use_c else 0, cfg.cmp_block,
                                   cfg.cmp_stride, cfg.slc_block, sel_rows.shape[-1], cfg.window, float(cfg.scale),
                                   branches, _pd(Q_rows), _pi(rows), rows.size, _pd(K), _pd(V), _pd(Kc), _pd(Vc),
                                   _pi(sel_rows), _pd(gates_rows), _pd(dO_rows), _pd(out["dq"]), _pd(out["dgates"]))
    if rc != 0:
        raise MemoryError("oracle_nsa_bwd_rows failed")
    return out


def nsa_bwd_keys(cfg, Q, K, V, Kc, Vc, sel, gates, dO, raw_keys, cmp_keys=(), branches=None) -> dict:
    """The key side of nsa_bwd for listed keys of one batch element: raw token indices
    ``raw_keys`` and compressed-block indices ``cmp_keys`` (both applied to every KV group).
    Q, K, V, Kc, Vc, sel, gates, dO as for nsa_bwd.  Returns dict(dk [Hkv,n_raw,dk],
    dv [Hkv,n_raw,dv], dkc [Hkv,n_ck,dk], dvc [Hkv,n_ck,dv]) equal to nsa_bwd's gradients at
    those keys."""
    Hkv, G = cfg.num_kv_heads, cfg.heads_per_group
    branches = cfg.branches if branches is None else branches
    Q, K, V, dO = _d(Q), _d(K), _d(V), _d(dO)
    sel = _i(sel)
    T = Q.shape[0]
    raw = _i(np.unique(np.asarray(raw_keys, dtype=np.int64)))
    ck = _i(np.unique(np.asarray(cmp_keys, dtype=np.int64)))
    use_c = bool(branches & 1)
    Kc = _d(Kc) if use_c else None
    Vc = _d(Vc) if use_c else None
    n_cmp = Kc.shape[1] if use_c else 0
    if not use_c:
        ck = _i(np.zeros(0))
    assert raw.size == 0 or (raw.min() >= 0 and raw.max() < T)
    assert ck.size == 0 or (ck.min() >= 0 and ck.max() < n_cmp)
    gates = None if gates is None else _d(gates)
    out = {"dk": np.zeros((Hkv, raw.size, cfg.d_k)), "dv": np.zeros((Hkv, raw.size, cfg.d_v)),
           "dkc": np.zeros((Hkv, ck.size, cfg.d_k)), "dvc": np.zeros((Hkv, ck.size, cfg.d_v)),
           "raw_keys": raw, "cmp_keys": ck}
    rc = lib().oracle_nsa_bwd_keys(Hkv, G, cfg.d_k, cfg.d_v, T, n_cmp, cfg.cmp_block, cfg.cmp_stride, cfg.slc_block,
                                   sel.shape[-1], cfg.window, float(cfg.scale), branches, _pd(Q), _pd(K), _pd(V),
                                   _pd(Kc), _pd(Vc), _pi(sel), _pd(gates), _pd(dO), _pi(raw), raw.size, _pi(ck),
                                   ck.size, _pd(out["dk"]), _pd(out["dv"]), _pd(out["dkc"]), _pd(out["dvc"]))
    if rc != 0:
        raise MemoryError("oracle_nsa_bwd_keys failed")
    return out
