"""The oracle's end-to-end chains (test infrastructure; see ``oracle/__init__.py``).

Each chain composes the C oracle's stages in the order the method runs them: compress
the keys and values block by block, score and select blocks per GQA group, then attend
and gate.  The compressed keys/values cross the library boundary in bf16, so the chain
rounds them to bf16 (nearest, ties to even) between step 1 and step 2 - the one place
where the stored precision of an intermediate enters the result.  ``round_cmp=False``
keeps them in fp64 (a pure-fp64 diagnostic).
"""
from __future__ import annotations

import numpy as np

from . import attend, compress_linear, compress_linear_bwd, compress_mean, nsa_bwd, score_select


def round_to_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (8 significant bits, ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def compress_all(cfg, K, V, w_k, w_v, pe_k, pe_v, round_cmp: bool = True):
    """Step 1 for every KV head of one batch element: K [Hkv,T,dk] -> Kc [Hkv,N,dk], Vc."""
    Kc, Vc = [], []
    for g in range(K.shape[0]):
        if cfg.phi == 0:
            kc = compress_linear(K[g], pe_k, w_k, cfg.cmp_block, cfg.cmp_stride)
            vc = compress_linear(V[g], pe_v, w_v, cfg.cmp_block, cfg.cmp_stride)
        else:
            kc = compress_mean(K[g], cfg.cmp_block, cfg.cmp_stride)
            vc = np.zeros((kc.shape[0], 0))
        Kc.append(round_to_bf16(kc) if round_cmp else kc)
        Vc.append(round_to_bf16(vc) if round_cmp else vc)
    return np.stack(Kc), np.stack(Vc)


def forward_rows(cfg, Q, K, V, Kc, Vc, gates, rows) -> dict:
    """Steps 2-7 for the listed rows of one batch element.

    Q [T,H,dk] (or any array indexable by ``rows``), K [Hkv,T,dk], V [Hkv,T,dv],
    Kc/Vc compressed (or mean-pooled) keys/values, gates [T,H,3] or None.
    """
    rows = np.asarray(rows, dtype=np.int32)
    Qr = np.asarray(Q[rows], dtype=np.float64)
    ss = score_select(cfg, Qr, rows, Kc, Vc if cfg.score_mode == 0 else None)
    gr = None if gates is None else np.asarray(gates[rows], dtype=np.float64)
    at = attend(cfg, Qr, rows, K, V, ss["sel"], ss["o_cmp"], gr)
    ss.update(at)
    return ss


def backward(cfg, Q, K, V, w_k, w_v, pe_k, pe_v, sel, gates, dO, branches=None) -> dict:
    """Gradients of one batch element's gated output through steps 1, 2 and 5-7 (the
    selection ``sel`` held fixed), with the compressed keys/values kept in fp64.

    Returns dict(dq, dk, dv, dgates, dkc, dvc, dw_k, dw_v, dpe_k, dpe_v): dk/dv include the
    compressed branch's contribution through the block map; dw_*/dpe_* are the block map's
    weight and position-embedding gradients summed over the KV heads.
    """
    branches = cfg.branches if branches is None else branches
    Kc, Vc = compress_all(cfg, K, V, w_k, w_v, pe_k, pe_v, round_cmp=False)
    g = nsa_bwd(cfg, Q, K, V, Kc, Vc, sel, gates, dO, branches)
    out = dict(g)
    out["dw_k"] = np.zeros_like(np.asarray(w_k, dtype=np.float64))
    out["dw_v"] = np.zeros_like(np.asarray(w_v, dtype=np.float64))
    out["dpe_k"] = np.zeros((cfg.cmp_block, cfg.d_k))
    out["dpe_v"] = np.zeros((cfg.cmp_block, cfg.d_v))
    if branches & 1:
        for h in range(K.shape[0]):
            bk = compress_linear_bwd(K[h], pe_k, w_k, g["dkc"][h], cfg.cmp_block, cfg.cmp_stride)
            bv = compress_linear_bwd(V[h], pe_v, w_v, g["dvc"][h], cfg.cmp_block, cfg.cmp_stride)
            out["dk"][h] += bk["dx"]
            out["dv"][h] += bv["dx"]
            out["dw_k"] += bk["dw"]
            out["dw_v"] += bv["dw"]
            out["dpe_k"] += bk["dpe"]
            out["dpe_v"] += bv["dpe"]
    return out
