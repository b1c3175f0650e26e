"""Independent dense-mask formulation of the NSA forward pass (test infrastructure).

Used only to pin the C oracle on tiny shapes.  It is written differently on purpose:
every branch is an explicit T x N boolean mask applied to a full score matrix, block
overlaps are an explicit 0/1 matrix built from interval intersection, and selection is
decided by counting ranks instead of sorting.  numpy float64 throughout.
"""
from __future__ import annotations

import itertools

import numpy as np


def _masked_softmax_rows(A, M):
    """Row softmax of A restricted to M (bool); rows with no allowed entry give zeros."""
    A = np.where(M, A, -np.inf)
    mx = A.max(axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    E = np.where(M, np.exp(A - mx), 0.0)
    S = E.sum(axis=1, keepdims=True)
    return np.divide(E, S, out=np.zeros_like(E), where=S > 0)


def overlap_matrix(n_cmp, n_slc, l, s, lp):
    """Ov[i, j] = 1 when compressed block i (tokens [i*s, i*s+l)) and selection block j
    (tokens [j*lp, (j+1)*lp)) share at least one token."""
    i = np.arange(n_cmp)[:, None]
    j = np.arange(n_slc)[None, :]
    return ((i * s < (j + 1) * lp) & (j * lp < i * s + l)).astype(np.float64)


def rank_select(score, jc, top_n, n_init, n_local):
    """Selection by rank counting.  score: [n_slc] (only 0..jc used)."""
    elig = np.arange(jc + 1)
    forced = (elig < n_init) | (elig >= jc - n_local + 1)
    free = elig[~forced]
    k = min(top_n, jc + 1) - int(forced.sum())
    chosen = []
    for j in free:
        better = sum(1 for j2 in free if score[j2] > score[j] or (score[j2] == score[j] and j2 < j))
        if better < k:
            chosen.append(int(j))
    out = sorted(list(elig[forced].tolist()) + chosen)
    return out + [-1] * (top_n - len(out))


def subset_select(score, jc, top_n, n_init, n_local):
    """Selection by exhaustive search: among all free subsets of the allowed size, the one
    with the largest score sum; equal sums prefer the smaller sum of block indices."""
    elig = list(range(jc + 1))
    forced = [j for j in elig if j < n_init or j >= jc - n_local + 1]
    free = [j for j in elig if j not in forced]
    k = min(top_n, jc + 1) - len(forced)
    best, best_key = None, None
    for sub in itertools.combinations(free, k):
        key = (sum(score[j] for j in sub), -sum(sub))
        if best_key is None or key > best_key:
            best, best_key = sub, key
    out = sorted(forced + list(best))
    return out + [-1] * (top_n - len(out))


def nsa_dense(cfg, Q, K, V, Kc, Vc, gates=None, sel=None, mode=None):
    """Full NSA forward of one batch element with explicit masks.

    Q [T,H,dk]; K [Hkv,T,dk]; V [Hkv,T,dv]; Kc [Hkv,N,dk]; Vc [Hkv,N,dv]; gates [T,H,3].
    ``sel`` overrides the selection ([T,Hkv,top_n]).  Returns a dict with o_cmp, scores,
    sel, o_slc, o_win, out (all float64).
    """
    T, H, dk = Q.shape
    Hkv = K.shape[0]
    G = H // Hkv
    dv = V.shape[2]
    l, s, lp = cfg.cmp_block, cfg.cmp_stride, cfg.slc_block
    n_slc = -(-T // lp)
    N = Kc.shape[1]
    scale = cfg.scale
    mode = cfg.score_mode if mode is None else mode
    t = np.arange(T)[:, None]
    key = np.arange(T)[None, :]

    o_cmp = np.zeros((T, H, dv))
    scores = np.zeros((T, Hkv, n_slc))
    if mode == 0:
        Mc = (np.arange(N)[None, :] * s + l - 1) <= t
        Ov = overlap_matrix(N, n_slc, l, s, lp)
        for h in range(H):
            g = h // G
            P = _masked_softmax_rows(scale * Q[:, h, :] @ Kc[g].T, Mc)
            o_cmp[:, h, :] = P @ Vc[g]
            scores[:, g, :] += P @ Ov
    else:
        blk = np.arange(n_slc)[None, :]
        Mb = (blk < t // lp) & (blk < N)
        for h in range(H):
            g = h // G
            A = np.zeros((T, n_slc))
            A[:, :N] = Q[:, h, :] @ Kc[g].T
            scores[:, g, :] += np.where(Mb, A, 0.0)

    if sel is None:
        sel = np.full((T, Hkv, cfg.top_n), -1, dtype=np.int32)
        for tt in range(T):
            for g in range(Hkv):
                sel[tt, g] = rank_select(scores[tt, g], tt // lp, cfg.top_n, cfg.n_init, cfg.n_local)

    o_slc = np.zeros((T, H, dv))
    o_win = np.zeros((T, H, dv))
    causal = key <= t
    Mw = causal & (key > t - cfg.window) if cfg.window > 0 else np.zeros((T, T), bool)
    for g in range(Hkv):
        chosen = np.zeros((T, n_slc), bool)
        for c in range(sel.shape[2]):
            j = sel[:, g, c]
            ok = j >= 0
            chosen[np.arange(T)[ok], j[ok]] = True
        Ms = chosen[:, np.arange(T) // lp] & causal
        for hh in range(G):
            h = g * G + hh
            A = scale * Q[:, h, :] @ K[g].T
            o_slc[:, h, :] = _masked_softmax_rows(A, Ms) @ V[g]
            o_win[:, h, :] = _masked_softmax_rows(A, Mw) @ V[g]

    sig = (lambda z: 1.0 / (1.0 + np.exp(-z)))
    w = np.ones((T, H, 3)) if gates is None else sig(np.asarray(gates, np.float64))
    br = cfg.branches
    out = np.zeros((T, H, dv))
    if br & 1:
        out += w[:, :, 0:1] * o_cmp
    if br & 2:
        out += w[:, :, 1:2] * o_slc
    if br & 4:
        out += w[:, :, 2:3] * o_win
    return {"o_cmp": o_cmp, "scores": scores, "sel": sel, "o_slc": o_slc, "o_win": o_win, "out": out}
