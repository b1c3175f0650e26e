"""Seeded synthetic inputs shared by the GPU path, the oracle, the tests and the bench.

This module only draws random numbers (numpy ``Generator(PCG64(seed))``) and rounds
them to bfloat16; it holds none of the attention method's arithmetic.  Everything the
GPU receives and everything the oracle receives comes from here (or from the oracle's
own outputs), so both sides see bit-identical inputs.

Distributions (one recipe for every workload):

* Q, K, V ~ N(0, 1), rounded to bf16 (round-to-nearest-even).
* Compression weights W_K ``[l*d_k, d_k]`` and W_V ``[l*d_v, d_v]``: Xavier-uniform,
  U(-a, a) with a = sqrt(6 / (fan_in + fan_out)), fan_in = l*d, fan_out = d.
* Intra-block position embeddings PE_K ``[l, d_k]``, PE_V ``[l, d_v]`` ~ N(0, 1).
* Gate logits ``[B, T, H, 3]`` (order: compressed, selected, window) ~ N(0, 1), fp32.

Draw order for a prefill workload: Q, K, V, W_K, W_V, PE_K, PE_V, gates.  Large
tensors are drawn in chunks; numpy's generator fills sequentially, so chunking does not
change the stream.

Stage inputs (used to feed one library call in isolation):

* compressed keys/values ~ N(0, 4) (the variance phi produces with the recipe above);
* block index lists with the workload's sparsity structure (first blocks and the
  blocks nearest the query always present, the rest drawn uniformly without
  replacement from the earlier blocks), sorted ascending and padded with -1;
* compressed-branch outputs ~ N(0, 0.25), fp32.
"""
from __future__ import annotations

import numpy as np

from .configs import NSAConfig

_CHUNK = 1 << 24


# ---------------------------------------------------------------------------
# bf16 helpers (bit manipulation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ---------------------------------------------------------------------------
# raw draws
# ---------------------------------------------------------------------------
def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def _normal_f32(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def _xavier_f32(rng: np.random.Generator, fan_in: int, fan_out: int) -> np.ndarray:
    a = np.sqrt(6.0 / (fan_in + fan_out))
    return rng.uniform(-a, a, size=(fan_in, fan_out)).astype(np.float32)


def prefill_inputs(cfg: NSAConfig, seed: int | None = None) -> dict:
    """All inputs of one prefill (or MoBA) workload.

    Returns a dict of uint16 bf16 bit arrays ``q [B,T,H,dk]``, ``k [B,Hkv,T,dk]``,
    ``v [B,Hkv,T,dv]``, ``w_k``, ``w_v``, ``pe_k``, ``pe_v`` and fp32 ``gates [B,T,H,3]``.
    For workloads drawn in fp32 (``cfg.fp32_inputs``) the unrounded draws are also
    returned under ``raw``.  Compressed-branch weights and gates are absent when the
    workload has no compressed branch (``phi`` = mean).
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    B, T, Hkv, H = cfg.batch, cfg.seq_len, cfg.num_kv_heads, cfg.num_heads
    dk, dv, l = cfg.d_k, cfg.d_v, cfg.cmp_block
    out: dict = {}
    raw: dict = {}
    shapes = {"q": (B, T, H, dk), "k": (B, Hkv, T, dk), "v": (B, Hkv, T, dv)}
    for name in ("q", "k", "v"):
        if cfg.fp32_inputs:
            x = _normal_f32(rng, shapes[name])
            raw[name] = x
            out[name] = f32_to_bf16_bits(x)
        else:
            out[name] = _normal_bf16(rng, shapes[name])
    if cfg.phi == 0:
        wk = _xavier_f32(rng, l * dk, dk)
        wv = _xavier_f32(rng, l * dv, dv)
        pek = rng.standard_normal((l, dk), dtype=np.float32)
        pev = rng.standard_normal((l, dv), dtype=np.float32)
        for name, x in (("w_k", wk), ("w_v", wv), ("pe_k", pek), ("pe_v", pev)):
            if cfg.fp32_inputs:
                raw[name] = x
            out[name] = f32_to_bf16_bits(x)
        out["gates"] = rng.standard_normal((B, T, H, 3), dtype=np.float32)
    if raw:
        out["raw"] = raw
    return out


def grad_output(cfg: NSAConfig, seed: int | None = None) -> np.ndarray:
    """Upstream gradient dO of a prefill's output: bf16 bits [B,T,H,dv] ~ N(0,1), drawn from
    its own stream (seed + 1000) so the forward inputs are unchanged."""
    rng = np.random.Generator(np.random.PCG64((cfg.seed if seed is None else seed) + 1000))
    return _normal_bf16(rng, (cfg.batch, cfg.seq_len, cfg.num_heads, cfg.d_v))


def decode_inputs(cfg: NSAConfig, seed: int | None = None, cache_len: np.ndarray | None = None) -> dict:
    """Inputs of one decode step: ``q [B,H,dk]``, caches ``k [B,Hkv,L,dk]``, ``v [B,Hkv,L,dv]``,
    compression weights, ``gates [B,H,3]`` and ``cache_len [B]`` (default: all L)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    B, L, Hkv, H = cfg.batch, cfg.seq_len, cfg.num_kv_heads, cfg.num_heads
    dk, dv, l = cfg.d_k, cfg.d_v, cfg.cmp_block
    out = {
        "q": _normal_bf16(rng, (B, H, dk)),
        "k": _normal_bf16(rng, (B, Hkv, L, dk)),
        "v": _normal_bf16(rng, (B, Hkv, L, dv)),
    }
    out["w_k"] = f32_to_bf16_bits(_xavier_f32(rng, l * dk, dk))
    out["w_v"] = f32_to_bf16_bits(_xavier_f32(rng, l * dv, dv))
    out["pe_k"] = f32_to_bf16_bits(rng.standard_normal((l, dk), dtype=np.float32))
    out["pe_v"] = f32_to_bf16_bits(rng.standard_normal((l, dv), dtype=np.float32))
    out["gates"] = rng.standard_normal((B, H, 3), dtype=np.float32)
    if cache_len is None:
        cache_len = np.full(B, L, dtype=np.int32)
    out["cache_len"] = np.asarray(cache_len, dtype=np.int32)
    return out


# ---------------------------------------------------------------------------
# stage inputs
# ---------------------------------------------------------------------------
def compressed_kv(cfg: NSAConfig, seed: int, n_cmp: int | None = None) -> dict:
    """Stand-alone compressed keys/values ``k_cmp [B,Hkv,N,dk]``, ``v_cmp [B,Hkv,N,dv]`` (bf16 bits)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = cfg.n_cmp if n_cmp is None else n_cmp
    B, Hkv = cfg.batch, cfg.num_kv_heads
    return {
        "k_cmp": _normal_bf16(rng, (B, Hkv, n, cfg.d_k), std=2.0),
        "v_cmp": _normal_bf16(rng, (B, Hkv, n, cfg.d_v), std=2.0),
    }


def block_lists(cfg: NSAConfig, seed: int, positions: np.ndarray | None = None) -> np.ndarray:
    """Random block index lists ``[B, P, Hkv, top_n]`` int32 with the workload's structure.

    For a query at position t the candidate blocks are 0 .. jc with jc = t // slc_block.
    The first ``n_init`` blocks and the ``n_local`` blocks ending at jc are always in the
    list; the other candidates form the contiguous range between them, from which the
    remaining slots (up to ``top_n`` entries in total, or all candidates if there are
    fewer) are drawn uniformly without replacement (Floyd's method, vectorized over rows).
    Lists are sorted ascending and padded with -1.  ``positions`` defaults to 0 .. T-1.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hkv, n = cfg.batch, cfg.num_kv_heads, cfg.top_n
    pos = np.arange(cfg.seq_len) if positions is None else np.asarray(positions)
    P = len(pos)
    jc = (pos.astype(np.int64) // cfg.slc_block)
    jc = np.broadcast_to(jc[None, :, None], (B, P, Hkv)).reshape(-1)
    R = jc.size
    f_init = np.minimum(cfg.n_init, jc + 1)
    f_lo = np.maximum(0, jc - cfg.n_local + 1)
    lo = f_init                                   # free candidates: lo .. f_lo-1
    m = np.maximum(0, f_lo - lo)
    n_forced = f_init + (jc - f_lo + 1) - np.maximum(0, f_init - f_lo)
    k = np.minimum(np.maximum(0, np.minimum(n, jc + 1) - n_forced), m)
    kmax = int(k.max()) if R else 0
    picks = np.full((R, max(kmax, 1)), -1, dtype=np.int64)
    for i in range(kmax):
        active = i < k
        j = m - k + i                             # Floyd: draw from 0 .. j
        u = rng.random(R)
        t = np.minimum((u * (j + 1)).astype(np.int64), j)
        dup = (picks[:, :i] == t[:, None]).any(axis=1) if i else np.zeros(R, bool)
        val = np.where(dup, j, t)
        picks[:, i] = np.where(active, val, -1)
    out = np.full((R, n), -1, dtype=np.int64)
    # assemble: forced init blocks, free picks (offset by lo), local blocks; then sort
    cols = np.full((R, n + 1), np.iinfo(np.int64).max, dtype=np.int64)
    c = 0
    for i in range(min(cfg.n_init, n)):
        cols[:, c] = np.where(i < f_init, i, cols[:, c]); c += 1
    for i in range(kmax):
        cols[:, c] = np.where(picks[:, i] >= 0, lo + picks[:, i], cols[:, c]); c += 1
    for i in range(min(cfg.n_local, n)):
        blk = jc - i
        ok = (blk >= f_lo) & (blk >= f_init)      # local blocks not already counted as initial
        cols[:, c] = np.where(ok, blk, cols[:, c]); c += 1
    cols = np.sort(cols[:, :c], axis=1) if c else cols[:, :0]
    cnt = np.minimum(n, jc + 1)
    take = min(n, cols.shape[1])
    body = cols[:, :take]
    body = np.where(np.arange(take)[None, :] < cnt[:, None], body, -1)
    out[:, :take] = body
    return out.reshape(B, P, Hkv, n).astype(np.int32)


def cmp_outputs(cfg: NSAConfig, seed: int) -> np.ndarray:
    """Stand-alone compressed-branch outputs ``[B, T, H, dv]`` fp32 ~ N(0, 0.25)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _normal_f32(rng, (cfg.batch, cfg.seq_len, cfg.num_heads, cfg.d_v), std=0.5)
