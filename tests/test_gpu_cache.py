"""GPU parity of decode cache maintenance (nsa_compress_prepare + nsa_cache_append).

Growing a cache token by token (and in chunks) must leave exactly the cache that the prefill
path builds from the whole sequence: raw rows copied, every completed compressed block equal
to nsa_compress's entry bit for bit and, to the bf16 rounding bound, to the fp64 oracle's
compression; blocks not yet complete stay untouched; cache_len advances and saturates at the
capacity.
"""
import numpy as np
import pytest
import torch

from oracle import pipeline
from dynamic_block_sparse_nsa_amd import inputs, ops
from dynamic_block_sparse_nsa_amd.configs import DECODE
from nsa_testlib import bf16_dev_to_f64, check_ulp, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a bf16 NaN pattern that no computed entry can take


def f64(bits):
    return inputs.bf16_bits_to_f64(bits)


def _sentinel_like(t):
    return torch.full(t.shape, SENTINEL, dtype=torch.int16, device=t.device).view(torch.bfloat16)


def _is_sentinel(t):
    return bool((t.contiguous().view(torch.int16) == SENTINEL).all())


def complete_blocks(cfg, n):
    """Compressed blocks whose last token is below length n."""
    return 0 if n < cfg.cmp_block else min((n - cfg.cmp_block) // cfg.cmp_stride + 1, cfg.n_cmp)


def _grow(cfg, start, steps):
    print(f"[case] cache append {cfg.name} start={list(start)} steps={steps}", flush=True)
    inp = inputs.decode_inputs(cfg)
    B, Hkv, L = cfg.batch, cfg.num_kv_heads, cfg.seq_len
    K, V = dev_bf16(inp["k"]), dev_bf16(inp["v"])
    wk, wv, pk, pv = (dev_bf16(inp[n]) for n in ("w_k", "w_v", "pe_k", "pe_v"))
    ref_k, ref_v = ops.compress(cfg, K, V, wk, wv, pk, pv)        # the prefill path's caches
    prep = ops.compress_prepare(cfg, wk, wv, pk, pv)
    # caches holding the first start[b] tokens (the rest filled with a sentinel) and the
    # compressed entries complete at that length (the rest sentinel)
    kc, vc, kcmp, vcmp = (_sentinel_like(t) for t in (K, V, ref_k, ref_v))
    for b in range(B):
        n = int(start[b])
        kc[b, :, :n] = K[b, :, :n]
        vc[b, :, :n] = V[b, :, :n]
        nb = complete_blocks(cfg, n)
        kcmp[b, :, :nb] = ref_k[b, :, :nb]
        vcmp[b, :, :nb] = ref_v[b, :, :nb]
    clen = dev_i32(np.asarray(start, dtype=np.int32))
    length = np.asarray(start, dtype=np.int64)
    for n_new in steps:
        # the next n_new tokens of every sequence (past the capacity: anything, dropped)
        idx = np.minimum(length[:, None] + np.arange(n_new)[None, :], L - 1)
        kn = torch.stack([K[b][:, torch.as_tensor(idx[b], device=K.device)] for b in range(B)]).contiguous()
        vn = torch.stack([V[b][:, torch.as_tensor(idx[b], device=V.device)] for b in range(B)]).contiguous()
        ops.cache_append(cfg, kn, vn, kc, vc, clen, kcmp, vcmp, prep)
        length = np.minimum(length + n_new, L)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(clen.cpu().numpy(), length)
    for b in range(B):
        n = int(length[b])
        nb = complete_blocks(cfg, n)
        assert torch.equal(kc[b, :, :n], K[b, :, :n]) and torch.equal(vc[b, :, :n], V[b, :, :n]), f"raw rows b={b}"
        assert _is_sentinel(kc[b, :, n:]) and _is_sentinel(vc[b, :, n:]), f"rows past b={b}"
        assert torch.equal(kcmp[b, :, :nb], ref_k[b, :, :nb]), f"K_cmp b={b}: appended entries differ from nsa_compress"
        assert torch.equal(vcmp[b, :, :nb], ref_v[b, :, :nb]), f"V_cmp b={b}"
        assert _is_sentinel(kcmp[b, :, nb:]) and _is_sentinel(vcmp[b, :, nb:]), f"incomplete blocks written b={b}"
    # the grown entries against the fp64 oracle's compression of the same tokens
    b = int(np.argmax(length))
    nb = complete_blocks(cfg, int(length[b]))
    rk, rv = pipeline.compress_all(cfg, f64(inp["k"][b]), f64(inp["v"][b]), f64(inp["w_k"]), f64(inp["w_v"]),
                                   f64(inp["pe_k"]), f64(inp["pe_v"]), round_cmp=False)
    check_ulp(bf16_dev_to_f64(kcmp[b])[:, :nb], rk[:, :nb], f"{cfg.name} appended K_cmp")
    check_ulp(bf16_dev_to_f64(vcmp[b])[:, :nb], rv[:, :nb], f"{cfg.name} appended V_cmp")


def test_append_token_by_token_varlen():
    cfg = DECODE.replace(name="append_small", batch=5, seq_len=1024, seed=31)
    # empty, inside the first block, at a block edge, mid-cache, and near the capacity
    _grow(cfg, [0, 20, 47, 500, 1000], [1] * 40)


def test_append_chunks_and_saturation():
    cfg = DECODE.replace(name="append_chunks", batch=3, seq_len=1024, seed=32)
    # chunks that complete several blocks at once, then run past the capacity
    _grow(cfg, [0, 31, 990], [7, 16, 33, 1, 64])


def test_append_then_decode_equals_prefill_caches():
    cfg = DECODE.replace(name="append_decode", batch=2, seq_len=2048, seed=33)
    print("[case] append then decode", flush=True)
    inp = inputs.decode_inputs(cfg)
    K, V = dev_bf16(inp["k"]), dev_bf16(inp["v"])
    wk, wv, pk, pv = (dev_bf16(inp[n]) for n in ("w_k", "w_v", "pe_k", "pe_v"))
    q, gates = dev_bf16(inp["q"]), torch.as_tensor(inp["gates"], device="cuda")
    ref_k, ref_v = ops.compress(cfg, K, V, wk, wv, pk, pv)
    prep = ops.compress_prepare(cfg, wk, wv, pk, pv)
    start = 1500
    kc, vc = K.clone(), V.clone()
    kc[:, :, start:] = 0
    vc[:, :, start:] = 0
    kcmp, vcmp = ref_k.clone(), ref_v.clone()
    kcmp[:, :, complete_blocks(cfg, start):] = 0
    vcmp[:, :, complete_blocks(cfg, start):] = 0
    clen = dev_i32(np.full(cfg.batch, start, dtype=np.int32))
    for t in range(start, cfg.seq_len):
        ops.cache_append(cfg, K[:, :, t:t + 1].contiguous(), V[:, :, t:t + 1].contiguous(), kc, vc, clen, kcmp, vcmp,
                         prep)
    out_a, sel_a = ops.decode(cfg, q, kc, vc, clen, kcmp, vcmp, gates)
    out_r, sel_r = ops.decode(cfg, q, K, V, dev_i32(np.full(cfg.batch, cfg.seq_len, dtype=np.int32)), ref_k, ref_v,
                              gates)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_r)
    assert torch.equal(out_a, out_r)
