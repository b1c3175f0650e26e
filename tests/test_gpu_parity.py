"""GPU parity of every library call against the fp64 oracle (needs an MI355X).

Each call is checked on its own, with both sides fed identical inputs: the seeded
generator's draws, the oracle's own upstream results, or (in the chained prefill tests) the
GPU's upstream bytes after the oracle has checked them against its own.  Sizes span
several tiles plus ragged tails; the full-size workloads (8K, 64K, decode at 65536, MoBA
at 131072) are checked on sampled rows that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import pipeline
from dynamic_block_sparse_nsa_amd import inputs, ops
from dynamic_block_sparse_nsa_amd.configs import (TINY, P8K, P64K, DECODE, MOBA, BR_CMP, BR_SLC, BR_WIN, PHI_LINEAR,
                                                  PHI_MEAN, SCORE_CMP_OVERLAP)
from nsa_testlib import (GAP, bf16_dev_to_f64, bf16_ulp, check_close, check_selection, check_ulp, dev_bf16, dev_f32,
                         dev_i32, f64_to_dev_bf16, sample_rows)

pytestmark = pytest.mark.gpu

RAGGED = TINY.replace(name="ragged", seq_len=1000, seed=11)
RAGGED16 = P8K.replace(name="ragged16", seq_len=2085, seed=12)


def f64(bits):
    return inputs.bf16_bits_to_f64(bits)


def announce(msg):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------------------
# compression
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [TINY, RAGGED, P8K], ids=lambda c: c.name)
def test_compress_linear_all_blocks(cfg):
    announce(f"compress linear {cfg.name}")
    inp = inputs.prefill_inputs(cfg)
    kc, vc = ops.compress(cfg, dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_bf16(inp["w_k"]), dev_bf16(inp["w_v"]),
                          dev_bf16(inp["pe_k"]), dev_bf16(inp["pe_v"]))
    torch.cuda.synchronize()
    gk, gv = bf16_dev_to_f64(kc), bf16_dev_to_f64(vc)
    K, V = f64(inp["k"][0]), f64(inp["v"][0])
    rk, rv = pipeline.compress_all(cfg, K, V, f64(inp["w_k"]), f64(inp["w_v"]), f64(inp["pe_k"]), f64(inp["pe_v"]),
                                   round_cmp=False)
    check_ulp(gk[0], rk, f"{cfg.name} K_cmp")
    check_ulp(gv[0], rv, f"{cfg.name} V_cmp")


@pytest.mark.parametrize("T", [16384, 65536])
def test_compress_linear_64k_sampled_blocks(T):
    """Sampled blocks of the 64K workload's shapes at 16K and 64K tokens (the kernel takes two
    and four 16-row tiles per workgroup there; the all-blocks test at 8K covers one)."""
    cfg = P64K.replace(seq_len=T)
    announce(f"compress linear T={T} sampled")
    inp = inputs.prefill_inputs(cfg)
    kc, vc = ops.compress(cfg, dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_bf16(inp["w_k"]), dev_bf16(inp["w_v"]),
                          dev_bf16(inp["pe_k"]), dev_bf16(inp["pe_v"]))
    torch.cuda.synchronize()
    blocks = np.unique(np.concatenate([[0, 1, 63, 64, cfg.n_cmp - 1],
                                       np.random.default_rng(5).integers(0, cfg.n_cmp, 40)]))
    gk, gv = bf16_dev_to_f64(kc), bf16_dev_to_f64(vc)
    for g in range(cfg.num_kv_heads):
        rk = oracle.compress_linear(f64(inp["k"][0, g]), f64(inp["pe_k"]), f64(inp["w_k"]), 32, 16, blocks)
        rv = oracle.compress_linear(f64(inp["v"][0, g]), f64(inp["pe_v"]), f64(inp["w_v"]), 32, 16, blocks)
        check_ulp(gk[0, g, blocks], rk, f"T={T} K_cmp g{g}")
        check_ulp(gv[0, g, blocks], rv, f"T={T} V_cmp g{g}")


def test_compress_mean_moba_full():
    cfg = MOBA
    announce("compress mean moba 128k")
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    k = inputs._normal_bf16(rng, (1, cfg.num_kv_heads, cfg.seq_len, cfg.d_k))
    kc, _ = ops.compress(cfg, dev_bf16(k))
    torch.cuda.synchronize()
    g = bf16_dev_to_f64(kc)
    for h in range(cfg.num_kv_heads):
        ref = oracle.compress_mean(f64(k[0, h]), cfg.cmp_block, cfg.cmp_stride)
        check_ulp(g[0, h], ref, f"moba mean key h{h}")


@pytest.mark.parametrize("cfg", [
    TINY.replace(name="mean_d64_l32s16", seq_len=1000, num_kv_heads=2, d_k=64, d_v=64, cmp_block=32, cmp_stride=16,
                 phi=PHI_MEAN, seed=51),
    TINY.replace(name="mean_d192_l64s32", seq_len=777, num_kv_heads=3, d_k=192, d_v=128, cmp_block=64, cmp_stride=32,
                 slc_block=64, phi=PHI_MEAN, seed=52)], ids=lambda c: c.name)
def test_compress_mean_shapes(cfg):
    """Mean pooling for the other head dims, with overlapping blocks (s < l) and a ragged
    tail of tokens that no block covers: every block within one bf16 ulp of the fp64 mean."""
    announce(f"compress mean {cfg.name}")
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    k = inputs._normal_bf16(rng, (1, cfg.num_kv_heads, cfg.seq_len, cfg.d_k))
    kc, _ = ops.compress(cfg, dev_bf16(k))
    torch.cuda.synchronize()
    g = bf16_dev_to_f64(kc)
    assert g.shape == (1, cfg.num_kv_heads, cfg.n_cmp, cfg.d_k)
    for h in range(cfg.num_kv_heads):
        check_ulp(g[0, h], oracle.compress_mean(f64(k[0, h]), cfg.cmp_block, cfg.cmp_stride), f"{cfg.name} h{h}")


# ---------------------------------------------------------------------------
# compressed attention + selection
# ---------------------------------------------------------------------------
def _score_select_case(cfg, rows, use_oracle_cmp):
    inp = inputs.prefill_inputs(cfg)
    if use_oracle_cmp:
        Kc, Vc = pipeline.compress_all(cfg, f64(inp["k"][0]), f64(inp["v"][0]), f64(inp["w_k"]), f64(inp["w_v"]),
                                       f64(inp["pe_k"]), f64(inp["pe_v"]))
        kc_dev, vc_dev = f64_to_dev_bf16(Kc[None]), f64_to_dev_bf16(Vc[None])
    else:
        ckv = inputs.compressed_kv(cfg, seed=100 + cfg.seed)
        Kc, Vc = f64(ckv["k_cmp"][0]), f64(ckv["v_cmp"][0])
        kc_dev, vc_dev = dev_bf16(ckv["k_cmp"]), dev_bf16(ckv["v_cmp"])
    sel, lse, ocmp = ops.score_select(cfg, dev_bf16(inp["q"]), kc_dev, vc_dev, want_lse=True)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy()[0, rows]
    glse = lse.cpu().numpy()[0, rows]
    goc = ocmp.cpu().numpy()[0, rows]
    ref = oracle.score_select(cfg, f64(inp["q"][0, rows]), rows, Kc, Vc)
    check_selection(gsel, ref["sel"], ref["gap"], ref["scores"], rows, cfg, f"{cfg.name} selection")
    fin = np.isfinite(ref["lse"])
    assert (np.isneginf(glse[~fin])).all()
    assert np.abs(glse[fin] - ref["lse"][fin]).max() < 1e-4, np.abs(glse[fin] - ref["lse"][fin]).max()
    check_close(goc, ref["o_cmp"], f"{cfg.name} o_cmp")


@pytest.mark.parametrize("cfg", [TINY, RAGGED], ids=lambda c: c.name)
def test_score_select_all_rows_oracle_compressed(cfg):
    announce(f"score_select {cfg.name} all rows")
    _score_select_case(cfg, np.arange(cfg.seq_len, dtype=np.int32), use_oracle_cmp=True)


@pytest.mark.parametrize("cfg", [P8K, RAGGED16], ids=lambda c: c.name)
def test_score_select_mid(cfg):
    announce(f"score_select {cfg.name}")
    rows = np.unique(np.concatenate([np.arange(0, cfg.seq_len, 7), sample_rows(cfg.seq_len, 64, 1)])).astype(np.int32)
    _score_select_case(cfg, rows, use_oracle_cmp=False)


def test_score_select_64k_sampled():
    announce("score_select 64k sampled")
    _score_select_case(P64K, sample_rows(P64K.seq_len, 48, 2), use_oracle_cmp=False)


def test_select_from_scores_exact_ties():
    cfg = P8K.replace(seq_len=2048, num_kv_heads=2)
    announce("select_from_scores ties")
    rng = np.random.default_rng(9)
    sc = rng.integers(0, 4, size=(1, cfg.seq_len, 2, cfg.n_slc)).astype(np.float32)
    sel = ops.select_from_scores(cfg, dev_f32(sc))
    torch.cuda.synchronize()
    g = sel.cpu().numpy()[0]
    jc = np.repeat(np.arange(cfg.seq_len) // cfg.slc_block, 2)
    ref, _ = oracle.select_from_scores(sc[0].reshape(-1, cfg.n_slc), jc, cfg.top_n, cfg.n_init, cfg.n_local)
    np.testing.assert_array_equal(g.reshape(-1, cfg.top_n), ref)


# ---------------------------------------------------------------------------
# selected + window attention, gate
# ---------------------------------------------------------------------------
def _attn_case(cfg, rows, branches=None):
    cfg = cfg if branches is None else cfg.replace(branches=branches)
    inp = inputs.prefill_inputs(cfg)
    sel = inputs.block_lists(cfg, seed=200 + cfg.seed)
    oc = inputs.cmp_outputs(cfg, seed=300 + cfg.seed) if cfg.branches & 1 else None
    out = ops.sparse_attn_fwd(cfg, dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_i32(sel),
                              None if oc is None else dev_f32(oc), dev_f32(inp["gates"]))
    torch.cuda.synchronize()
    gout = bf16_dev_to_f64(out)[0, rows]
    ref = oracle.attend(cfg, f64(inp["q"][0, rows]), rows, f64(inp["k"][0]), f64(inp["v"][0]), sel[0, rows],
                        None if oc is None else oc[0, rows], inp["gates"][0, rows])
    check_close(gout, ref["out"], f"{cfg.name} output (branches {cfg.branches})")


@pytest.mark.parametrize("cfg", [TINY, RAGGED], ids=lambda c: c.name)
def test_sparse_attn_all_rows(cfg):
    announce(f"sparse_attn {cfg.name} all rows")
    _attn_case(cfg, np.arange(cfg.seq_len, dtype=np.int32))


@pytest.mark.parametrize("cfg", [P8K, RAGGED16], ids=lambda c: c.name)
def test_sparse_attn_mid(cfg):
    announce(f"sparse_attn {cfg.name}")
    _attn_case(cfg, sample_rows(cfg.seq_len, 200, 3))


def test_sparse_attn_64k_sampled():
    announce("sparse_attn 64k sampled")
    _attn_case(P64K, sample_rows(P64K.seq_len, 40, 4))


@pytest.mark.parametrize("branches", [BR_SLC, BR_WIN, BR_CMP], ids=["slc", "win", "cmp"])
def test_sparse_attn_single_branch(branches):
    announce(f"sparse_attn single branch {branches}")
    _attn_case(TINY, np.arange(TINY.seq_len, dtype=np.int32), branches=branches)


def test_sparse_attn_value_scales():
    """The attention kernel multiplies P by an fp16 copy of V scaled per (sequence, group) by
    a power of two.  Groups whose values are 1e5 times (beyond fp16's range unscaled) and
    1e-4 times those of others, in a batch of two: each group's heads within the output bar
    once both sides are divided by the group's factor."""
    cfg = TINY.replace(name="vscale", batch=2, seq_len=700, num_kv_heads=2, heads_per_group=4, d_k=128, d_v=128,
                       top_n=5, window=96, branches=BR_SLC | BR_WIN, seed=71)
    announce("sparse_attn value scales")
    inp = inputs.prefill_inputs(cfg)
    scale = np.array([[1e5, 1.0], [1e-4, 3.0]])   # [B, Hkv]
    v_dev = f64_to_dev_bf16(f64(inp["v"]) * scale[:, :, None, None])
    v = bf16_dev_to_f64(v_dev)                   # the values the kernel sees
    sel = inputs.block_lists(cfg, seed=271)
    out = ops.sparse_attn_fwd(cfg, dev_bf16(inp["q"]), dev_bf16(inp["k"]), v_dev, dev_i32(sel), None,
                              dev_f32(inp["gates"]))
    torch.cuda.synchronize()
    gout = bf16_dev_to_f64(out)
    rows = np.arange(cfg.seq_len, dtype=np.int32)
    G = cfg.heads_per_group
    for b in range(cfg.batch):
        ref = oracle.attend(cfg, f64(inp["q"][b]), rows, f64(inp["k"][b]), v[b], sel[b], None, inp["gates"][b])["out"]
        for g in range(cfg.num_kv_heads):
            hs = slice(g * G, (g + 1) * G)
            check_close(gout[b, :, hs] / scale[b, g], ref[:, hs] / scale[b, g], f"vscale b={b} g={g} x{scale[b, g]:g}")


# ---------------------------------------------------------------------------
# end to end: the GPU chain compress -> score_select -> sparse_attn_fwd, staged against
# the oracle at each step on the GPU's own upstream bytes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [TINY, RAGGED, RAGGED16, P8K, P64K], ids=lambda c: c.name)
def test_prefill_end_to_end(cfg):
    _prefill_end_to_end(cfg)


def _prefill_end_to_end(cfg, inp=None):
    """The whole prefill path as one chain on the GPU, each step against the oracle:
      * the GPU's compressed keys/values within one bf16 ulp of the oracle's compression of
        the same inputs (sampled blocks at 64K);
      * the oracle's scoring and selection run on the GPU's compressed key/value bytes: the
        GPU's block lists equal the oracle's on every (row, group) whose score gap is at
        least 1e-6, and are a valid selection on the others;
      * the gated output of every checked row within the output bar, the oracle attending
        with its own o_cmp and its own list (the GPU's list on near-tie rows, which are
        validated first).
    Rows: all of them up to 2100 tokens, else the edges plus 64 (64K) or 300 drawn ones.
    The fused call nsa_prefill_fwd must reproduce the three calls' outputs, lists, LSE and
    o_cmp bit for bit (same arithmetic, one launch)."""
    announce(f"end to end {cfg.name}")
    inp = inputs.prefill_inputs(cfg) if inp is None else inp
    args = [dev_bf16(inp[n]) for n in ("q", "k", "v", "w_k", "w_v", "pe_k", "pe_v")] + [dev_f32(inp["gates"])]
    r = ops.prefill(cfg, *args)
    # the fused call (nsa_prefill_fwd) runs the same arithmetic in one launch: identical bits
    rf = ops.prefill(cfg, *args, fused=True)
    torch.cuda.synchronize()
    for key in ("out", "sel", "lse", "o_cmp", "k_cmp", "v_cmp"):
        assert torch.equal(r[key], rf[key]), f"{cfg.name}: fused prefill differs from the three calls in {key}"
    del rf
    if cfg.seq_len <= 2100:
        rows = np.arange(cfg.seq_len, dtype=np.int32)
    else:
        rows = sample_rows(cfg.seq_len, 64 if cfg.seq_len > 20000 else 300, 6)
    gk_all, gv_all = bf16_dev_to_f64(r["k_cmp"]), bf16_dev_to_f64(r["v_cmp"])
    for b in range(cfg.batch):
        K, V = f64(inp["k"][b]), f64(inp["v"][b])
        # step 1 against the oracle's compression of the same bytes
        blocks = (np.arange(cfg.n_cmp) if cfg.n_cmp <= 600 else
                  np.unique(np.concatenate([[0, 1, cfg.n_cmp - 1],
                                            np.random.default_rng(b).integers(0, cfg.n_cmp, 48)])))
        for g in range(cfg.num_kv_heads):
            rk = oracle.compress_linear(K[g], f64(inp["pe_k"]), f64(inp["w_k"]), cfg.cmp_block, cfg.cmp_stride,
                                        blocks)
            rv = oracle.compress_linear(V[g], f64(inp["pe_v"]), f64(inp["w_v"]), cfg.cmp_block, cfg.cmp_stride,
                                        blocks)
            check_ulp(gk_all[b, g, blocks], rk, f"{cfg.name} b={b} g={g} chained K_cmp")
            check_ulp(gv_all[b, g, blocks], rv, f"{cfg.name} b={b} g={g} chained V_cmp")
        # steps 2-4 on the GPU's compressed bytes
        Kc, Vc = gk_all[b], gv_all[b]
        Qr = f64(inp["q"][b, rows])
        ss = oracle.score_select(cfg, Qr, rows, Kc, Vc)
        gsel = r["sel"][b].cpu().numpy()[rows]
        n_exact, n_tie = check_selection(gsel, ss["sel"], ss["gap"], ss["scores"], rows, cfg,
                                         f"{cfg.name} b={b} chained selection")
        glse = r["lse"][b].cpu().numpy()[rows]
        fin = np.isfinite(ss["lse"])
        assert np.isneginf(glse[~fin]).all()
        assert np.abs(glse[fin] - ss["lse"][fin]).max() < 1e-4, np.abs(glse[fin] - ss["lse"][fin]).max()
        check_close(r["o_cmp"][b].cpu().numpy()[rows], ss["o_cmp"], f"{cfg.name} b={b} chained o_cmp")
        # steps 5-7: the oracle's list, or the GPU's validated list where the two differ
        same = (gsel == ss["sel"]).all(axis=-1, keepdims=True)
        lists = np.where(same, ss["sel"], gsel).astype(np.int32)
        at = oracle.attend(cfg, Qr, rows, K, V, lists, ss["o_cmp"], inp["gates"][b, rows])
        gout = bf16_dev_to_f64(r["out"])[b, rows]
        check_close(gout, at["out"], f"{cfg.name} b={b} chained output ({n_exact} exact rows, {n_tie} near ties)")
        if cfg.seq_len <= 8192:
            # diagnostic only: the pure-fp64 chain (compressed keys never rounded to bf16)
            Kc64, Vc64 = pipeline.compress_all(cfg, K, V, f64(inp["w_k"]), f64(inp["w_v"]), f64(inp["pe_k"]),
                                               f64(inp["pe_v"]), round_cmp=False)
            ref64 = oracle.score_select(cfg, Qr, rows, Kc64, Vc64, want_ocmp=False)
            agree = (gsel == ref64["sel"]).all(axis=-1).mean()
            print(f"[diag] {cfg.name} b={b} selection agreement with the pure-fp64 chain: {agree:.5f}", flush=True)


@pytest.mark.parametrize("T", [1, 20, 31])
def test_prefill_shorter_than_one_compressed_block(T):
    """Sequences with no complete compressed block (T < l = 32): o_cmp = 0 and LSE = -inf on
    every row, the selection holds the forced blocks only, and the selected and window
    branches and the gated sum are as usual; the fused call equals the three calls."""
    cfg = TINY.replace(name=f"short{T}", seq_len=T, seed=60 + T)
    announce(f"prefill T={T} < cmp_block")
    inp = inputs.prefill_inputs(cfg)
    args = [dev_bf16(inp[n]) for n in ("q", "k", "v", "w_k", "w_v", "pe_k", "pe_v")] + [dev_f32(inp["gates"])]
    r = ops.prefill(cfg, *args)
    rf = ops.prefill(cfg, *args, fused=True)
    torch.cuda.synchronize()
    for key in ("out", "sel", "lse", "o_cmp"):
        assert torch.equal(r[key], rf[key]), f"T={T}: fused prefill differs from the three calls in {key}"
    rows = np.arange(T, dtype=np.int32)
    Kc, Vc = pipeline.compress_all(cfg, f64(inp["k"][0]), f64(inp["v"][0]), f64(inp["w_k"]), f64(inp["w_v"]),
                                   f64(inp["pe_k"]), f64(inp["pe_v"]))
    assert Kc.shape[1] == 0
    ref = pipeline.forward_rows(cfg, f64(inp["q"][0]), f64(inp["k"][0]), f64(inp["v"][0]), Kc, Vc, inp["gates"][0],
                                rows)
    np.testing.assert_array_equal(r["sel"][0].cpu().numpy(), ref["sel"])
    assert np.isneginf(r["lse"].cpu().numpy()).all()
    assert not r["o_cmp"].any().item()
    check_close(bf16_dev_to_f64(r["out"])[0], ref["out"], f"T={T} output")


# Other shapes the kernels support: group sizes 1, 2, 8; head dims 128/128 and 64/64;
# other block geometries, top-n and windows; a batch of two; every row checked.
SHAPES = [
    TINY.replace(name="g2_d128_b2", batch=2, seq_len=1500, num_kv_heads=2, heads_per_group=2, d_k=128, d_v=128,
                 top_n=8, window=256, seed=41),
    TINY.replace(name="g8_d64_l64", seq_len=2100, num_kv_heads=1, heads_per_group=8, d_k=64, d_v=64,
                 cmp_block=64, cmp_stride=32, slc_block=128, top_n=6, n_init=2, n_local=1, window=200, seed=42),
    TINY.replace(name="g1_d128_nsa", seq_len=1200, num_kv_heads=3, heads_per_group=1, d_k=128, d_v=128,
                 top_n=5, window=100, seed=43),
    TINY.replace(name="g16_d192_w0", seq_len=900, num_kv_heads=1, heads_per_group=16, d_k=192, d_v=128,
                 top_n=4, window=0, branches=3, seed=44),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_prefill_shape_matrix(cfg):
    _prefill_end_to_end(cfg)


def _ramped_keys(inp, top=16.0, v_scale=1.0):
    """The inputs with every key row scaled from x1 at the first token to x`top` at the last
    (bf16 again), so that scores grow along the sequence: the largest scaled scores of the
    last keys lie tens of log2 units above those of the first ones.  v_scale scales the
    values: attention this peaked makes a branch's output nearly one value row, and the
    gated sum of three such rows reaches |O| ~ 13, where half a bf16 ulp (2^-5) exceeds the
    output bar's absolute tolerance; 1/4 keeps |O| below 4 (half an ulp 2^-8)."""
    k = f64(inp["k"])
    T = k.shape[2]
    ramp = 1.0 + (top - 1.0) * np.arange(T) / max(T - 1, 1)
    out = dict(inp)
    out["k"] = inputs.f32_to_bf16_bits((k * ramp[None, None, :, None]).astype(np.float32))
    if v_scale != 1.0:
        out["v"] = inputs.f32_to_bf16_bits((f64(inp["v"]) * v_scale).astype(np.float32))
    return out


def test_prefill_growing_scores():
    """Keys growing along the sequence (_ramped_keys): later chunks exceed the softmax
    references that the kernels move lazily (by more than 2^8 in the selected / window
    branches, by more than 2^32 in the sum of the compressed branch's statistics), so the
    paths that move a reference and rescale run; the whole chain still matches the oracle
    on every row of the 64K workload's shapes."""
    cfg = RAGGED16.replace(name="kramp16", seed=81)
    _prefill_end_to_end(cfg, _ramped_keys(inputs.prefill_inputs(cfg), v_scale=0.25))


DECODE_SHAPES = [
    DECODE.replace(name="dec_g4_d128", batch=3, seq_len=3000, num_kv_heads=2, heads_per_group=4, d_k=128, d_v=128,
                   top_n=8, window=256, seed=51),
    DECODE.replace(name="dec_g8_d64_nowin", batch=2, seq_len=2500, num_kv_heads=1, heads_per_group=8, d_k=64,
                   d_v=64, window=0, branches=3, seed=52),
    DECODE.replace(name="dec_g16_l64", batch=2, seq_len=5000, cmp_block=64, cmp_stride=32, slc_block=128,
                   top_n=12, window=300, seed=53),
]


@pytest.mark.parametrize("cfg", DECODE_SHAPES, ids=lambda c: c.name)
def test_decode_shape_matrix(cfg):
    announce(f"decode shape {cfg.name}")
    rng = np.random.default_rng(cfg.seed)
    lens = np.concatenate([[cfg.seq_len], rng.integers(1, cfg.seq_len + 1, cfg.batch - 1)]).astype(np.int32)
    _decode_case(cfg, lens, cmp_from_oracle=True)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def _decode_case(cfg, cache_len, cmp_from_oracle, v_scale=1.0):
    inp = inputs.decode_inputs(cfg, cache_len=cache_len)
    if v_scale != 1.0:
        inp["v"] = inputs.f32_to_bf16_bits((f64(inp["v"]) * v_scale).astype(np.float32))
    if cmp_from_oracle:
        per_b = [pipeline.compress_all(cfg, f64(inp["k"][b]), f64(inp["v"][b]), f64(inp["w_k"]), f64(inp["w_v"]),
                                       f64(inp["pe_k"]), f64(inp["pe_v"])) for b in range(cfg.batch)]
        kc_f64 = np.stack([x[0] for x in per_b])
        vc_f64 = np.stack([x[1] for x in per_b])
        kc_dev, vc_dev = f64_to_dev_bf16(kc_f64), f64_to_dev_bf16(vc_f64)
    else:
        ckv = inputs.compressed_kv(cfg, seed=400 + cfg.seed)
        kc_f64, vc_f64 = f64(ckv["k_cmp"]), f64(ckv["v_cmp"])
        kc_dev, vc_dev = dev_bf16(ckv["k_cmp"]), dev_bf16(ckv["v_cmp"])
    out, sel = ops.decode(cfg, dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_i32(inp["cache_len"]),
                          kc_dev, vc_dev, dev_f32(inp["gates"]))
    torch.cuda.synchronize()
    gout = bf16_dev_to_f64(out)
    gsel = sel.cpu().numpy()
    refs_out, refs_sel, gaps, scores, pos = [], [], [], [], []
    for b in range(cfg.batch):
        t = int(inp["cache_len"][b]) - 1
        q = f64(inp["q"][b])[None]
        ss = oracle.score_select(cfg, q, [t], kc_f64[b], vc_f64[b])
        at = oracle.attend(cfg, q, [t], f64(inp["k"][b]), f64(inp["v"][b]), ss["sel"], ss["o_cmp"],
                           inp["gates"][b][None])
        refs_out.append(at["out"][0]); refs_sel.append(ss["sel"][0]); gaps.append(ss["gap"][0])
        scores.append(ss["scores"][0]); pos.append(t)
    check_selection(gsel, np.stack(refs_sel), np.stack(gaps), np.stack(scores), np.array(pos), cfg,
                    f"{cfg.name} decode selection")
    check_close(gout / v_scale, np.stack(refs_out) / v_scale, f"{cfg.name} decode output")


def test_decode_large_values():
    """Values 3000 times the usual scale: each decode partial is a sum over up to 256 keys,
    so it is stored normalized by its own softmax sum to stay inside fp16's range."""
    cfg = DECODE.replace(name="decode_large_v", batch=3, seq_len=4096, seed=24)
    announce("decode large values")
    _decode_case(cfg, np.array([4096, 2000, 700], dtype=np.int32), cmp_from_oracle=True, v_scale=3000.0)


def test_decode_varlen_small():
    cfg = DECODE.replace(name="decode_small", batch=6, seq_len=4096, seed=21)
    announce("decode varlen small")
    _decode_case(cfg, np.array([4096, 1, 31, 32, 100, 2049], dtype=np.int32), cmp_from_oracle=True)


def test_decode_varlen_multi_round():
    # 32 x 32768: the compressed branch's workgroups take two 256-key splits each; the
    # lengths put split and workgroup boundaries inside, at and just past the visible keys
    cfg = DECODE.replace(name="decode_varlen_rounds", seq_len=32768, seed=29)
    fixed = [32768, 1, 17, 31, 32, 33, 4111, 4112, 4127, 8207, 8208, 8223, 16384, 32767]
    rng = np.random.default_rng(29)
    lens = np.array(fixed + list(rng.integers(1, 32769, cfg.batch - len(fixed))), dtype=np.int32)
    announce("decode varlen multi-round 32 x 32768")
    _decode_case(cfg, lens, cmp_from_oracle=False)


def test_decode_full():
    announce("decode full 32 x 65536")
    _decode_case(DECODE, None, cmp_from_oracle=False)


def test_decode_equals_prefill_last_row():
    cfg = P8K.replace(name="dp", batch=2, seq_len=2048, seed=23)
    announce("decode == prefill last row")
    inp = inputs.prefill_inputs(cfg)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    wk, wv, pk, pv = (dev_bf16(inp[n]) for n in ("w_k", "w_v", "pe_k", "pe_v"))
    gates = dev_f32(inp["gates"])
    r = ops.prefill(cfg, q, k, v, wk, wv, pk, pv, gates)
    dcfg = cfg.replace(decode=True)
    L = cfg.seq_len
    out, sel = ops.decode(dcfg, q[:, L - 1].contiguous(), k, v, dev_i32(np.full(cfg.batch, L)), r["k_cmp"],
                          r["v_cmp"], gates[:, L - 1].contiguous())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), r["sel"].cpu().numpy()[:, L - 1])
    # Both paths round an fp32 result with an absolute arithmetic error of about 1e-3 to
    # bf16, so two values may sit on either side of a rounding midpoint: they may differ by
    # one ulp of the larger magnitude plus the two arithmetic errors.
    got, want = bf16_dev_to_f64(out), bf16_dev_to_f64(r["out"])[:, L - 1]
    check_close(got, want, "decode vs prefill row", atol=2e-2, rel=2e-3)
    lim = bf16_ulp(np.maximum(np.abs(got), np.abs(want))) + 2e-3
    assert (np.abs(got - want) <= lim).all(), np.abs(got - want).max()


# ---------------------------------------------------------------------------
# MoBA mode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,top_n", [(8192, 3), (MOBA.seq_len, 3), (1 << 20, 3), (8192, 8)],
                         ids=["8k", "128k", "1m", "8k_top8"])
def test_moba(T, top_n):
    """MoBA mode at 8K, at the 128K workload, and at 1M tokens (2048 blocks of 512: the
    longest context the selection supports), on sampled rows.  Top-3 selects inside the
    scoring kernel; top-8 (7 free picks) goes through the scores workspace."""
    cfg = MOBA.replace(seq_len=T, top_n=top_n)
    announce(f"moba {T} top{top_n}")
    inp = inputs.prefill_inputs(cfg)
    Kbar = pipeline.compress_all(cfg, f64(inp["k"][0]), None, None, None, None, None)[0]
    rows = sample_rows(T, 40, 7, lp=512, l=512)
    sel, _, _ = ops.score_select(cfg, dev_bf16(inp["q"]), f64_to_dev_bf16(Kbar[None]))
    torch.cuda.synchronize()
    ref = oracle.score_select(cfg, f64(inp["q"][0, rows]), rows, Kbar)
    check_selection(sel.cpu().numpy()[0, rows], ref["sel"], ref["gap"], ref["scores"], rows, cfg, f"moba{T} selection")
    lists = inputs.block_lists(cfg, seed=500, positions=None) if T <= 8192 else None
    if lists is None:
        lists = inputs.block_lists(cfg.replace(seq_len=T), seed=500)
    args = (dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_i32(lists))
    out = ops.sparse_attn_fwd(cfg, *args)
    torch.cuda.synchronize()
    at = oracle.attend(cfg, f64(inp["q"][0, rows]), rows, f64(inp["k"][0]), f64(inp["v"][0]), lists[0, rows])
    check_close(bf16_dev_to_f64(out)[0, rows], at["out"], f"moba{T} output")
    # the block lists are filled with atomics, so a second run groups the queries of a block
    # into work items differently; each (query, slot) result must not depend on its companions
    out2 = ops.sparse_attn_fwd(cfg, *args)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), f"moba{T}: the output differs between two runs"


@pytest.mark.parametrize("top_n,T", [(2, 8192), (3, 8192), (5, 8192), (3, 8100)],
                         ids=["picks1", "picks2", "picks4", "picks2_ragged"])
def test_moba_fused_selection_exact_ties(top_n, T):
    """The fused MoBA scoring + selection (one, two or four free picks per row) on integer
    queries and keys, so that every score is an exact small integer on both sides and equal
    scores are common (blocks repeat in pairs): the lists equal the oracle's on every row and
    head, the lower block index winning each tie.  T = 8100 ends inside a block and inside a
    workgroup's 64 tokens (rows past T, an own block with no mean key)."""
    cfg = MOBA.replace(name=f"moba_ties{top_n}_{T}", seq_len=T, top_n=top_n, num_kv_heads=4)
    announce(f"moba fused selection, exact ties, top{top_n}, T={T}")
    rng = np.random.default_rng(70 + top_n)
    Hkv, d, lp = cfg.num_kv_heads, cfg.d_k, cfg.slc_block
    blocks = rng.integers(-2, 3, size=(Hkv, -(-T // lp), d)).astype(np.float64)
    blocks[:, 1::2] = blocks[:, 0::2]   # blocks 2i and 2i+1 equal: their scores tie exactly
    K = np.repeat(blocks, lp, axis=1)[:, :T]   # every row of a block equal: its mean is exact
    Q = rng.integers(-2, 3, size=(T, Hkv, d)).astype(np.float64)
    kbar, _ = ops.compress(cfg, f64_to_dev_bf16(K[None]))
    sel, _, _ = ops.score_select(cfg, f64_to_dev_bf16(Q[None]), kbar)
    torch.cuda.synchronize()
    Kbar = pipeline.compress_all(cfg, K, None, None, None, None, None)[0]
    np.testing.assert_array_equal(bf16_dev_to_f64(kbar)[0], Kbar)
    ref = oracle.score_select(cfg, Q, np.arange(T, dtype=np.int32), Kbar)
    np.testing.assert_array_equal(sel.cpu().numpy()[0], ref["sel"])


def test_block_major_large_values():
    """The block-major MoBA schedule keeps its per-slot partials in fp16 in V's scaled units,
    so values far beyond fp16's range (1e5) pass; every row of a ragged batch of two."""
    cfg = MOBA.replace(name="bm_large_v", batch=2, seq_len=900, num_kv_heads=2, cmp_block=64, cmp_stride=64,
                       slc_block=64, top_n=3, seed=23)
    announce("block-major large values")
    inp = inputs.prefill_inputs(cfg)
    v_dev = f64_to_dev_bf16(f64(inp["v"]) * 1e5)
    v = bf16_dev_to_f64(v_dev)
    lists = inputs.block_lists(cfg, seed=601)
    out = ops.sparse_attn_fwd(cfg, dev_bf16(inp["q"]), dev_bf16(inp["k"]), v_dev, dev_i32(lists))
    torch.cuda.synchronize()
    gout = bf16_dev_to_f64(out)
    rows = np.arange(cfg.seq_len, dtype=np.int32)
    for b in range(cfg.batch):
        ref = oracle.attend(cfg, f64(inp["q"][b]), rows, f64(inp["k"][b]), v[b], lists[b])["out"]
        check_close(gout[b] / 1e5, ref / 1e5, f"block-major large values b={b}")


@pytest.mark.parametrize("case", ["b2_lp64_gated", "lp128_own_optional", "top1", "top2", "top12", "top32", "ramp"])
def test_block_major_all_rows(case):
    """G = 1 with only the selected branch runs the block-major schedule (per-block query
    lists, per-slot partials, merge); every row of a ragged batch is checked.  "ramp": keys
    growing x1 -> x16 along the sequence, so within a 512-token block later tiles exceed a
    column's lazily moved softmax reference and it moves."""
    if case == "b2_lp64_gated":
        cfg = MOBA.replace(name=case, batch=2, seq_len=1000, num_kv_heads=3, cmp_block=64, cmp_stride=64,
                           slc_block=64, top_n=3, seed=21)
    elif case == "lp128_own_optional":   # the own block is not forced, so some lists lack it
        cfg = MOBA.replace(name=case, batch=1, seq_len=1500, num_kv_heads=2, cmp_block=128, cmp_stride=128,
                           slc_block=128, top_n=4, n_local=0, n_init=1, phi=PHI_LINEAR,
                           score_mode=SCORE_CMP_OVERLAP, seed=22)
    elif case == "ramp":
        cfg = MOBA.replace(name=case, batch=1, seq_len=3000, num_kv_heads=2, seed=29)
    elif case in ("top1", "top2"):   # the merge's one- and two-slot forms
        n = int(case[3:])
        cfg = MOBA.replace(name=case, batch=1, seq_len=1800, num_kv_heads=2, cmp_block=64, cmp_stride=64,
                           slc_block=64, top_n=n, seed=40 + n)
    else:   # longer lists: the merge's 8-slot and 32-slot forms (ragged, 64-token blocks)
        n = 12 if case == "top12" else 32
        cfg = MOBA.replace(name=case, batch=1, seq_len=2500, num_kv_heads=2, cmp_block=64, cmp_stride=64,
                           slc_block=64, top_n=n, seed=24 + n)
    announce(f"block-major {case}")
    inp = inputs.prefill_inputs(cfg)
    if case == "ramp":
        inp = _ramped_keys(inp)
    lists = inputs.block_lists(cfg, seed=600)
    gates = None
    if case == "b2_lp64_gated":
        gates = np.random.Generator(np.random.PCG64(7)).standard_normal(
            (cfg.batch, cfg.seq_len, cfg.num_heads, 3)).astype(np.float32)
    out = ops.sparse_attn_fwd(cfg, dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_i32(lists),
                              None, None if gates is None else dev_f32(gates))
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out)
    rows = np.arange(cfg.seq_len, dtype=np.int32)
    for b in range(cfg.batch):
        at = oracle.attend(cfg, f64(inp["q"][b]), rows, f64(inp["k"][b]), f64(inp["v"][b]), lists[b],
                           gates=None if gates is None else gates[b])
        check_close(got[b], at["out"], f"{case} batch {b} output")


# ---------------------------------------------------------------------------
# dense causal attention (the comparison kernel)
# ---------------------------------------------------------------------------
def _full_case(cfg, rows, inp=None):
    inp = inputs.prefill_inputs(cfg) if inp is None else inp
    out = ops.full_attn_fwd(cfg, dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]))
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out)[0, rows]
    ref = np.zeros_like(got)
    for h in range(cfg.num_heads):
        g = h // cfg.heads_per_group
        ref[:, h] = oracle.causal_attention_rows(f64(inp["q"][0, rows, h]), rows, f64(inp["k"][0, g]),
                                                 f64(inp["v"][0, g]), cfg.scale)
    check_close(got, ref, f"{cfg.name} dense causal attention")


@pytest.mark.parametrize("cfg", [TINY, RAGGED], ids=lambda c: c.name)
def test_full_attn_all_rows(cfg):
    announce(f"dense attention {cfg.name} all rows")
    _full_case(cfg, np.arange(cfg.seq_len, dtype=np.int32))


def test_full_attn_growing_scores():
    """Dense causal attention on keys growing along the sequence: its lazily moved softmax
    reference moves (and rescales) on later tiles; every row against the oracle."""
    cfg = RAGGED16.replace(name="kramp16_dense", seed=82)
    announce("dense attention growing scores")
    _full_case(cfg, np.arange(cfg.seq_len, dtype=np.int32), _ramped_keys(inputs.prefill_inputs(cfg)))


@pytest.mark.parametrize("cfg", [P8K, RAGGED16, P64K], ids=lambda c: c.name)
def test_full_attn_sampled(cfg):
    announce(f"dense attention {cfg.name} sampled rows")
    _full_case(cfg, sample_rows(cfg.seq_len, 24 if cfg.seq_len > 10000 else 48, 8))


def test_select_all_blocks_equals_dense_attention_on_gpu():
    """Selecting every block makes the selected branch full causal attention (sunshychen.top);
    checked GPU against GPU on 2048 tokens, 32 blocks of 64."""
    cfg = P8K.replace(name="all32", seq_len=2048, top_n=32, branches=BR_SLC, seed=27)
    announce("select-all == dense attention (GPU)")
    inp = inputs.prefill_inputs(cfg)
    jc = np.arange(cfg.seq_len) // cfg.slc_block
    sel = np.where(np.arange(cfg.top_n)[None, :] <= jc[:, None], np.arange(cfg.top_n)[None, :], -1).astype(np.int32)
    sel = np.broadcast_to(sel[None, :, None, :], (1, cfg.seq_len, cfg.num_kv_heads, cfg.top_n)).copy()
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    slc = ops.sparse_attn_fwd(cfg, q, k, v, dev_i32(sel))
    full = ops.full_attn_fwd(cfg, q, k, v)
    torch.cuda.synchronize()
    a, b = bf16_dev_to_f64(slc), bf16_dev_to_f64(full)
    check_close(a, b, "select-all vs dense", atol=2e-2, rel=2e-3)
    # two GPU paths with ~1e-3 arithmetic error each, rounded to bf16
    lim = bf16_ulp(np.maximum(np.abs(a), np.abs(b))) + 2e-3
    assert (np.abs(a - b) <= lim).all(), np.abs(a - b).max()


# ---------------------------------------------------------------------------
# the pages' special cases, run on the GPU
# ---------------------------------------------------------------------------
def test_gpu_select_all_is_full_causal_and_window_only_is_swa():
    cfg = TINY.replace(top_n=16, branches=BR_SLC)
    announce("gpu special cases")
    inp = inputs.prefill_inputs(cfg)
    T = cfg.seq_len
    allsel = np.full((1, T, 1, 16), -1, dtype=np.int32)
    for t in range(T):
        allsel[0, t, 0, :t // 64 + 1] = np.arange(t // 64 + 1)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    o1 = bf16_dev_to_f64(ops.sparse_attn_fwd(cfg, q, k, v, dev_i32(allsel)))[0]
    cw = cfg.replace(branches=BR_WIN)
    o2 = bf16_dev_to_f64(ops.sparse_attn_fwd(cw, q, k, v))[0]
    Q, K, V = f64(inp["q"][0]), f64(inp["k"][0, 0]), f64(inp["v"][0, 0])
    for h in range(cfg.num_heads):
        check_close(o1[:, h], oracle.causal_attention(Q[:, h], K, V, cfg.scale), f"select-all head {h}")
        check_close(o2[:, h], oracle.causal_attention(Q[:, h], K, V, cfg.scale, window=cfg.window), f"window head {h}")


def test_gpu_causality_and_determinism():
    cfg = P8K.replace(seq_len=2048, seed=31)
    announce("gpu causality + determinism")
    inp = inputs.prefill_inputs(cfg)
    args = [dev_bf16(inp[n]) for n in ("q", "k", "v", "w_k", "w_v", "pe_k", "pe_v")] + [dev_f32(inp["gates"])]
    a = ops.prefill(cfg, *args)
    b = ops.prefill(cfg, *args)
    torch.cuda.synchronize()
    for key in ("out", "sel", "o_cmp", "k_cmp", "v_cmp"):
        assert torch.equal(a[key], b[key]), key
    t0 = 1500
    pert = [x.clone() for x in args]
    g = torch.Generator(device="cpu").manual_seed(1)
    pert[0][:, t0 + 1:] = torch.randn(pert[0][:, t0 + 1:].shape, generator=g).to(pert[0])
    pert[1][:, :, t0 + 1:] = (5 * torch.randn(pert[1][:, :, t0 + 1:].shape, generator=g)).to(pert[1])
    pert[2][:, :, t0 + 1:] = (5 * torch.randn(pert[2][:, :, t0 + 1:].shape, generator=g)).to(pert[2])
    c = ops.prefill(cfg, *pert)
    torch.cuda.synchronize()
    assert torch.equal(a["out"][:, :t0 + 1], c["out"][:, :t0 + 1])
    assert torch.equal(a["sel"][:, :t0 + 1], c["sel"][:, :t0 + 1])
