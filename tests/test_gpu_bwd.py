"""GPU parity of the backward pass (nsa_sparse_attn_bwd, nsa_compress_bwd) against the fp64
oracle (oracle.nsa_bwd, oracle.compress_linear_bwd), whose own pins are in
test_oracle_bwd_pins.py.

Staged like the forward: the oracle is fed the exact bf16 inputs, the GPU's compressed keys
and values and the GPU's selection (the selection passes no gradient).  Gradients are fp32;
the bar is the output bar applied to gradients scaled by their largest magnitude: max abs
error <= 2e-2 * max|ref| and relative L2 error <= 5e-3.  Expected error: the compressed
branch's o_cmp enters D_cmp = sigma <dO, o_cmp> with its forward rounding (fp16
probabilities against an fp16 value copy, 2^-11 relative), probabilities and dS enter the
MFMA as bf16 high + low parts (about 2^-17), everything else is fp32 accumulation, so the
expected relative error is about 1e-3 at worst, well inside the bar.
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_block_sparse_nsa_amd import inputs, ops
from dynamic_block_sparse_nsa_amd.configs import (TINY, P8K, P64K, BR_ALL, BR_CMP, BR_SLC, BR_WIN, PHI_MEAN,
                                                  SCORE_MEAN_DOT)
from nsa_testlib import bf16_dev_to_f64, check_close, dev_bf16, sample_rows, OUT_ATOL, OUT_REL_L2

pytestmark = pytest.mark.gpu

f64 = inputs.bf16_bits_to_f64


def check_grad(gpu, ref, what):
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    scale = float(np.abs(ref).max())
    if scale == 0.0:
        # an exactly zero gradient (e.g. a single visible compressed key: its probability is 1
        # for every row, so dS = 0): the GPU may only show rounding noise
        print(f"[parity] {what}: reference exactly zero, GPU max abs {np.abs(gpu).max():.3e}", flush=True)
        assert np.abs(gpu).max() <= 1e-4, what
        return
    check_close(gpu / scale, ref / scale, what, atol=OUT_ATOL, rel=OUT_REL_L2)


GQA = TINY.replace(name="bwd_gqa16", num_kv_heads=2, heads_per_group=16, d_k=192, d_v=128, top_n=8, window=256,
                   fp32_inputs=False, seed=41)
RAGGED = TINY.replace(name="bwd_ragged", seq_len=1000, num_kv_heads=2, heads_per_group=8, d_k=128, d_v=128, top_n=6,
                      window=200, fp32_inputs=False, seed=42)
LP128 = TINY.replace(name="bwd_lp128", seq_len=1536, num_kv_heads=1, heads_per_group=16, d_k=64, d_v=64,
                     slc_block=128, top_n=5, window=96, fp32_inputs=False, seed=43)
LP32 = TINY.replace(name="bwd_lp32", seq_len=700, num_kv_heads=1, heads_per_group=2, d_k=64, d_v=64, slc_block=32,
                    cmp_block=16, cmp_stride=8, top_n=7, n_init=2, n_local=2, window=64, fp32_inputs=False, seed=44)
# (config, with gates, training forward: the backward reads the saved branch statistics)
CASES = [
    (TINY.replace(fp32_inputs=False, seed=40), True, False),
    (TINY.replace(fp32_inputs=False, seed=40), True, True),
    (GQA, True, False),
    (GQA, True, True),
    (RAGGED, True, False),
    (RAGGED, True, True),
    (LP128, True, False),
    (LP32, False, False),
    (LP32, False, True),
    (GQA.replace(name="bwd_slc_only", branches=BR_SLC), False, False),
    (GQA.replace(name="bwd_cmp_only", branches=BR_CMP), True, False),
    (RAGGED.replace(name="bwd_win_only", branches=BR_WIN), True, True),
    # edges: one compressed block and one selection block; a window longer than the
    # sequence; one query head per group with all three branches
    (TINY.replace(name="bwd_short", seq_len=40, window=16, fp32_inputs=False, seed=49), True, True),
    (RAGGED.replace(name="bwd_wide_window", seq_len=200, window=512, seed=50), True, False),
    (TINY.replace(name="bwd_g1", num_kv_heads=3, heads_per_group=1, seq_len=700, fp32_inputs=False, seed=51), True,
     True),
]


def _run(cfg, with_gates, train=False):
    print(f"[case] backward {cfg.name} T={cfg.seq_len} Hkv={cfg.num_kv_heads} G={cfg.heads_per_group} "
          f"d={cfg.d_k}/{cfg.d_v} br={cfg.branches} gates={with_gates} train={train}", flush=True)
    inp = inputs.prefill_inputs(cfg)
    dO_bits = inputs.grad_output(cfg)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    wk, wv, pk, pv = ((dev_bf16(inp[n]) if cfg.phi == 0 else None) for n in ("w_k", "w_v", "pe_k", "pe_v"))
    gates = torch.as_tensor(inp["gates"], device="cuda") if with_gates else None
    dO = dev_bf16(dO_bits)
    fwd = ops.prefill(cfg, q, k, v, wk, wv, pk, pv, gates, train=train)
    g = ops.backward(cfg, fwd, q, k, v, wk, wv, pk, pv, gates, dO)
    torch.cuda.synchronize()
    return inp, dO_bits, fwd, g


@pytest.mark.parametrize("cfg,with_gates,train", CASES,
                         ids=[c.name + ("_g" if wg else "") + ("_train" if tr else "") for c, wg, tr in CASES])
def test_backward_matches_oracle(cfg, with_gates, train):
    inp, dO_bits, fwd, g = _run(cfg, with_gates, train)
    use_c = bool(cfg.branches & 1)
    b = 0
    kc = bf16_dev_to_f64(fwd["k_cmp"][b]) if use_c else None
    vc = bf16_dev_to_f64(fwd["v_cmp"][b]) if use_c else None
    sel = fwd["sel"][b].cpu().numpy()
    gates = inp["gates"][b].astype(np.float64) if with_gates else None
    ref = oracle.nsa_bwd(cfg, f64(inp["q"][b]), f64(inp["k"][b]), f64(inp["v"][b]), kc, vc, sel, gates,
                         f64(dO_bits[b]))
    name = cfg.name
    check_grad(g["dq"][b].cpu().numpy(), ref["dq"], f"{name} dQ")
    if with_gates:
        check_grad(g["dgates"][b].cpu().numpy(), ref["dgates"], f"{name} dgates")
    if use_c:
        check_grad(g["dk_cmp"][b].cpu().numpy(), ref["dkc"], f"{name} dK_cmp")
        check_grad(g["dv_cmp"][b].cpu().numpy(), ref["dvc"], f"{name} dV_cmp")
        # the block map's backward on the oracle's dK_cmp / dV_cmp (staged through the GPU's)
        dk_tot, dv_tot = ref["dk"].copy(), ref["dv"].copy()
        dwk = np.zeros(inp["w_k"].shape)
        dwv = np.zeros(inp["w_v"].shape)
        dpk = np.zeros(inp["pe_k"].shape)
        dpv = np.zeros(inp["pe_v"].shape)
        gk = g["dk_cmp"][b].cpu().numpy().astype(np.float64)
        gv = g["dv_cmp"][b].cpu().numpy().astype(np.float64)
        for h in range(cfg.num_kv_heads):
            rk = oracle.compress_linear_bwd(f64(inp["k"][b, h]), f64(inp["pe_k"]), f64(inp["w_k"]), gk[h],
                                            cfg.cmp_block, cfg.cmp_stride)
            rv = oracle.compress_linear_bwd(f64(inp["v"][b, h]), f64(inp["pe_v"]), f64(inp["w_v"]), gv[h],
                                            cfg.cmp_block, cfg.cmp_stride)
            dk_tot[h] += rk["dx"]
            dv_tot[h] += rv["dx"]
            dwk += rk["dw"]
            dwv += rv["dw"]
            dpk += rk["dpe"]
            dpv += rv["dpe"]
        check_grad(g["dk"][b].cpu().numpy(), dk_tot, f"{name} dK (all branches)")
        check_grad(g["dv"][b].cpu().numpy(), dv_tot, f"{name} dV (all branches)")
        check_grad(g["dw_k"].cpu().numpy(), dwk, f"{name} dW_k")
        check_grad(g["dw_v"].cpu().numpy(), dwv, f"{name} dW_v")
        check_grad(g["dpe_k"].cpu().numpy(), dpk, f"{name} dpe_k")
        check_grad(g["dpe_v"].cpu().numpy(), dpv, f"{name} dpe_v")
    else:
        check_grad(g["dk"][b].cpu().numpy(), ref["dk"], f"{name} dK")
        check_grad(g["dv"][b].cpu().numpy(), ref["dv"], f"{name} dV")


def test_backward_batch_two():
    """Two sequences: every gradient of the second batch element against the oracle."""
    cfg = RAGGED.replace(name="bwd_batch2", batch=2, seed=45)
    inp, dO_bits, fwd, g = _run(cfg, True)
    for b in range(2):
        ref = oracle.nsa_bwd(cfg, f64(inp["q"][b]), f64(inp["k"][b]), f64(inp["v"][b]),
                             bf16_dev_to_f64(fwd["k_cmp"][b]), bf16_dev_to_f64(fwd["v_cmp"][b]),
                             fwd["sel"][b].cpu().numpy(), inp["gates"][b].astype(np.float64), f64(dO_bits[b]))
        check_grad(g["dq"][b].cpu().numpy(), ref["dq"], f"batch {b} dQ")
        check_grad(g["dk_cmp"][b].cpu().numpy(), ref["dkc"], f"batch {b} dK_cmp")
        check_grad(g["dgates"][b].cpu().numpy(), ref["dgates"], f"batch {b} dgates")


@pytest.mark.parametrize("train", [False, True])
def test_backward_moba_mode(train):
    """MoBA mode (mean-pooled block keys, G = 1, selected branch only): the selected-branch
    backward on its own block lists."""
    cfg = TINY.replace(name="bwd_moba", seq_len=2048, num_kv_heads=2, heads_per_group=1, d_k=128, d_v=128,
                       cmp_block=128, cmp_stride=128, slc_block=128, top_n=3, n_init=0, n_local=1, window=0,
                       phi=PHI_MEAN, score_mode=SCORE_MEAN_DOT, branches=BR_SLC, fp32_inputs=False, seed=46)
    inp, dO_bits, fwd, g = _run(cfg, False, train)
    ref = oracle.nsa_bwd(cfg, f64(inp["q"][0]), f64(inp["k"][0]), f64(inp["v"][0]), None, None,
                         fwd["sel"][0].cpu().numpy(), None, f64(dO_bits[0]))
    for k, r in (("dq", "dq"), ("dk", "dk"), ("dv", "dv")):
        check_grad(g[k][0].cpu().numpy(), ref[r], f"moba {k}")


def test_backward_repeatable_shapes():
    """Two calls in a row give the same dQ bit for bit (dQ has no atomics) and dK within
    the atomics' reordering."""
    cfg = GQA.replace(name="bwd_repeat", seed=47)
    inp, dO_bits, fwd, g1 = _run(cfg, True)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    wk, wv, pk, pv = (dev_bf16(inp[n]) for n in ("w_k", "w_v", "pe_k", "pe_v"))
    g2 = ops.backward(cfg, fwd, q, k, v, wk, wv, pk, pv, torch.as_tensor(inp["gates"], device="cuda"),
                      dev_bf16(dO_bits))
    torch.cuda.synchronize()
    assert torch.equal(g1["dq"], g2["dq"])
    assert torch.equal(g1["dgates"], g2["dgates"])
    d = (g1["dk"] - g2["dk"]).abs().max().item()
    assert d <= 1e-5 * max(g1["dk"].abs().max().item(), 1.0)


@pytest.mark.parametrize("cfg", [GQA, RAGGED, TINY.replace(fp32_inputs=False, seed=48)], ids=lambda c: c.name)
def test_training_forward_saves_branch_outputs(cfg):
    """nsa_sparse_attn_fwd_train returns the forward's O bit for bit and saves each branch's
    normalized output (checked against the oracle's o_slc / o_win for the same selection and
    o_cmp) and base-2 log-sum-exp (checked against the oracle's scores of the same keys)."""
    inp = inputs.prefill_inputs(cfg)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    wk, wv, pk, pv = (dev_bf16(inp[n]) for n in ("w_k", "w_v", "pe_k", "pe_v"))
    gates = torch.as_tensor(inp["gates"], device="cuda")
    fwd = ops.prefill(cfg, q, k, v, wk, wv, pk, pv, gates)
    out_t, s_lse, s_o = ops.sparse_attn_fwd_train(cfg, q, k, v, fwd["sel"], fwd["o_cmp"], gates)
    torch.cuda.synchronize()
    assert torch.equal(out_t, fwd["out"])
    rows = np.arange(cfg.seq_len)
    ref = oracle.attend(cfg, f64(inp["q"][0]), rows, f64(inp["k"][0]), f64(inp["v"][0]), fwd["sel"][0].cpu().numpy(),
                        fwd["o_cmp"][0].cpu().numpy().astype(np.float64), inp["gates"][0].astype(np.float64))
    so = s_o[0].cpu().numpy()
    check_close(so[:, :, 0], ref["o_slc"], f"{cfg.name} saved o_slc")
    check_close(so[:, :, 1], ref["o_win"], f"{cfg.name} saved o_win")
    # window LSE of a few rows written out: log2 sum 2^(scale log2e q.k) over t-w+1 .. t
    qq, kk = f64(inp["q"][0]), f64(inp["k"][0])
    sl = s_lse[0].cpu().numpy()
    for t in (0, 5, cfg.seq_len // 2, cfg.seq_len - 1):
        for h in range(0, cfg.num_heads, max(1, cfg.num_heads // 4)):
            g = h // cfg.heads_per_group
            a = cfg.scale * (kk[g, max(0, t - cfg.window + 1):t + 1] @ qq[t, h])
            ref_lse2 = (a.max() + np.log(np.exp(a - a.max()).sum())) / np.log(2.0)
            assert abs(sl[t, h, 1] - ref_lse2) <= 1e-4 * max(1.0, abs(ref_lse2)), (t, h, sl[t, h, 1], ref_lse2)


@pytest.mark.parametrize("cfg", [P8K, P64K], ids=lambda c: c.name)
def test_backward_full_size(cfg):
    """The 8K and 64K workloads in the benchmark's configuration (training forward, backward
    on the saved statistics): dQ and the gate gradients on sampled rows against the oracle,
    computed row by row; dK, dV, dK_cmp and dV_cmp element by element on listed keys against
    the oracle's sums over every row that sees them; and, as extra checks over all keys, two
    identities that hold at any size (every branch's probabilities of a row sum to one):
        sum over keys of dV  = sum over the group's (token, head) rows of sigma_c dO   (per branch
                               group: raw keys carry the selected + window branches, compressed
                               keys the compressed branch, counted for rows that see one)
        sum over keys of dK  = 0   (each row's dS sums to zero)."""
    print(f"[case] backward {cfg.name} full size", flush=True)
    inp = inputs.prefill_inputs(cfg)
    dO_bits = inputs.grad_output(cfg)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    wk, wv, pk, pv = (dev_bf16(inp[n]) for n in ("w_k", "w_v", "pe_k", "pe_v"))
    gates = torch.as_tensor(inp["gates"], device="cuda")
    fwd = ops.prefill(cfg, q, k, v, wk, wv, pk, pv, gates, train=True)
    g = ops.sparse_attn_bwd(cfg, q, k, v, fwd["k_cmp"], fwd["v_cmp"], fwd["sel"], fwd["lse"], fwd["o_cmp"], gates,
                            dev_bf16(dO_bits), saved_lse=fwd["saved_lse"], saved_o=fwd["saved_o"])
    torch.cuda.synchronize()
    rows = sample_rows(cfg.seq_len, 24, 11)
    kc, vc = bf16_dev_to_f64(fwd["k_cmp"][0]), bf16_dev_to_f64(fwd["v_cmp"][0])
    ref = oracle.nsa_bwd_rows(cfg, f64(inp["q"][0, rows]), rows, f64(inp["k"][0]), f64(inp["v"][0]), kc, vc,
                              fwd["sel"][0, rows].cpu().numpy(), inp["gates"][0, rows].astype(np.float64),
                              f64(dO_bits[0, rows]))
    check_grad(g["dq"][0, rows].cpu().numpy(), ref["dq"], f"{cfg.name} dQ sampled rows")
    check_grad(g["dgates"][0, rows].cpu().numpy(), ref["dgates"], f"{cfg.name} dgates sampled rows")
    # key side element by element: per KV group, the oracle's sums over every row that sees
    # each listed key (oracle.nsa_bwd_keys).  At 8K every raw and compressed key; at 64K
    # 8 selection blocks per group (32 in all, block 0 excluded, the last block included) and
    # the last 32 compressed keys of each group (the rows that see a compressed key are every
    # later row, so early ones would cost the fp64 oracle minutes).
    G, Hkv = cfg.heads_per_group, cfg.num_kv_heads
    rng = np.random.default_rng(12)
    Qf, dOf = f64(inp["q"][0]), f64(dO_bits[0])
    Kf, Vf = f64(inp["k"][0]), f64(inp["v"][0])
    sel_all = fwd["sel"][0].cpu().numpy()
    gk, gv = g["dk"][0].cpu().numpy(), g["dv"][0].cpu().numpy()
    gkc, gvc = g["dk_cmp"][0].cpu().numpy(), g["dv_cmp"][0].cpu().numpy()
    lp = cfg.slc_block
    for grp in range(Hkv):
        if cfg.seq_len <= 8192:
            raw, ck = np.arange(cfg.seq_len), np.arange(cfg.n_cmp)
        else:
            blocks = rng.choice(np.arange(1, cfg.n_slc - 1), 8 if grp else 7, replace=False)
            if grp == 0:
                blocks = np.append(blocks, cfg.n_slc - 1)
            raw = np.concatenate([np.arange(j * lp, min((j + 1) * lp, cfg.seq_len)) for j in np.sort(blocks)])
            ck = np.arange(cfg.n_cmp - 32, cfg.n_cmp)
        hs = slice(grp * G, (grp + 1) * G)
        c1 = cfg.replace(num_kv_heads=1)
        ref_k = oracle.nsa_bwd_keys(c1, Qf[:, hs], Kf[grp:grp + 1], Vf[grp:grp + 1], kc[grp:grp + 1],
                                    vc[grp:grp + 1], sel_all[:, grp:grp + 1], inp["gates"][0, :, hs].astype(np.float64),
                                    dOf[:, hs], raw, ck)
        what = f"{cfg.name} group {grp} ({len(raw)} keys, {len(ck)} compressed keys)"
        check_grad(gk[grp, raw], ref_k["dk"][0], f"{what} dK")
        check_grad(gv[grp, raw], ref_k["dv"][0], f"{what} dV")
        check_grad(gkc[grp, ck], ref_k["dkc"][0], f"{what} dK_cmp")
        check_grad(gvc[grp, ck], ref_k["dvc"][0], f"{what} dV_cmp")
    # identities, per KV group
    G, T, l = cfg.heads_per_group, cfg.seq_len, cfg.cmp_block
    sig = 1.0 / (1.0 + np.exp(-inp["gates"][0].astype(np.float64)))      # [T, H, 3]
    dO = inputs.bf16_bits_to_f32(dO_bits[0]).astype(np.float64)         # [T, H, dv]
    seen = (np.arange(T) >= l - 1)[:, None]
    for grp in range(cfg.num_kv_heads):
        hs = slice(grp * G, (grp + 1) * G)
        want_raw = np.einsum("th,thd->d", sig[:, hs, 1] + sig[:, hs, 2], dO[:, hs])
        want_cmp = np.einsum("th,thd->d", sig[:, hs, 0] * seen, dO[:, hs])
        for name, got, want in (("dV", g["dv"][0, grp], want_raw), ("dV_cmp", g["dv_cmp"][0, grp], want_cmp)):
            s = got.double().sum(0).cpu().numpy()
            err = np.linalg.norm(s - want) / np.linalg.norm(want)
            print(f"[parity] {cfg.name} group {grp} sum of {name} over keys: rel err {err:.3e}", flush=True)
            assert err <= 5e-3, (name, grp, err)
        for name, got in (("dK", g["dk"][0, grp]), ("dK_cmp", g["dk_cmp"][0, grp])):
            gd = got.double()
            rel = (gd.sum(0).norm() / gd.norm()).item()
            print(f"[parity] {cfg.name} group {grp} sum of {name} over keys / Frobenius norm: {rel:.3e}", flush=True)
            assert rel <= 1e-2, (name, grp, rel)
