"""Pins of the fp64 backward oracle (oracle.nsa_bwd, oracle.compress_linear_bwd and the
chain in oracle.pipeline.backward) against facts that do not come from that code.

  finite differences   the forward oracle (pinned on its own in test_oracle_pins.py) is
                       differentiated numerically along random directions of every input
                       (central differences in fp64, the selection held fixed): a dropped
                       term, a wrong sign, a transposed operand or a wrong index in any
                       gradient changes the directional derivative.
  closed forms         the block map is linear: its gradients along a direction equal the
                       map applied to that direction exactly.
  textbook routine     with every block selected and the other branches off, the
                       gradients equal torch autograd of dense causal attention in fp64
                       (an independent implementation).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import pipeline
from dynamic_block_sparse_nsa_amd.configs import TINY, BR_ALL, BR_CMP, BR_SLC, BR_WIN

# small geometry that keeps every rule in play: several compressed blocks per selection
# block, forced and free picks, a window that crosses block edges, ragged last block
BW = TINY.replace(name="bwd_pin", seq_len=150, num_kv_heads=2, heads_per_group=2, d_k=16, d_v=8, cmp_block=8,
                  cmp_stride=4, slc_block=16, top_n=4, n_init=1, n_local=2, window=24)


def case(cfg, seed):
    rng = np.random.default_rng(7000 + seed)
    T, H, Hkv, dk, dv, l = cfg.seq_len, cfg.num_heads, cfg.num_kv_heads, cfg.d_k, cfg.d_v, cfg.cmp_block
    c = {"Q": rng.standard_normal((T, H, dk)), "K": rng.standard_normal((Hkv, T, dk)),
         "V": rng.standard_normal((Hkv, T, dv)), "gates": rng.standard_normal((T, H, 3)),
         "w_k": rng.uniform(-0.2, 0.2, (l * dk, dk)), "w_v": rng.uniform(-0.2, 0.2, (l * dv, dv)),
         "pe_k": rng.standard_normal((l, dk)), "pe_v": rng.standard_normal((l, dv)),
         "dO": rng.standard_normal((T, H, dv))}
    c["Kc"], c["Vc"] = pipeline.compress_all(cfg, c["K"], c["V"], c["w_k"], c["w_v"], c["pe_k"], c["pe_v"],
                                             round_cmp=False)
    rows = np.arange(T)
    c["sel"] = oracle.score_select(cfg, c["Q"], rows, c["Kc"], c["Vc"])["sel"]
    return c


def forward_out(cfg, Q, K, V, Kc, Vc, sel, gates, branches):
    rows = np.arange(Q.shape[0])
    o_cmp = oracle.score_select(cfg, Q, rows, Kc, Vc)["o_cmp"] if branches & 1 else None
    return oracle.attend(cfg, Q, rows, K, V, sel, o_cmp, gates, branches=branches)["out"]


def loss(cfg, c, branches, **over):
    x = {k: over.get(k, c[k]) for k in ("Q", "K", "V", "Kc", "Vc", "gates")}
    out = forward_out(cfg, x["Q"], x["K"], x["V"], x["Kc"], x["Vc"], c["sel"], x["gates"], branches)
    return float(np.sum(c["dO"] * out))


def fd(f, x, u, eps=1e-6):
    return (f(x + eps * u) - f(x - eps * u)) / (2 * eps)


GRAD_OF = {"Q": "dq", "K": "dk", "V": "dv", "Kc": "dkc", "Vc": "dvc", "gates": "dgates"}


@pytest.mark.parametrize("branches", [BR_ALL, BR_CMP, BR_SLC, BR_WIN, BR_SLC | BR_WIN])
@pytest.mark.parametrize("name", ["Q", "K", "V", "Kc", "Vc", "gates"])
def test_directional_derivatives(name, branches):
    c = case(BW, 1)
    if name in ("Kc", "Vc") and not branches & 1:
        pytest.skip("no compressed branch")
    g = oracle.nsa_bwd(BW, c["Q"], c["K"], c["V"], c["Kc"], c["Vc"], c["sel"], c["gates"], c["dO"], branches)
    rng = np.random.default_rng(11)
    for _ in range(2):
        u = rng.standard_normal(c[name].shape)
        num = fd(lambda x: loss(BW, c, branches, **{name: x}), c[name], u)
        ana = float(np.sum(g[GRAD_OF[name]] * u))
        assert abs(num - ana) <= 1e-7 * max(1.0, abs(ana)), (name, branches, num, ana)


def test_gradients_without_gates():
    """gates = None means weight 1 on every branch: the gradients equal those of logits
    so large that every sigmoid is 1 to machine precision."""
    c = case(BW, 2)
    g0 = oracle.nsa_bwd(BW, c["Q"], c["K"], c["V"], c["Kc"], c["Vc"], c["sel"], None, c["dO"])
    g1 = oracle.nsa_bwd(BW, c["Q"], c["K"], c["V"], c["Kc"], c["Vc"], c["sel"], np.full_like(c["gates"], 60.0),
                        c["dO"])
    assert g0["dgates"] is None
    for k in ("dq", "dk", "dv", "dkc", "dvc"):
        np.testing.assert_allclose(g0[k], g1[k], rtol=1e-12, atol=1e-12)
    # and a direction check of the no-gate case itself
    u = np.random.default_rng(3).standard_normal(c["Q"].shape)
    num = fd(lambda x: float(np.sum(c["dO"] * forward_out(BW, x, c["K"], c["V"], c["Kc"], c["Vc"], c["sel"], None,
                                                            BR_ALL))), c["Q"], u)
    assert abs(num - np.sum(g0["dq"] * u)) <= 1e-7 * max(1.0, abs(num))


def test_compress_bwd_is_the_adjoint_of_the_map():
    """The block map is linear in X, in PE and in W separately: the gradient contracted
    with any direction equals <dY, map(direction)> exactly (the map's adjoint)."""
    rng = np.random.default_rng(5)
    n_tok, d, d_out, l, s = 75, 6, 5, 8, 4
    nblk = (n_tok - l) // s + 1
    X, pe = rng.standard_normal((n_tok, d)), rng.standard_normal((l, d))
    W, dY = rng.standard_normal((l * d, d_out)), rng.standard_normal((nblk, d_out))
    g = oracle.compress_linear_bwd(X, pe, W, dY, l, s)
    uX, upe, uW = rng.standard_normal(X.shape), rng.standard_normal(pe.shape), rng.standard_normal(W.shape)
    # along X (PE off): map(uX)
    assert np.isclose(np.sum(g["dx"] * uX), np.sum(dY * oracle.compress_linear(uX, None, W, l, s)), rtol=1e-12)
    # along PE: every block gains vec(uPE).W, the map of a zero sequence with PE = uPE
    assert np.isclose(np.sum(g["dpe"] * upe),
                      np.sum(dY * oracle.compress_linear(np.zeros_like(X), upe, W, l, s)), rtol=1e-12)
    # along W: map with weights uW
    assert np.isclose(np.sum(g["dw"] * uW), np.sum(dY * oracle.compress_linear(X, pe, uW, l, s)), rtol=1e-12)


@pytest.mark.parametrize("name", ["K", "V", "w_k", "w_v", "pe_k", "pe_v"])
def test_chain_through_compression(name):
    """pipeline.backward's key/value and block-map gradients include the compressed
    branch's path through step 1: checked against differences of the whole forward chain
    (compression recomputed from the perturbed input)."""
    c = case(BW, 3)
    g = pipeline.backward(BW, c["Q"], c["K"], c["V"], c["w_k"], c["w_v"], c["pe_k"], c["pe_v"], c["sel"],
                          c["gates"], c["dO"])

    def full_loss(x):
        a = {k: c[k] for k in ("K", "V", "w_k", "w_v", "pe_k", "pe_v")}
        a[name] = x
        Kc, Vc = pipeline.compress_all(BW, a["K"], a["V"], a["w_k"], a["w_v"], a["pe_k"], a["pe_v"],
                                       round_cmp=False)
        out = forward_out(BW, c["Q"], a["K"], a["V"], Kc, Vc, c["sel"], c["gates"], BR_ALL)
        return float(np.sum(c["dO"] * out))

    key = {"K": "dk", "V": "dv", "w_k": "dw_k", "w_v": "dw_v", "pe_k": "dpe_k", "pe_v": "dpe_v"}[name]
    u = np.random.default_rng(4).standard_normal(c[name].shape)
    num = fd(full_loss, c[name], u)
    ana = float(np.sum(g[key] * u))
    assert abs(num - ana) <= 1e-7 * max(1.0, abs(ana)), (name, num, ana)


def test_select_all_equals_dense_causal_autograd():
    """Every block selected, selected branch only, no gates: the branch is dense causal
    attention (the forward pin p1), so its gradients are those of the textbook routine,
    here differentiated by torch autograd in fp64."""
    cfg = BW.replace(top_n=BW.n_slc, branches=BR_SLC)
    c = case(cfg, 4)
    T, H, G = cfg.seq_len, cfg.num_heads, cfg.heads_per_group
    sel = np.tile(np.arange(cfg.n_slc, dtype=np.int32), (T, cfg.num_kv_heads, 1))
    g = oracle.nsa_bwd(cfg, c["Q"], c["K"], c["V"], None, None, sel, None, c["dO"], BR_SLC)
    Q = torch.tensor(c["Q"], requires_grad=True)
    K = torch.tensor(c["K"], requires_grad=True)
    V = torch.tensor(c["V"], requires_grad=True)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    total = 0.0
    for h in range(H):
        a = (Q[:, h, :] @ K[h // G].T) * cfg.scale
        a = a.masked_fill(~mask, -math.inf)
        o = torch.softmax(a, dim=-1) @ V[h // G]
        total = total + (torch.tensor(c["dO"][:, h, :]) * o).sum()
    total.backward()
    np.testing.assert_allclose(g["dq"], Q.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dk"], K.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dv"], V.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_rows_variant_equals_full_backward():
    """oracle.nsa_bwd_rows (the query side for listed rows, used at sizes where the full
    backward is too slow) gives exactly the full backward's dq and gate gradients; the full
    backward is the one pinned above."""
    c = case(BW, 5)
    g = oracle.nsa_bwd(BW, c["Q"], c["K"], c["V"], c["Kc"], c["Vc"], c["sel"], c["gates"], c["dO"])
    rows = np.array([0, 3, 7, 31, 64, 100, 149])
    r = oracle.nsa_bwd_rows(BW, c["Q"][rows], rows, c["K"], c["V"], c["Kc"], c["Vc"], c["sel"][rows],
                            c["gates"][rows], c["dO"][rows])
    np.testing.assert_allclose(r["dq"], g["dq"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dgates"], g["dgates"][rows], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("branches,gated", [(BR_ALL, True), (BR_ALL, False), (BR_SLC, True), (BR_WIN | BR_CMP, True)],
                         ids=["all_gated", "all", "slc", "win_cmp"])
def test_keys_variant_equals_full_backward(branches, gated):
    """oracle.nsa_bwd_keys (the key side for listed keys only, as the full-size GPU tests use
    it) equals oracle.nsa_bwd's key-side gradients at those keys, which the finite-difference
    pins above fix; also with lists that hold the first and last keys, several keys of one
    selection block, and compressed blocks at both ends."""
    cfg = BW.replace(branches=branches)
    c = case(cfg, 60 + branches)
    gates = c["gates"] if gated else None
    full = oracle.nsa_bwd(cfg, c["Q"], c["K"], c["V"], c["Kc"], c["Vc"], c["sel"], gates, c["dO"])
    T, n_cmp = cfg.seq_len, c["Kc"].shape[1]
    raw = np.array([0, 1, 15, 16, 17, 40, 63, 64, 100, 127, 128, T - 2, T - 1])
    ck = np.array([0, 3, n_cmp // 2, n_cmp - 1])
    got = oracle.nsa_bwd_keys(cfg, c["Q"], c["K"], c["V"], c["Kc"], c["Vc"], c["sel"], gates, c["dO"], raw, ck)
    np.testing.assert_allclose(got["dk"], full["dk"][:, raw], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["dv"], full["dv"][:, raw], rtol=1e-12, atol=1e-12)
    assert np.abs(full["dk"][:, raw]).max() > 0
    if branches & 1:
        np.testing.assert_allclose(got["dkc"], full["dkc"][:, ck], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dvc"], full["dvc"][:, ck], rtol=1e-12, atol=1e-12)
        assert np.abs(full["dkc"][:, ck]).max() > 0
    # every raw key at once equals the whole array
    allk = oracle.nsa_bwd_keys(cfg, c["Q"], c["K"], c["V"], c["Kc"], c["Vc"], c["sel"], gates, c["dO"],
                               np.arange(T), np.arange(n_cmp) if branches & 1 else ())
    np.testing.assert_allclose(allk["dk"], full["dk"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(allk["dv"], full["dv"], rtol=1e-12, atol=1e-12)
