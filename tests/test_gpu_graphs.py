"""Replays of captured HIP graphs, the form a serving loop uses for the decode step and the
cache maintenance before it, against eager calls.  Each graph is replayed several times
with the program's own eager work and synchronizations between the replays, and every
replay must reproduce the eager result bit for bit (the kernels are deterministic and use
no memset or copy nodes).
"""
import pytest
import torch

from dynamic_block_sparse_nsa_amd import ops
from dynamic_block_sparse_nsa_amd.configs import DECODE

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[graphs] {msg}", flush=True)


CFG = DECODE.replace(name="graph_decode", batch=4, seq_len=8192, seed=61)


def _setup(cfg, seed):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    B, L, H, Hkv, l = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads, cfg.cmp_block

    def bf(shape, scale=1.0):
        return (torch.randn(shape, generator=g, device=dev) * scale).to(torch.bfloat16)

    w = {"wk": bf((l * cfg.d_k, cfg.d_k), 0.05), "wv": bf((l * cfg.d_v, cfg.d_v), 0.05),
         "pk": bf((l, cfg.d_k)), "pv": bf((l, cfg.d_v))}
    K, V = bf((B, Hkv, L, cfg.d_k)), bf((B, Hkv, L, cfg.d_v))
    kc, vc = ops.compress(cfg, K, V, w["wk"], w["wv"], w["pk"], w["pv"])
    return dev, g, w, K, V, kc, vc


def test_decode_graph_replays_match_eager():
    announce("decode graph replays")
    cfg = CFG
    dev, g, w, K, V, kc, vc = _setup(cfg, 61)
    B, H = cfg.batch, cfg.num_heads
    q = torch.randn((B, H, cfg.d_k), generator=g, device=dev).to(torch.bfloat16)
    q2 = torch.randn((B, H, cfg.d_k), generator=g, device=dev).to(torch.bfloat16)
    gates = torch.randn((B, H, 3), generator=g, device=dev)
    clen = torch.tensor([cfg.seq_len, cfg.seq_len - 1000, 5000, 77], dtype=torch.int32, device=dev)
    ws = torch.empty(ops.workspace_size(cfg, ops.OP_DECODE), dtype=torch.uint8, device=dev)
    o_e, s_e = ops.decode(cfg, q, K, V, clen, kc, vc, gates, workspace=ws)
    torch.cuda.synchronize()
    o_e, s_e = o_e.clone(), s_e.clone()
    o_g = torch.empty_like(o_e)
    s_g = torch.empty_like(s_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.decode(cfg, q, K, V, clen, kc, vc, gates, out=o_g, sel=s_g, workspace=ws)
    for rep in range(4):
        # eager work in between: another decode through the same workspace, and the
        # graph's outputs overwritten
        o_x, _ = ops.decode(cfg, q2, K, V, clen, kc, vc, gates, workspace=ws)
        o_g.fill_(float("nan"))
        s_g.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(s_g, s_e), f"replay {rep}: selection differs from the eager call"
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), f"replay {rep}: output differs"
        assert not torch.equal(o_x.view(torch.int16), o_e.view(torch.int16))   # the eager call did other work


def test_cache_append_graph_replays_match_eager():
    announce("cache append graph replays")
    cfg = CFG
    dev, g, w, K, V, kc, vc = _setup(cfg, 62)
    B, Hkv, s = cfg.batch, cfg.num_kv_heads, cfg.cmp_stride
    prep = ops.compress_prepare(cfg, w["wk"], w["wv"], w["pk"], w["pv"])
    kn = torch.randn((B, Hkv, 1, cfg.d_k), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, Hkv, 1, cfg.d_v), generator=g, device=dev).to(torch.bfloat16)
    start = torch.tensor([cfg.seq_len - 4 * s, 3000, 1001, 31], dtype=torch.int32, device=dev)
    state0 = [t.clone() for t in (K, V, kc, vc)]
    clen = start.clone()

    def restore():
        for dst, src in zip((K, V, kc, vc), state0):
            dst.copy_(src)
        clen.copy_(start)

    # eager: s single-token appends (one of them completes a compressed block per sequence)
    for _ in range(s):
        ops.cache_append(cfg, kn, vn, K, V, clen, kc, vc, prep)
    torch.cuda.synchronize()
    want = [t.clone() for t in (K, V, kc, vc, clen)]
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(s):
            ops.cache_append(cfg, kn, vn, K, V, clen, kc, vc, prep)
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("K", "V", "K_cmp", "V_cmp", "cache_len"), (K, V, kc, vc, clen), want):
            a = got.view(torch.int16) if got.dtype == torch.bfloat16 else got
            b = ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager appends"
