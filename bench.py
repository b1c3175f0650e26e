#!/usr/bin/env python3
"""Benchmark of the NSA forward hot path on one MI355X.

A step is one pass of the prefill hot path over the 64K workload (batch 1, 65536 tokens,
4 KV groups x 16 query heads, d_k 192, d_v 128, compression 32/16, 64-token selection
blocks, top-16, window 512): nsa_compress -> nsa_score_select -> nsa_sparse_attn_fwd, with
every input resident in HBM before the timed region.  The headline ``value`` is prefill
tokens/s; the line also carries the algorithmic TFLOP/s and MFMA-peak fraction, a
roofline entry for the dominant kernel (timed live with HIP events on the stream it runs
on), the oracle timed on the host cores on a bounded sample, the backward pass of the same
64K step (nsa_sparse_attn_bwd + nsa_compress_bwd), and the decode step (batch 32 x
65536-token caches, HBM GB/s) and MoBA (131072 and 1048576 tokens) figures.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-moba]
                       [--no-dense] [--no-backward] [--no-ceilings] [--locality]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from dynamic_block_sparse_nsa_amd.configs import P8K, P64K, DECODE, MOBA, NSAConfig  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


# ---------------------------------------------------------------------------
# algorithmic work (unmasked (query, head, key) pairs x 2*(d_k + d_v) flops)
# ---------------------------------------------------------------------------
def cmp_pairs(cfg: NSAConfig) -> int:
    t = np.arange(cfg.seq_len, dtype=np.int64)
    nv = np.where(t >= cfg.cmp_block - 1, np.minimum((t - cfg.cmp_block + 1) // cfg.cmp_stride + 1, cfg.n_cmp), 0)
    return int(nv.sum()) * cfg.num_heads


def slc_pairs(cfg: NSAConfig) -> int:
    """Selected-branch keys with top_n blocks chosen (the own block causal, the rest full)."""
    t = np.arange(cfg.seq_len, dtype=np.int64)
    jc = t // cfg.slc_block
    m = np.minimum(cfg.top_n, jc + 1)
    keys = (m - 1) * cfg.slc_block + (t - jc * cfg.slc_block + 1)
    return int(keys.sum()) * cfg.num_heads


def win_pairs(cfg: NSAConfig) -> int:
    t = np.arange(cfg.seq_len, dtype=np.int64)
    return int(np.minimum(t + 1, cfg.window).sum()) * cfg.num_heads


def prefill_flops(cfg: NSAConfig) -> dict:
    f = 2 * (cfg.d_k + cfg.d_v)
    return {"cmp": cmp_pairs(cfg) * f, "slc": slc_pairs(cfg) * f, "win": win_pairs(cfg) * f}


def moba_flops(cfg: NSAConfig) -> int:
    return slc_pairs(cfg) * 2 * (cfg.d_k + cfg.d_v)


def backward_flops(cfg: NSAConfig) -> dict:
    """Five products per unmasked pair (S recomputed, dP = dO.v, dV, dQ, dK):
    2 * (3 d_k + 2 d_v) flops; the block map: dX = dY.W^T and dW = X^T.dY for keys and values."""
    pairs = cmp_pairs(cfg) + slc_pairs(cfg) + win_pairs(cfg)
    bm = 2 * 2 * cfg.batch * cfg.num_kv_heads * cfg.n_cmp * cfg.cmp_block * (cfg.d_k * cfg.d_k + cfg.d_v * cfg.d_v)
    return {"attention": pairs * 2 * (3 * cfg.d_k + 2 * cfg.d_v), "block_map": bm}


# ---------------------------------------------------------------------------
def locality(cfg, Q, K, V, ocmp, gates, out, ws, call_ms, result, time_calls, torch, dev):
    """The headline inputs are random, so neighbouring tokens share no free pick.  For
    contrast: the same kernel on valid lists in which the 64 tokens of each selection block
    share their free picks (forced blocks as the rule has them), the locality trained
    attention tends to show."""
    from dynamic_block_sparse_nsa_amd import ops
    T, Hkv = cfg.seq_len, cfg.num_kv_heads
    rng = np.random.default_rng(cfg.seed + 77)
    coh = np.full((T, Hkv, cfg.top_n), -1, dtype=np.int32)
    for jc in range(cfg.n_slc):
        t0, t1 = jc * cfg.slc_block, min((jc + 1) * cfg.slc_block, T)
        forced = sorted(set(range(min(cfg.n_init, jc + 1))) | set(range(max(0, jc - cfg.n_local + 1), jc + 1)))
        pool = [j for j in range(jc + 1) if j not in forced]
        n_free = min(cfg.top_n, jc + 1) - len(forced)
        for gg in range(Hkv):
            picks = rng.choice(pool, n_free, replace=False).tolist() if n_free > 0 else []
            row = sorted(forced + picks)
            coh[t0:t1, gg, :len(row)] = row
    sel_coh = torch.from_numpy(coh[None]).to(dev)
    pcc, _ = time_calls([lambda: ops.sparse_attn_fwd(cfg, Q, K, V, sel_coh, ocmp, gates, out=out, workspace=ws[2])],
                        5, 1, torch)
    cms = float(pcc.mean())
    result["selected_locality"] = {
        "workload": "nsa_sparse_attn_fwd_64k_shared_picks", "ms": round(cms, 3),
        "vs_random_picks_ms": round(float(call_ms[2]), 3),
        "gathered_gbs": round(slc_pairs(cfg) // cfg.heads_per_group * (cfg.d_k + cfg.d_v) * 2 / (cms * 1e-3) / 1e9, 1),
        "note": "free picks shared by the 64 tokens of each selection block"}


def load_traffic(kernel: str, sources) -> dict | None:
    """HBM traffic per launch from the committed counter record, if it was taken on the
    current sources of the kernel (otherwise None: the kernel changed since)."""
    from dynamic_block_sparse_nsa_amd.profsum import source_sha
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or sorted(rec.get("sources", [])) != sorted(sources) or rec.get("source_sha") != source_sha(rec["sources"]):
        return None
    return rec


def time_calls(fns, steps, warmup, torch):
    """Run the list of callables per step; per-call and per-step times from HIP events
    recorded on the current stream."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = np.array([[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(len(fns))] for s in range(steps)])
    return per_call, wall


def cpu_baseline(cfg: NSAConfig, inp: dict, budget_rows: int = 3072) -> dict:
    """The fp64 oracle on a bounded sample of the same workload, scaled to tokens/s: the
    whole compression (every block of every KV group, rounded to bf16 as the path stores
    it), then the score, select and attend stages on those compressed keys for the last
    ``budget_rows`` rows (the most expensive ones; scaled to T rows at that cost, which
    overstates the CPU's speed on earlier rows only through their shorter compressed
    history)."""
    from oracle import pipeline
    import oracle
    from dynamic_block_sparse_nsa_amd.inputs import bf16_bits_to_f64 as f64

    threads = oracle.num_threads()
    K, V = f64(inp["k"][0]), f64(inp["v"][0])
    t0 = time.perf_counter()
    Kc, Vc = pipeline.compress_all(cfg, K, V, f64(inp["w_k"]), f64(inp["w_v"]), f64(inp["pe_k"]), f64(inp["pe_v"]))
    t_cmp = time.perf_counter() - t0
    rows = np.arange(cfg.seq_len - budget_rows, cfg.seq_len, dtype=np.int32)
    Qr = f64(inp["q"][0, rows])
    t1 = time.perf_counter()
    ss = oracle.score_select(cfg, Qr, rows, Kc, Vc, want_scores=False)
    oracle.attend(cfg, Qr, rows, K, V, ss["sel"], ss["o_cmp"], inp["gates"][0, rows])
    t_rows = time.perf_counter() - t1
    total = t_cmp + t_rows * cfg.seq_len / budget_rows
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(cfg.seq_len / total, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "sample": (f"fp64 oracle: compression of all {cfg.n_cmp} blocks of every KV group ({t_cmp:.2f} s) + "
                       f"score/select/attend on those compressed keys for the last {budget_rows} of {cfg.seq_len} "
                       f"rows ({t_rows:.2f} s, scaled to all rows); {threads} OpenMP threads")}


def ceilings(torch, dev) -> dict:
    """Measured ceilings of the units the kernels are bound by (libnsa_ceilings.so): bf16 MFMA
    from registers, a streaming read of 4 GiB, and random 40 KB block gathers (the selected
    branch's access pattern: 24 KB of K + 16 KB of V per block) over a 168 MB buffer (the 64K
    workload's K and V) and over a 4 MB one (one XCD's L2)."""
    import ctypes
    from dynamic_block_sparse_nsa_amd.build import CEIL_LIB, build_ceilings
    if not os.path.exists(CEIL_LIB):
        build_ceilings()
    C = ctypes.CDLL(CEIL_LIB)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p

    def timed(launch, reps=5):
        launch()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = launch()
            e1.record()
            torch.cuda.synchronize()
            assert rc == 0, rc
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    res = {}
    n_wg, iters = 4096, 400
    out = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    sec = timed(lambda: C.nsa_ceiling_mfma(P(out.data_ptr()), n_wg, iters, st))
    res["mfma_bf16_tflops"] = round(n_wg * 4 * iters * 32 * 16384 / sec / 1e12, 1)
    buf = torch.empty(1 << 32, dtype=torch.uint8, device=dev).fill_(3)
    wout = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    sec = timed(lambda: C.nsa_ceiling_stream(P(buf.data_ptr()), ctypes.c_size_t(1 << 32), P(wout.data_ptr()), 4096, st))
    res["hbm_stream_read_gbs"] = round((1 << 32) / sec / 1e9, 1)
    blk = 40 * 1024
    for name, span in (("gather_40k_168mb_gbs", 168 * (1 << 20)), ("gather_40k_4mb_gbs", 4 * (1 << 20))):
        rng = np.random.default_rng(5)
        n_blk = 100000
        offs = torch.from_numpy(rng.integers(0, span // blk, n_blk).astype(np.int64) * blk).to(dev)
        gout = torch.empty(n_blk * 256, dtype=torch.int32, device=dev)
        sec = timed(lambda: C.nsa_ceiling_gather(P(buf.data_ptr()), P(offs.data_ptr()), n_blk, blk,
                                                 P(gout.data_ptr()), st))
        res[name] = round(n_blk * blk / sec / 1e9, 1)
    del buf, wout, out
    torch.cuda.empty_cache()
    res["note"] = ("mfma: 4096 workgroups x 4 waves x 12800 bf16 16x16x32 products from registers; stream: 4 GiB "
                   "read once; gather: 100000 random 40 KB blocks of the named buffer")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-moba", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense causal attention comparison")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward pass timing")
    ap.add_argument("--locality", action="store_true",
                    help="also time the selected-branch kernel on lists with shared picks per selection block "
                         "(off by default: the same kernel and grid as the headline call, so a profile of the "
                         "default command keeps the headline kernel's own average)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured MFMA / HBM / gather ceilings")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one elementwise kernel over 1 GiB (reads and writes 1 GiB: the known-size kernel that scales HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the NSA forward shards by KV group / batch with no exchange, "
              "and the benchmark runs on a single MI355X; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from dynamic_block_sparse_nsa_amd import inputs, ops

    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.copy_probe:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)   # an elementwise kernel: reads and writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    # ---------------- prefill 64K ----------------
    cfg = P64K
    print(f"[bench] drawing inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = inputs.prefill_inputs(cfg)
    Q, K, V = d(inp["q"]), d(inp["k"]), d(inp["v"])
    wk, wv, pk, pv = d(inp["w_k"]), d(inp["w_v"]), d(inp["pe_k"]), d(inp["pe_v"])
    gates = torch.from_numpy(inp["gates"]).to(dev)
    B, T, H, Hkv = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads
    kc = torch.empty((B, Hkv, cfg.n_cmp, cfg.d_k), dtype=torch.bfloat16, device=dev)
    vc = torch.empty((B, Hkv, cfg.n_cmp, cfg.d_v), dtype=torch.bfloat16, device=dev)
    sel = torch.empty((B, T, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    ocmp = torch.empty((B, T, H, cfg.d_v), dtype=torch.float32, device=dev)
    out = torch.empty((B, T, H, cfg.d_v), dtype=torch.bfloat16, device=dev)
    ws = {op: torch.empty(max(ops.workspace_size(cfg, op), 256), dtype=torch.uint8, device=dev) for op in range(3)}

    ws[ops.OP_PREFILL] = torch.empty(ops.workspace_size(cfg, ops.OP_PREFILL), dtype=torch.uint8, device=dev)
    calls3 = [
        lambda: ops.compress(cfg, K, V, wk, wv, pk, pv, out_k=kc, out_v=vc, workspace=ws[0]),
        lambda: ops.score_select(cfg, Q, kc, vc, sel=sel, o_cmp=ocmp, workspace=ws[1]),
        lambda: ops.sparse_attn_fwd(cfg, Q, K, V, sel, ocmp, gates, out=out, workspace=ws[2]),
    ]
    # the headline step: compression, then scoring + selection + attention + gate in the
    # fused call (nsa_prefill_fwd: the same arithmetic as the two calls above, one launch)
    calls = [
        calls3[0],
        lambda: ops.prefill_fwd(cfg, Q, K, V, kc, vc, gates, out=out, sel=sel, workspace=ws[ops.OP_PREFILL]),
    ]
    print("[bench] timing prefill (three calls)", file=sys.stderr, flush=True)
    per_call3, wall3 = time_calls(calls3, args.steps, args.warmup, torch)
    ms3 = wall3 / args.steps * 1e3
    print("[bench] timing prefill (fused)", file=sys.stderr, flush=True)
    per_call, wall = time_calls(calls, args.steps, args.warmup, torch)
    ms = wall / args.steps * 1e3   # the K timed steps between two synchronizations
    # cold caches: a 2 GiB write before each step evicts L2 and the memory-side cache; the
    # step alone is timed with events (the flush is outside the pair)
    scratch = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(3):
        scratch.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for f in calls:
            f()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del scratch
    fl = prefill_flops(cfg)
    total_flops = sum(fl.values())
    tflops = total_flops / (ms * 1e-3) / 1e12
    call_ms = per_call.mean(axis=0)
    call_ms3 = per_call3.mean(axis=0)
    names = ["nsa_compress", "nsa_prefill_fwd"]
    names3 = ["nsa_compress", "nsa_score_select", "nsa_sparse_attn_fwd"]
    # the dominant call (the fused one) and its algorithmic work: the three branches
    dom = 1
    dom_flops = total_flops
    dom_kernel = "prefill_fused_kernel"
    # every kernel the call launches (the first is the main one)
    dom_launches = ["prefill_fused_kernel", "cmp_vmax_kernel", "tile_cmp_kernel"]
    csrc = "dynamic_block_sparse_nsa_amd/csrc/"
    dom_src = [csrc + f for f in ("prefill.hip", "cmp_attn.hpp", "sparse_attn.hpp", "select.hpp", "common.hpp")]
    dom_tf = dom_flops / (call_ms[dom] * 1e-3) / 1e12
    traffic = load_traffic(dom_kernel, dom_src)
    torch.cuda.synchronize()

    result = {
        "metric": "NSA prefill tokens/s at 64K (also TFLOP/s, % MFMA peak; decode HBM GB/s)",
        "value": round(B * T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "nsa_prefill_64k", "batch": B, "seq_len": T, "kv_groups": Hkv,
                   "heads_per_group": cfg.heads_per_group, "d_k": cfg.d_k, "d_v": cfg.d_v,
                   "cmp_block": cfg.cmp_block, "cmp_stride": cfg.cmp_stride, "slc_block": cfg.slc_block,
                   "top_n": cfg.top_n, "window": cfg.window},
        "tflops_algorithmic": round(tflops, 2),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "timing": "ms_per_step: warm mean over the timed steps; cold_ms_per_step: median of 3 steps "
                  "each after a 2 GiB write that flushes L2 and the memory-side cache",
        "cold_ms_per_step": round(float(np.median(cold)), 4),
        "algorithmic_flops": {k: int(v) for k, v in fl.items()},
        "per_call_ms": {n: round(float(c), 4) for n, c in zip(names, call_ms)},
        "three_calls": {"ms_per_step": round(ms3, 4), "tokens_per_s": round(B * T / (ms3 * 1e-3), 1),
                        "per_call_ms": {n: round(float(c), 4) for n, c in zip(names3, call_ms3)}},
        "wall_s_timed": round(wall, 3),
    }
    # The roofline of the dominant kernel: its algorithmic flops against the bf16 MFMA peak
    # (the prefill's roofline: the path's algorithmic work is counted in flops), and beside
    # it the HBM axis, the bytes the counters record per launch (FETCH_SIZE + WRITE_SIZE,
    # scaled) against the HBM peak.  "limiter" names the axis with the larger fraction.
    sec = call_ms[dom] * 1e-3
    hbm_bytes = None if traffic is None else traffic.get("bytes_per_launch")
    hbm_frac = None if hbm_bytes is None else hbm_bytes / sec / 1e9 / PEAK_HBM_GBS
    mfma_frac = dom_tf / PEAK_BF16_TFLOPS
    result["roofline"] = {
        "bound": "mfma",
        "limiter": None if hbm_frac is None else ("hbm" if hbm_frac > mfma_frac else "mfma"),
        "kernel": dom_kernel, "call": names[dom], "call_kernels": dom_launches,
        "achieved": round(dom_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(mfma_frac, 4),
        "traffic": hbm_bytes,
        "hbm_gbs": None if hbm_bytes is None else round(hbm_bytes / sec / 1e9, 1),
        "hbm_peak_gbs": PEAK_HBM_GBS,
        "hbm_frac": None if hbm_frac is None else round(hbm_frac, 4)}
    if traffic is not None and traffic.get("mfma_busy_frac") is not None:
        result["roofline"]["mfma_busy_frac"] = traffic["mfma_busy_frac"]
    # The selected branch reads each chosen block's keys and values per (token, group):
    # (d_k + d_v) * 2 bytes per selected key, most of it from L2 and the memory-side cache.
    gathered = slc_pairs(cfg) // cfg.heads_per_group * (cfg.d_k + cfg.d_v) * 2
    result["roofline_gather"] = {"kernel": dom_kernel, "gathered_bytes": int(gathered),
                                 "gathered_gbs": round(gathered / sec / 1e9, 1)}

    # ---------------- decode ----------------
    # ---------------- dense causal attention on the same inputs ----------------
    if not args.no_dense:
        print("[bench] dense causal attention", file=sys.stderr, flush=True)
        wsf = torch.empty(ops.workspace_size(cfg, ops.OP_FULL_ATTN), dtype=torch.uint8, device=dev)
        pcf, _ = time_calls([lambda: ops.full_attn_fwd(cfg, Q, K, V, out=out, workspace=wsf)], 3, 1, torch)
        fms = float(pcf.mean())
        dfl = 2 * (cfg.d_k + cfg.d_v) * H * T * (T + 1) / 2
        cmp8 = {}
        # the same comparison at 8K tokens (NSA's compression and fused call against the dense kernel)
        c8 = P8K
        g8 = torch.Generator(device=dev).manual_seed(c8.seed)
        r8 = lambda *sh: torch.randn(sh, generator=g8, device=dev).to(torch.bfloat16)
        Q8, K8, V8 = (r8(1, c8.seq_len, c8.num_heads, c8.d_k), r8(1, c8.num_kv_heads, c8.seq_len, c8.d_k),
                      r8(1, c8.num_kv_heads, c8.seq_len, c8.d_v))
        w8 = (r8(c8.cmp_block * c8.d_k, c8.d_k) * 0.03, r8(c8.cmp_block * c8.d_v, c8.d_v) * 0.03,
              r8(c8.cmp_block, c8.d_k), r8(c8.cmp_block, c8.d_v))
        gt8 = torch.randn((1, c8.seq_len, c8.num_heads, 3), generator=g8, device=dev)
        kc8, vc8 = ops.compress(c8, K8, V8, *w8)
        sel8, _, oc8 = ops.score_select(c8, Q8, kc8, vc8)
        o8 = torch.empty((1, c8.seq_len, c8.num_heads, c8.d_v), dtype=torch.bfloat16, device=dev)
        n8, _ = time_calls([lambda: ops.compress(c8, K8, V8, *w8, out_k=kc8, out_v=vc8),
                            lambda: ops.prefill_fwd(c8, Q8, K8, V8, kc8, vc8, gt8, out=o8, sel=sel8)], 10, 2, torch)
        f8, _ = time_calls([lambda: ops.full_attn_fwd(c8, Q8, K8, V8, out=o8)], 10, 2, torch)
        n8ms, f8ms = float(n8.sum(axis=1).mean()), float(f8.mean())
        result["vs_dense"] = {
            "workload": "dense_causal_64k", "kernel": "full_attn_kernel", "dense_ms": round(fms, 3),
            "dense_tflops": round(dfl / (fms * 1e-3) / 1e12, 1),
            "dense_mfma_frac": round(dfl / (fms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "nsa_ms": round(ms, 3), "nsa_speedup": round(fms / ms, 2),
            "at_8k": {"nsa_ms": round(n8ms, 3), "dense_ms": round(f8ms, 3), "nsa_speedup": round(f8ms / n8ms, 2)}}
        del Q8, K8, V8, kc8, vc8, sel8, oc8, o8, wsf
        torch.cuda.empty_cache()

    # ---------------- the selected branch with selection locality (opt-in) ----------------
    if args.locality:
        locality(cfg, Q, K, V, ocmp, gates, out, ws, call_ms3, result, time_calls, torch, dev)

    # ---------------- backward of the same step ----------------
    if not args.no_backward:
        print("[bench] backward", file=sys.stderr, flush=True)
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
        ops.score_select(cfg, Q, kc, vc, sel=sel, lse=lse, o_cmp=ocmp, workspace=ws[1])
        gdo = torch.Generator(device=dev).manual_seed(cfg.seed + 1000)
        dO = torch.randn((B, T, H, cfg.d_v), generator=gdo, device=dev).to(torch.bfloat16)
        wsb = torch.empty(ops.workspace_size(cfg, ops.OP_SPARSE_BWD), dtype=torch.uint8, device=dev)
        wsc = torch.empty(max(ops.workspace_size(cfg, ops.OP_COMPRESS_BWD), 256), dtype=torch.uint8, device=dev)
        grads = {}
        # the training forward: the same O plus the selected and window branches' LSE and
        # outputs, which the backward reads instead of recomputing them
        saved = {}

        def fwd_train():
            _, saved["lse"], saved["o"] = ops.sparse_attn_fwd_train(cfg, Q, K, V, sel, ocmp, gates, out=out,
                                                                    workspace=ws[2])

        pct, _ = time_calls([fwd_train], 3, 1, torch)

        def bwd_attn():
            grads.update(ops.sparse_attn_bwd(cfg, Q, K, V, kc, vc, sel, lse, ocmp, gates, dO, saved_lse=saved["lse"],
                                             saved_o=saved["o"], workspace=wsb))

        def bwd_map():
            grads.update(ops.compress_bwd(cfg, K, V, wk, wv, pk, pv, grads["dk_cmp"], grads["dv_cmp"], grads["dk"],
                                          grads["dv"], workspace=wsc))

        pcb, wallb = time_calls([bwd_attn, bwd_map], 3, 1, torch)
        bms = float(pcb.sum(axis=1).mean())
        bfl = backward_flops(cfg)
        btf = sum(bfl.values()) / (bms * 1e-3) / 1e12
        result["backward"] = {
            "workload": "nsa_backward_64k", "ms_per_step": round(bms, 3),
            "tokens_per_s": round(B * T / (bms * 1e-3), 1),
            "saved_statistics": "from nsa_sparse_attn_fwd_train",
            "fwd_train_ms": round(float(pct.mean()), 3),
            "per_call_ms": {"nsa_sparse_attn_bwd": round(float(pcb[:, 0].mean()), 3),
                            "nsa_compress_bwd": round(float(pcb[:, 1].mean()), 3)},
            "algorithmic_flops": {k: int(v) for k, v in bfl.items()},
            "tflops_algorithmic": round(btf, 2), "mfma_peak_frac": round(btf / PEAK_BF16_TFLOPS, 4)}
        del grads, dO, wsb, wsc, lse, saved
        torch.cuda.empty_cache()

    if not args.no_decode:
        del Q, K, V, ocmp, out
        torch.cuda.empty_cache()
        dc = DECODE
        print("[bench] decode inputs", file=sys.stderr, flush=True)
        g = torch.Generator(device=dev).manual_seed(dc.seed)
        Bd, L = dc.batch, dc.seq_len
        q = torch.randn((Bd, dc.num_heads, dc.d_k), generator=g, device=dev).to(torch.bfloat16)
        Kd = torch.randn((Bd, dc.num_kv_heads, L, dc.d_k), generator=g, device=dev).to(torch.bfloat16)
        Vd = torch.randn((Bd, dc.num_kv_heads, L, dc.d_v), generator=g, device=dev).to(torch.bfloat16)
        gd = torch.randn((Bd, dc.num_heads, 3), generator=g, device=dev)
        clen = torch.full((Bd,), L, dtype=torch.int32, device=dev)
        kcd, vcd = ops.compress(dc, Kd, Vd, wk, wv, pk, pv)
        od = torch.empty((Bd, dc.num_heads, dc.d_v), dtype=torch.bfloat16, device=dev)
        sd = torch.empty((Bd, dc.num_kv_heads, dc.top_n), dtype=torch.int32, device=dev)
        wsd = torch.empty(ops.workspace_size(dc, ops.OP_DECODE), dtype=torch.uint8, device=dev)
        dcall = [lambda: ops.decode(dc, q, Kd, Vd, clen, kcd, vcd, gd, out=od, sel=sd, workspace=wsd)]
        pcd, _ = time_calls(dcall, max(20, args.steps), args.warmup + 3, torch)
        dms = float(pcd.mean())
        # bytes: compressed caches + raw K/V of the union of selected blocks and the window + q, O
        s_np = sd.cpu().numpy()
        raw_tok = 0
        for b in range(Bd):
            t = L - 1
            for gg in range(dc.num_kv_heads):
                toks = set()
                for j in s_np[b, gg]:
                    if j >= 0:
                        toks.update(range(j * dc.slc_block, min((j + 1) * dc.slc_block, t + 1)))
                toks.update(range(max(0, t - dc.window + 1), t + 1))
                raw_tok += len(toks)
        bytes_step = (kcd.numel() + vcd.numel()) * 2 + raw_tok * (dc.d_k + dc.d_v) * 2 + (q.numel() + od.numel()) * 2
        gbs = bytes_step / (dms * 1e-3) / 1e9
        result["decode"] = {"workload": "nsa_decode_b32_l65536", "ms_per_step": round(dms, 4),
                            "bytes_per_step": int(bytes_step), "hbm_gbs": round(gbs, 1),
                            "hbm_peak_frac": round(gbs / PEAK_HBM_GBS, 4)}
        # the same step replayed from a captured HIP graph of 20 steps (the serving loop's
        # form: no host launch work between the kernels)
        try:
            gd_ = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gd_):
                for _ in range(20):
                    dcall[0]()
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gd_.replay()
            torch.cuda.synchronize()
            ea.record()
            gd_.replay()
            eb.record()
            torch.cuda.synchronize()
            gms = ea.elapsed_time(eb) / 20
            result["decode"]["graph_ms_per_step"] = round(gms, 4)
            result["decode"]["graph_hbm_gbs"] = round(bytes_step / (gms * 1e-3) / 1e9, 1)
            del gd_
        except RuntimeError as e:
            result["decode"]["graph_note"] = f"graph capture failed: {e}"[:200]
        # cache maintenance before each step: one new token per sequence into the caches,
        # a new compressed entry every s calls (timed over 2*s calls, after the decode timing)
        prep = ops.compress_prepare(dc, wk, wv, pk, pv)
        kn = torch.randn((Bd, dc.num_kv_heads, 1, dc.d_k), generator=g, device=dev).to(torch.bfloat16)
        vn = torch.randn((Bd, dc.num_kv_heads, 1, dc.d_v), generator=g, device=dev).to(torch.bfloat16)
        clen2 = torch.full((Bd,), L - 4 * dc.cmp_stride * 4, dtype=torch.int32, device=dev)
        acall = [lambda: ops.cache_append(dc, kn, vn, Kd, Vd, clen2, kcd, vcd, prep)]
        pca, _ = time_calls(acall, 2 * dc.cmp_stride, 2, torch)
        result["decode"]["append_us_per_token_eager"] = round(float(pca.mean()) * 1e3, 2)
        # one eager call is bound by the host (a ctypes call and two launches); the GPU time
        # comes from replaying a captured graph of s consecutive appends (one of which
        # completes a compressed block)
        try:
            clen2.fill_(L - 4 * dc.cmp_stride * 4)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(dc.cmp_stride):
                    ops.cache_append(dc, kn, vn, Kd, Vd, clen2, kcd, vcd, prep)
            ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            clen2.fill_(L - 4 * dc.cmp_stride * 4)
            torch.cuda.synchronize()
            ga.record()
            gr.replay()
            gb.record()
            torch.cuda.synchronize()
            result["decode"]["append_us_per_token"] = round(ga.elapsed_time(gb) * 1e3 / dc.cmp_stride, 2)
            del gr
        except RuntimeError as e:   # capture unavailable: the eager figure stands
            result["decode"]["append_us_per_token"] = result["decode"]["append_us_per_token_eager"]
            result["decode"]["append_note"] = f"graph capture failed: {e}"[:200]
        del Kd, Vd, kcd, vcd
        torch.cuda.empty_cache()

    # ---------------- MoBA (the 128K workload, and 1M tokens) ----------------
    if not args.no_moba:
        for mc, key, steps in ((MOBA, "moba", 10), (MOBA.replace(name="moba_1m", seq_len=1 << 20), "moba_1m", 3)):
            print(f"[bench] {key} inputs", file=sys.stderr, flush=True)
            g = torch.Generator(device=dev).manual_seed(mc.seed)
            Qm = torch.randn((1, mc.seq_len, mc.num_heads, mc.d_k), generator=g, device=dev).to(torch.bfloat16)
            Km = torch.randn((1, mc.num_kv_heads, mc.seq_len, mc.d_k), generator=g, device=dev).to(torch.bfloat16)
            Vm = torch.randn((1, mc.num_kv_heads, mc.seq_len, mc.d_v), generator=g, device=dev).to(torch.bfloat16)
            kbar = torch.empty((1, mc.num_kv_heads, mc.n_cmp, mc.d_k), dtype=torch.bfloat16, device=dev)
            selm = torch.empty((1, mc.seq_len, mc.num_kv_heads, mc.top_n), dtype=torch.int32, device=dev)
            om = torch.empty((1, mc.seq_len, mc.num_heads, mc.d_v), dtype=torch.bfloat16, device=dev)
            wsm = torch.empty(ops.workspace_size(mc, ops.OP_SPARSE_ATTN), dtype=torch.uint8, device=dev)
            mcalls = [lambda: ops.compress(mc, Km, out_k=kbar),
                      lambda: ops.score_select(mc, Qm, kbar, sel=selm),
                      lambda: ops.sparse_attn_fwd(mc, Qm, Km, Vm, selm, out=om, workspace=wsm)]
            pcm, _ = time_calls(mcalls, steps, 1, torch)
            mms = float(pcm.sum(axis=1).mean())
            result[key] = {"workload": f"moba_{mc.seq_len}_h8_d128", "ms_per_step": round(mms, 3),
                           "tokens_per_s": round(mc.seq_len / (mms * 1e-3), 1),
                           "tflops_algorithmic": round(moba_flops(mc) / (mms * 1e-3) / 1e12, 2),
                           "per_call_ms": {n: round(float(c), 3) for n, c in zip(names3, pcm.mean(axis=0))}}
            del Qm, Km, Vm, kbar, selm, om, wsm
            torch.cuda.empty_cache()

    # ---------------- measured ceilings ----------------
    if not args.no_ceilings:
        print("[bench] ceilings", file=sys.stderr, flush=True)
        result["ceilings"] = ceilings(torch, dev)

    # ---------------- CPU baseline ----------------
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(P64K, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
