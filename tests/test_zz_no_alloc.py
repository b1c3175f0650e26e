"""nsa_decode_noalloc (the decode step with the library's fixed device scratch instead of
a caller workspace) against nsa_decode with a workspace, through the C ABI.

Two calls in a row, the second with a smaller input: the 32 x 65536-token decode step
(30 MiB of scratch), then 4 sequences of 8192-token caches at mixed lengths.  The two entry
points run the same kernels on the same inputs, so their outputs and selections must be
equal bit for bit (this is stricter than the output bar, which is checked as well).  A
configuration that needs more scratch than the array holds is rejected before any launch.
"""
import ctypes

import pytest
import torch

from dynamic_block_sparse_nsa_amd import ops
from dynamic_block_sparse_nsa_amd.configs import DECODE
from nsa_testlib import check_close

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[no-alloc] {msg}", flush=True)


def _inputs(cfg, seed, lens):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    B, L, H, Hkv, l = cfg.batch, cfg.seq_len, cfg.num_heads, cfg.num_kv_heads, cfg.cmp_block

    def bf(shape, scale=1.0):
        return (torch.randn(shape, generator=g, device=dev) * scale).to(torch.bfloat16)

    wk, wv = bf((l * cfg.d_k, cfg.d_k), 0.03), bf((l * cfg.d_v, cfg.d_v), 0.03)
    pk, pv = bf((l, cfg.d_k)), bf((l, cfg.d_v))
    K, V = bf((B, Hkv, L, cfg.d_k)), bf((B, Hkv, L, cfg.d_v))
    kc, vc = ops.compress(cfg, K, V, wk, wv, pk, pv)
    q = bf((B, H, cfg.d_k))
    gates = torch.randn((B, H, 3), generator=g, device=dev)
    clen = torch.tensor(lens, dtype=torch.int32, device=dev)
    return q, K, V, clen, kc, vc, gates


def _one_call(cfg, seed, lens):
    announce(f"{cfg.name}: B={cfg.batch} L={cfg.seq_len} scratch need "
             f"{ops.workspace_size(cfg, ops.OP_DECODE) / 2**20:.1f} MiB")
    q, K, V, clen, kc, vc, gates = _inputs(cfg, seed, lens)
    o_ref, s_ref = ops.decode(cfg, q, K, V, clen, kc, vc, gates)
    out = torch.full_like(o_ref, float("nan"))
    sel = torch.full_like(s_ref, -7)
    ops.decode_noalloc(cfg, q, K, V, clen, kc, vc, gates, out=out, sel=sel)
    torch.cuda.synchronize()
    assert torch.equal(sel, s_ref), f"{cfg.name}: selections differ"
    check_close(out.float().cpu().numpy(), o_ref.float().cpu().numpy(), f"{cfg.name} no-alloc vs workspace")
    assert torch.equal(out, o_ref), f"{cfg.name}: outputs differ"
    del q, K, V, kc, vc
    torch.cuda.empty_cache()


def test_decode_noalloc_matches_workspace_entry_point():
    big = DECODE.replace(name="noalloc_b32_l65536")
    _one_call(big, 81, [big.seq_len] * big.batch)
    small = DECODE.replace(name="noalloc_b4_l8192", batch=4, seq_len=8192)
    _one_call(small, 82, [8192, 4097, 600, 31])


def test_decode_noalloc_rejects_oversize():
    cfg = DECODE.replace(name="noalloc_oversize", batch=160)
    need = ops.workspace_size(cfg, ops.OP_DECODE)
    announce(f"oversize: need {need / 2**20:.1f} MiB")
    assert need > 64 * 2**20
    fake = ctypes.c_void_p(256)
    rc = ops.lib().nsa_decode_noalloc(ctypes.byref(ops.c_config(cfg)), fake, fake, fake, fake, fake, fake, None,
                                      fake, None, None)
    assert rc == 4, rc
    assert "scratch" in ops.lib().nsa_last_error_detail().decode()
