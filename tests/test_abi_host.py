"""Host-side checks of the C ABI and the input generators (no GPU needed).

Every library call validates its arguments before launching anything, so the error
paths run here without a device.  The library must load and export every entry point
that include/nsa.h declares.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from dynamic_block_sparse_nsa_amd import inputs
from dynamic_block_sparse_nsa_amd.configs import CONFIGS, TINY, P8K, MOBA, DECODE

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa.h")

torch = pytest.importorskip("torch")
from dynamic_block_sparse_nsa_amd import ops  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:nsa_status|const char\*)\s+(nsa_\w+)\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = ops.lib()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    # nothing beyond the header is exported under the nsa_ prefix
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r" T (nsa_\w+)", out)))
    assert exported == names


def test_ceilings_library_exports_its_header():
    """libnsa_ceilings.so (the roofline microbenchmarks) exports exactly what
    include/nsa_ceilings.h declares, and rejects invalid arguments before any launch."""
    from dynamic_block_sparse_nsa_amd.build import CEIL_LIB, build_ceilings
    if not os.path.exists(CEIL_LIB):
        build_ceilings()
    text = open(os.path.join(os.path.dirname(HEADER), "nsa_ceilings.h")).read()
    names = sorted(set(re.findall(r"^int\s+(nsa_\w+)\(", text, re.M)))
    assert names == ["nsa_ceiling_gather", "nsa_ceiling_mfma", "nsa_ceiling_stream"]
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", CEIL_LIB], capture_output=True, text=True).stdout
    assert sorted(set(re.findall(r" T (nsa_\w+)", out))) == names
    C = ctypes.CDLL(CEIL_LIB)
    fake = ctypes.c_void_p(0x1000)
    assert C.nsa_ceiling_mfma(None, 1, 1, None) == 1
    assert C.nsa_ceiling_stream(fake, ctypes.c_size_t(17), fake, 1, None) == 1
    assert C.nsa_ceiling_gather(fake, fake, 4, 1000, fake, None) == 1


def test_struct_layout_matches_header():
    # 1 uint32 + 16 int32 + 1 float
    assert ctypes.sizeof(ops.CConfig) == 4 * 18


def _cfg(c=P8K, **over):
    return ctypes.byref(ops.c_config(c, **over))


def _ws(c=P8K, op=0, **over):
    n = ctypes.c_size_t(0)
    rc = ops.lib().nsa_workspace_size(_cfg(c, **over), op, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_sizes(name):
    c = CONFIGS[name]
    for op in range(5):
        rc, n = _ws(c, op)
        assert rc == 0
        assert n % 256 == 0
    # the scores workspace (B*T*Hkv*N_slc fp32), absent when mean-key scoring with one query
    # head per KV head and at most 4 free picks selects inside the scoring kernel
    rc, n = _ws(c, ops.OP_SCORE_SELECT)
    al = lambda x: -(-x // 256) * 256
    if c.score_mode == 1 and c.heads_per_group == 1 and c.top_n - c.n_local <= 4:
        assert n == 0
    else:
        assert n >= al(c.batch * c.seq_len * c.num_kv_heads * c.n_slc * 4)
    # dense attention: K in bf16 and V in fp16, fragment order, roundup(T, 64) keys, plus the
    # value scaling (64 partial maxima and one exponent per (b, g))
    rc, n = _ws(c, ops.OP_FULL_ATTN)
    tp = -(-c.seq_len // 64) * 64
    al = lambda x: -(-x // 256) * 256
    bg = c.batch * c.num_kv_heads
    assert n == al(bg * c.d_k * tp * 2) + al(bg * c.d_v * tp * 2) + al(bg * 64 * 4) + al(bg * 4)
    # the attention workspace holds V in MFMA fragment order, padded:
    # B*Hkv*d_v*(roundup(T,64)+64)*2 bytes (each part 256-byte aligned), V's fp16 scaling (64
    # partial maxima and one exponent per (b, g)), then K in the same order; G = 1 with only
    # the selected branch puts the block lists and per-slot partials (max and sum in fp32,
    # the normalized partial output in fp16) over the K copy's bytes, the larger of the two
    rc, n = _ws(c, ops.OP_SPARSE_ATTN)
    tp = -(-c.seq_len // 64) * 64 + 64
    al = lambda x: -(-x // 256) * 256
    bg = c.batch * c.num_kv_heads
    union = al(bg * c.d_k * tp * 2)
    if c.heads_per_group == 1 and c.branches == 2:
        n_chunk = -(-c.seq_len // 1024)
        rows = bg * c.seq_len * c.top_n
        max_tiles = rows // 128 + bg * c.n_slc   # every bucket: at most ceil(n / 128) list tiles
        union = max(union, al(bg * n_chunk * c.n_slc * 4) + al(bg * c.n_slc * 4) + 2 * al((bg * c.n_slc + 1) * 4)
                    + al(max_tiles * 4) + 3 * al(rows * 4) + al(rows * c.d_v * 2))
    want = al(bg * c.d_v * tp * 2) + al(bg * 64 * 4) + al(bg * 4) + union
    assert n == want
    # the fused prefill: the scoring call's and the attention call's workspaces side by side,
    # then room for the lists (int32) and o_cmp (fp32) the caller may not take
    rc, n = _ws(c, ops.OP_PREFILL)
    assert rc == 0
    if c.score_mode == 0:
        _, n_sel = _ws(c, ops.OP_SCORE_SELECT)
        _, n_att = _ws(c, ops.OP_SPARSE_ATTN)
        assert n == n_sel + n_att + al(c.batch * c.seq_len * c.num_kv_heads * c.top_n * 4) + al(
            c.batch * c.seq_len * c.num_heads * c.d_v * 4)


def test_prefill_fwd_validation():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    big = 1 << 40
    # Q, K, V, K_cmp, V_cmp and O are required
    for i in range(6):
        args = [fake] * 6
        args[i] = None
        q, k, v, kc, vc, o = args
        assert L.nsa_prefill_fwd(_cfg(), q, k, v, kc, vc, None, o, None, None, None, fake, big, None) == 1
    # workspace too small / unaligned
    assert L.nsa_prefill_fwd(_cfg(), fake, fake, fake, fake, fake, None, fake, None, None, None, fake, 16, None) == 4
    assert L.nsa_prefill_fwd(_cfg(), fake, fake, fake, fake, fake, None, fake, None, None, None,
                             ctypes.c_void_p(0x1001), big, None) == 4
    # mean-key scores are not fused
    assert L.nsa_prefill_fwd(_cfg(MOBA), fake, fake, fake, fake, fake, None, fake, None, None, None, fake, big,
                             None) == 3
    # window branch with window 0
    assert L.nsa_prefill_fwd(_cfg(P8K, window=0), fake, fake, fake, fake, fake, None, fake, None, None, None, fake,
                             big, None) == 2


@pytest.mark.parametrize("over,status", [
    ({"heads_per_group": 3}, 3),
    ({"d_k": 96}, 3),
    ({"cmp_stride": 5}, 3),
    ({"slc_block": 48}, 3),
    ({"top_n": 2}, 3),               # fewer than the 3 forced blocks
    ({"top_n": 40}, 3),
    ({"batch": 0}, 2),
    ({"seq_len": -1}, 2),
    ({"window": -1}, 2),
    ({"branches": 0}, 2),
    ({"branches": 9}, 2),
    ({"phi": 7}, 2),
    ({"score_mode": 1}, 3),          # mean-key scores need l == s == l'
    ({"struct_size": 8}, 2),
])
def test_config_validation(over, status):
    rc, _ = _ws(P8K, 0, **over)
    assert rc == status
    assert ops.lib().nsa_last_error_detail().decode() != ""


def test_null_config_and_output():
    L = ops.lib()
    n = ctypes.c_size_t(0)
    assert L.nsa_workspace_size(None, 0, ctypes.byref(n)) == 1
    assert L.nsa_workspace_size(_cfg(), 0, None) == 1
    assert L.nsa_workspace_size(_cfg(), 9, ctypes.byref(n)) == 2


def test_calls_reject_null_pointers_before_launch():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.nsa_compress(_cfg(), None, fake, fake, fake, fake, fake, fake, fake, None, 0, None) == 1
    assert L.nsa_compress(_cfg(), fake, None, fake, fake, fake, fake, fake, fake, None, 0, None) == 1
    assert L.nsa_score_select(_cfg(), None, fake, fake, fake, None, None, None, 0, None) == 1
    assert L.nsa_score_select(_cfg(), fake, fake, fake, None, None, None, None, 0, None) == 1
    assert L.nsa_sparse_attn_fwd(_cfg(), fake, fake, None, fake, fake, None, fake, None, 0, None) == 1
    assert L.nsa_sparse_attn_fwd(_cfg(), fake, fake, fake, None, fake, None, fake, None, 0, None) == 1
    assert L.nsa_sparse_attn_fwd(_cfg(), fake, fake, fake, fake, None, None, fake, None, 0, None) == 1
    assert L.nsa_decode(_cfg(DECODE), fake, fake, fake, None, fake, fake, None, fake, None, None, 0, None) == 1
    assert L.nsa_decode_noalloc(_cfg(DECODE), fake, fake, fake, None, fake, fake, None, fake, None, None) == 1
    assert L.nsa_decode_noalloc(_cfg(DECODE), fake, fake, fake, fake, fake, fake, None, None, None, None) == 1
    assert L.nsa_select_from_scores(_cfg(), None, fake, None) == 1
    assert L.nsa_full_attn_fwd(_cfg(), fake, fake, fake, None, fake, 1 << 40, None) == 1
    assert L.nsa_full_attn_fwd(_cfg(), None, fake, fake, fake, fake, 1 << 40, None) == 1


def test_calls_reject_small_workspace_before_launch():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.nsa_compress(_cfg(), fake, fake, fake, fake, fake, fake, fake, fake, None, 0, None) == 4
    assert L.nsa_score_select(_cfg(), fake, fake, fake, fake, None, fake, fake, 16, None) == 4
    assert L.nsa_sparse_attn_fwd(_cfg(), fake, fake, fake, fake, fake, None, fake, fake, 16, None) == 4
    assert L.nsa_decode(_cfg(DECODE), fake, fake, fake, fake, fake, fake, None, fake, None, fake, 16, None) == 4
    # the allocation-free decode: a configuration whose scratch exceeds the fixed 64 MiB array
    big_b = _cfg(DECODE.replace(batch=160))
    assert L.nsa_decode_noalloc(big_b, fake, fake, fake, fake, fake, fake, None, fake, None, None) == 4
    assert b"scratch" in L.nsa_last_error_detail()
    assert L.nsa_full_attn_fwd(_cfg(), fake, fake, fake, fake, fake, 16, None) == 4
    # unaligned workspace
    big = 1 << 40
    assert L.nsa_sparse_attn_fwd(_cfg(), fake, fake, fake, fake, fake, None, fake, ctypes.c_void_p(0x1001), big,
                                 None) == 4


def test_mode_specific_rules():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    # MEAN_DOT mode cannot produce o_cmp / lse
    assert L.nsa_score_select(_cfg(MOBA), fake, fake, None, fake, fake, None, None, 0, None) == 2
    # decode implements the NSA mode only
    assert L.nsa_decode(_cfg(MOBA), fake, fake, fake, fake, fake, fake, None, fake, None, fake, 1 << 40, None) == 3
    # decode: a selection block overlapping more compressed keys than one 256-key split holds
    wide = _cfg(DECODE, cmp_stride=1, slc_block=256, seq_len=1024)
    assert L.nsa_decode(wide, fake, fake, fake, fake, fake, fake, None, fake, None, fake, 1 << 40, None) == 3
    assert "cmp_stride" in L.nsa_last_error_detail().decode()
    # window branch needs a window
    assert L.nsa_sparse_attn_fwd(_cfg(P8K, window=0), fake, fake, fake, fake, fake, None, fake, None, 0, None) == 2
    # shorter than one compressed block: supported (no compressed key; the compressed tensors
    # may be NULL), still validated before any launch
    short = _cfg(P8K, seq_len=16)
    assert L.nsa_score_select(short, fake, None, None, None, None, None, fake, 1 << 40, None) == 1
    assert L.nsa_score_select(short, fake, None, None, fake, None, None, fake, 0, None) == 4
    n = ctypes.c_size_t(0)
    assert L.nsa_workspace_size(short, ops.OP_SCORE_SELECT, ctypes.byref(n)) == 0
    assert n.value >= 16 * 4 * 1 * 4   # the zero score rows [B, T, H_kv, N_slc]


def test_cache_maintenance_validation():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    big = 1 << 40
    prep_ok = ctypes.c_void_p(0x100000)
    # prepare: null weights, short or unaligned buffer, non-linear phi
    assert L.nsa_compress_prepare(_cfg(DECODE), None, fake, fake, fake, prep_ok, big, None) == 1
    assert L.nsa_compress_prepare(_cfg(DECODE), fake, fake, fake, fake, prep_ok, 16, None) == 4
    assert L.nsa_compress_prepare(_cfg(DECODE), fake, fake, fake, fake, ctypes.c_void_p(0x100010), big, None) == 4
    assert L.nsa_compress_prepare(_cfg(MOBA), fake, fake, fake, fake, prep_ok, big, None) == 3
    # append: null arguments, n_new outside [1, L], short prep, unaligned tokens, mean phi
    args = lambda n_new, prep_bytes=big, knew=fake: (knew, fake, n_new, fake, fake, fake, fake, fake, prep_ok,
                                                     prep_bytes, None)
    assert L.nsa_cache_append(_cfg(DECODE), *args(1, knew=None)) == 1
    assert L.nsa_cache_append(_cfg(DECODE), *args(0)) == 2
    assert L.nsa_cache_append(_cfg(DECODE), *args(DECODE.seq_len + 1)) == 2
    assert L.nsa_cache_append(_cfg(DECODE), *args(1, prep_bytes=16)) == 4
    assert L.nsa_cache_append(_cfg(DECODE), *args(1, knew=ctypes.c_void_p(0x1008))) == 2
    assert L.nsa_cache_append(_cfg(MOBA), *args(1)) == 3
    assert L.nsa_last_error_detail().decode() != ""


def test_status_strings():
    L = ops.lib()
    for code in range(6):
        assert L.nsa_status_string(code).decode()
    assert L.nsa_status_string(77).decode() == "unknown status"


# ---------------------------------------------------------------------------
# input generators
# ---------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:8] = [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0078125, 65504.0, 1e-30]
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(inputs.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_chunked_draws_equal_single_draw():
    a = inputs._normal_bf16(np.random.Generator(np.random.PCG64(3)), (5, (1 << 24) // 5 + 7))
    b = inputs.f32_to_bf16_bits(np.random.Generator(np.random.PCG64(3)).standard_normal(a.size, dtype=np.float32))
    np.testing.assert_array_equal(a.reshape(-1), b)


def test_prefill_inputs_shapes_and_determinism():
    a = inputs.prefill_inputs(TINY)
    b = inputs.prefill_inputs(TINY)
    for k in ("q", "k", "v", "w_k", "w_v", "pe_k", "pe_v", "gates"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["q"].shape == (1, 1024, 4, 64) and a["k"].shape == (1, 1, 1024, 64)
    assert a["w_k"].shape == (32 * 64, 64)
    # the fp32 draws round to the bf16 arrays
    np.testing.assert_array_equal(inputs.f32_to_bf16_bits(a["raw"]["q"]), a["q"])
    # Xavier bound
    wk = inputs.bf16_bits_to_f32(a["w_k"])
    assert np.abs(wk).max() <= np.sqrt(6.0 / (32 * 64 + 64)) * 1.01


def test_block_lists_structure():
    cfg = TINY.replace(seq_len=700)
    pos = np.arange(700)
    sel = inputs.block_lists(cfg, 5, pos)
    for t in range(0, 700, 7):
        row = sel[0, t, 0]
        jc = t // 64
        valid = row[row >= 0]
        assert (np.diff(valid) > 0).all()
        assert valid.max() == jc and valid.min() == 0
        assert len(valid) == min(cfg.top_n, jc + 1)
        assert (row[len(valid):] == -1).all()
        if jc >= 1:
            assert jc - 1 in valid


def test_backward_validation():
    """nsa_sparse_attn_bwd, nsa_sparse_attn_fwd_train and nsa_compress_bwd reject missing
    pointers, a lone saved buffer, misalignment, a small workspace and the mean block map
    before launching anything."""
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    big = 1 << 40
    for op in (ops.OP_SPARSE_BWD, ops.OP_COMPRESS_BWD):
        rc, n = _ws(P8K, op)
        assert rc == 0 and n > 0
    ws_ok = ctypes.c_void_p(0x100000)

    def bwd(**over):
        a = dict(Q=fake, K=fake, V=fake, Kc=fake, Vc=fake, sel=fake, lse=fake, ocmp=fake, gates=fake, slse=None,
                 so=None, dO=fake, dQ=fake, dK=fake, dV=fake, dKc=fake, dVc=fake, dg=fake, ws=ws_ok, nws=big)
        a.update(over)
        cfg = a.pop("cfg", _cfg())
        return L.nsa_sparse_attn_bwd(cfg, a["Q"], a["K"], a["V"], a["Kc"], a["Vc"], a["sel"], a["lse"], a["ocmp"],
                                     a["gates"], a["slse"], a["so"], a["dO"], a["dQ"], a["dK"], a["dV"], a["dKc"],
                                     a["dVc"], a["dg"], a["ws"], a["nws"], None)

    assert bwd(dO=None) == 1
    assert bwd(dQ=None) == 1
    assert bwd(sel=None) == 1                          # selected branch on
    assert bwd(lse=None) == 1                          # compressed branch on
    assert bwd(dKc=None) == 1
    assert bwd(gates=None) == 1                        # d_gate_logits without gate logits
    assert bwd(slse=fake) == 1                         # saved LSE without saved outputs
    assert bwd(so=fake) == 1
    assert bwd(slse=fake, so=odd) == 2                 # saved outputs misaligned
    assert bwd(dK=odd) == 2
    assert bwd(ws=None, nws=0) == 4
    assert bwd(nws=16) == 4
    assert bwd(cfg=_cfg(P8K, window=0)) == 2           # window branch with window 0
    # with the compressed branch off, its buffers may be NULL (fails later only on the workspace)
    assert bwd(cfg=_cfg(P8K, branches=6), Kc=None, Vc=None, lse=None, ocmp=None, dKc=None, dVc=None, nws=16) == 4

    def train(**over):
        a = dict(Q=fake, K=fake, V=fake, sel=fake, ocmp=fake, gates=None, O=fake, slse=fake, so=fake, ws=ws_ok,
                 nws=big)
        a.update(over)
        return L.nsa_sparse_attn_fwd_train(_cfg(), a["Q"], a["K"], a["V"], a["sel"], a["ocmp"], a["gates"], a["O"],
                                           a["slse"], a["so"], a["ws"], a["nws"], None)

    assert train(slse=None) == 1
    assert train(so=None) == 1
    assert train(so=odd) == 2
    assert train(O=None) == 1
    assert train(nws=16) == 4

    def cbwd(**over):
        a = dict(K=fake, V=fake, wk=fake, wv=fake, pk=fake, pv=fake, dKc=fake, dVc=fake, dK=fake, dV=fake, dWk=fake,
                 dWv=fake, dpk=fake, dpv=fake, ws=ws_ok, nws=big)
        a.update(over)
        cfg = a.pop("cfg", _cfg())
        return L.nsa_compress_bwd(cfg, a["K"], a["V"], a["wk"], a["wv"], a["pk"], a["pv"], a["dKc"], a["dVc"], a["dK"],
                                  a["dV"], a["dWk"], a["dWv"], a["dpk"], a["dpv"], a["ws"], a["nws"], None)

    assert cbwd(dKc=None) == 1
    assert cbwd(dpv=None) == 1
    assert cbwd(dWk=odd) == 2
    assert cbwd(nws=16) == 4
    assert cbwd(cfg=_cfg(MOBA)) == 3
