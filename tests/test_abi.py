"""C-ABI boundary checks that run without a GPU.

The library must load, export every function include/msa.h declares, and
reject bad arguments on the host before any HIP call (every case below stops
in validation, so no device is touched).
"""
import ctypes
import os
import re

import pytest

import block_sparse_top_msa_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # never dereferenced: validation fails before any launch


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", src)))


def test_header_declarations_are_exported():
    names = _declared_functions()
    assert len(names) == 15, names
    assert set(names) == set(msa.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(msa.lib, n), n


def test_status_strings_and_version():
    assert msa.lib.msa_status_string(0) == b"MSA_OK"
    assert msa.lib.msa_status_string(4) == b"MSA_ERR_CONFLICT"
    assert msa.lib.msa_status_string(8) == b"MSA_ERR_CONTRACT"
    assert msa.lib.msa_version().decode().count(".") == 2


def _attn(**kw):
    a = msa.AttnArgs()
    a.batch, a.total_q, a.num_qo_heads, a.num_kv_heads = 2, 8, 8, 2
    a.head_dim, a.topk, a.max_seqlen_q, a.max_k_tiles = 128, 4, 4, 4
    a.q = a.k = a.v = a.out = a.q2k = a.cu_seqlens_q = a.cu_seqlens_k = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _call(a, ws=None, nbytes=0):
    st = msa.lib.msa_sparse_attention(ctypes.byref(a), ws, nbytes, None)
    return st, msa.lib.msa_last_error().decode()


def _size(a):
    n = ctypes.c_size_t(0)
    st = msa.lib.msa_sparse_attention_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, 2),
    ("num_kv_heads", 3, 2),
    ("topk", 0, 2),
    ("topk", 65, 2),
    ("kv_dtype", 7, 3),
    ("max_k_tiles", 1 << 20, 2),
])
def test_attention_rejects_bad_shapes(field, value, status):
    st, msg = _call(_attn(**{field: value}))
    assert st == status and msg


def test_attention_paged_conflict_and_missing_lengths():
    a = _attn(page_table=FAKE, seqused_k=FAKE, page_table_width=4)  # cu_seqlens_k still set
    st, msg = _call(a)
    assert st == 4 and "seqused_k" in msg
    b = _attn(page_table=FAKE, page_table_width=4)
    b.cu_seqlens_k = None
    st, _ = _call(b)
    assert st == 1
    c = _attn(page_table=FAKE, seqused_k=FAKE, page_table_width=2)
    c.cu_seqlens_k = None
    st, msg = _call(c)
    assert st == 2 and "page_table_width" in msg


def test_attention_rejects_unreadable_views():
    a = _attn()
    a.k_strides = msa.Strides(0, 256, 100)  # token stride not 16-byte aligned
    st, msg = _call(a)
    assert st == 5 and "never copied" in msg
    b = _attn(q=FAKE + 8)
    st, _ = _call(b)
    assert st == 5
    # a 128-token block is addressed as base + 32-bit lane offset: token
    # strides past 16 MiB are refused
    c = _attn()
    c.v_strides = msa.Strides(0, 256, (1 << 24) + 16)
    st, msg = _call(c)
    assert st == 5 and "token stride" in msg


def test_attention_e2m1_needs_scales_with_contiguous_rows():
    st, _ = _call(_attn(kv_dtype=2))  # flat E2M1 without scales
    assert st == 1
    # paged scales whose rows are 16 bytes apart: the decode kernel's
    # two-row staging cannot read them
    a = _attn(kv_dtype=2, page_table=FAKE, seqused_k=FAKE, page_table_width=4, k_scale=FAKE,
              v_scale=FAKE)
    a.cu_seqlens_k = None
    a.k_scale_strides = msa.Strides(0, 0, 16)
    st, msg = _call(a)
    assert st == 5 and "paged k_scale/v_scale" in msg
    a = _attn(kv_dtype=2, page_table=FAKE, seqused_k=FAKE, page_table_width=4)
    a.cu_seqlens_k = None
    st, _ = _call(a)
    assert st == 1  # no scales
    st, _ = _call(_attn(k_scale=FAKE))  # scales with bf16
    assert st == 5


def test_temperature_lse_needs_a_finite_positive_scale():
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        st, msg = _call(_attn(lse_t=FAKE, lse_temperature_scale=tau))
        assert st == 5 and "lse_temperature_scale" in msg
    # the temperature LSE keeps the decode route and its split partials: the
    # workspace grows by one partial per row and split
    a = _attn(num_qo_heads=32, num_kv_heads=2, total_q=4, batch=4, max_seqlen_q=1,
              max_k_tiles=64, topk=16, page_table=FAKE, seqused_k=FAKE, page_table_width=64,
              splits=4)
    a.cu_seqlens_k = None
    st, n0 = _size(a)
    assert _plan(a)[:2] == (0, 1)
    a.lse_t, a.lse_temperature_scale = FAKE, 2.0
    st, n1 = _size(a)
    assert st == 0 and n1 > n0
    assert _plan(a)[:2] == (0, 1)


def test_workspace_sizing_and_enforcement():
    # decode shape (1 query x 16 heads per KV head): splits > 1 need a workspace
    a = _attn(num_qo_heads=32, num_kv_heads=2, total_q=4, batch=4, max_seqlen_q=1,
              max_k_tiles=64, topk=16, page_table=FAKE, seqused_k=FAKE, page_table_width=64)
    a.cu_seqlens_k = None
    st, n = _size(a)
    assert st == 0 and n > 0
    st, msg = _call(a, None, 0)
    assert st == 6 and "workspace" in msg
    st, _ = _call(a, FAKE, n - 1)
    assert st == 6
    st, _ = _call(a, FAKE + 4, n + 8)  # misaligned
    assert st == 6
    # forcing one split needs no workspace
    a.splits = 1
    assert _size(a) == (0, 0)
    # prefill shape never splits
    assert _size(_attn(max_seqlen_q=512, num_qo_heads=16, num_kv_heads=2)) == (0, 0)


def test_proxy_and_topk_validation():
    p = msa.ProxyArgs()
    p.batch, p.total_q, p.num_qo_heads, p.num_kv_heads = 1, 4, 4, 2
    p.head_dim, p.max_seqlen_q, p.max_k_tiles, p.kv_dtype = 128, 4, 2, 0
    p.q = p.k = p.out = p.cu_seqlens_q = FAKE
    assert msa.lib.msa_proxy_score(ctypes.byref(p), None) == 1  # no cu_seqlens_k
    p.cu_seqlens_k = FAKE
    p.kv_dtype = 2
    assert msa.lib.msa_proxy_score(ctypes.byref(p), None) == 3  # E2M1 proxy K
    p.kv_dtype = 0
    p.page_table, p.seqused_k, p.page_table_width = FAKE, FAKE, 2
    assert msa.lib.msa_proxy_score(ctypes.byref(p), None) == 4  # both lengths
    p.head_dim = 64
    assert msa.lib.msa_proxy_score(ctypes.byref(p), None) == 2
    p.head_dim, p.page_table, p.seqused_k, p.page_table_width = 128, None, None, 0
    p.reduce_heads = 3
    assert msa.lib.msa_proxy_score(ctypes.byref(p), None) == 5  # unknown head reduction
    p.reduce_heads = 0
    f = msa.lib.msa_topk_select
    assert f(FAKE, 2, 64, 8, 0, 2, 0, FAKE, None) == 2          # topk 0
    assert f(FAKE, 3, 64, 8, 4, 2, 0, FAKE, None) == 2          # NONE with 3 != 2 heads
    assert f(FAKE, 3, 64, 8, 4, 2, 2, FAKE, None) == 2          # GROUP 3 % 2
    assert f(FAKE, 2, 20000, 8, 4, 2, 0, FAKE, None) == 5       # too many blocks
    assert f(FAKE, 2, 64, 8, 4, 2, 9, FAKE, None) == 5          # unknown mode
    assert f(FAKE, 2, 64, 0, 4, 2, 0, FAKE, None) == 0          # empty: no launch
    u = msa.lib.msa_tile_union
    assert u(FAKE, FAKE, FAKE, 1, 8, 1, 4, 8, 8, 65, 8, FAKE, FAKE, FAKE, None) == 2
    assert u(FAKE, FAKE, FAKE, 1, 8, 1, 4, 8, 8, 4, 3, FAKE, FAKE, FAKE, None) == 2


def test_validate_attention_host_checks_run_first():
    # the device check is reached only after the host checks pass; these fail
    # before any HIP call
    f = msa.lib.msa_validate_attention
    assert f(None, None) == 1
    a = msa.AttnArgs()
    a.batch, a.total_q, a.num_qo_heads, a.num_kv_heads, a.head_dim, a.topk = 1, 4, 8, 2, 128, 4
    a.max_seqlen_q, a.max_k_tiles = 4, 8
    a.cu_seqlens_k = FAKE
    a.head_dim = 64
    assert f(ctypes.byref(a), None) == 2                  # head_dim
    a.head_dim = 128
    assert f(ctypes.byref(a), None) == 1                  # q, k, v, q2k ... missing
    a.total_q = 0
    assert f(ctypes.byref(a), None) == 0                  # nothing to check


def test_qsa_validation():
    a = msa.QsaArgs()
    a.total_q, a.num_qo_heads, a.num_kv_heads, a.head_dim, a.width = 8, 12, 1, 256, 8
    a.q = a.k = a.v = a.out = a.indices = FAKE
    f = lambda: msa.lib.msa_qsa_indexed_forward(ctypes.byref(a), None)
    a.head_dim = 128
    assert f() == 5                       # head_dim other than 256
    a.head_dim = 256
    a.width = 6
    assert f() == 2                       # width not a multiple of 4
    a.width = 2056
    assert f() == 2                       # wider than 2052
    a.width = 8
    a.num_qo_heads = 24
    assert f() == 5                       # 24 query heads on one KV head
    a.num_qo_heads, a.num_kv_heads = 13, 2
    assert f() == 2                       # Hq not a multiple of Hkv
    a.num_qo_heads, a.num_kv_heads = 12, 1
    a.out = None
    assert f() == 1                       # missing output
    a.total_q = 0
    assert f() == 0                       # nothing to do, nothing launched


def test_qsa_bitmap_validation():
    a = msa.QsaArgs()
    a.total_q, a.num_qo_heads, a.num_kv_heads, a.head_dim = 8, 12, 1, 256
    a.q = a.k = a.v = a.out = FAKE
    a.num_kv_tokens = 100
    f = lambda: msa.lib.msa_qsa_bitmap_forward(ctypes.byref(a), None)
    assert f() == 1                       # no bitmap (width / indices are not needed)
    a.bitmap = FAKE
    a.num_kv_tokens = -1
    assert f() == 2                       # negative Tk
    a.num_kv_tokens = 100
    a.head_dim = 64
    assert f() == 5                       # head_dim other than 256
    a.head_dim = 256
    a.num_qo_heads = 17
    a.num_kv_heads = 1
    assert f() == 5                       # more than 16 query heads per KV head
    a.num_qo_heads = 12
    a.q = FAKE + 4
    assert f() == 5                       # misaligned q
    a.q = FAKE
    a.total_q = 0
    assert f() == 0                       # nothing to do, nothing launched


def test_package_refuses_to_import_without_the_library(tmp_path):
    # no fallback: a copy of the package without libmsa.so fails at import
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "block_sparse_top_msa_amd")
    dst = tmp_path / "block_sparse_top_msa_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    r = subprocess.run([sys.executable, "-c", "import block_sparse_top_msa_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libmsa.so" in r.stderr


def test_nvfp4_decode_preparation_checks_shapes():
    import torch
    q = torch.zeros(4, 16, 128, dtype=torch.bfloat16)
    k = torch.zeros(8, 1, 128, 64, dtype=torch.uint8)
    sc = torch.zeros(8, 1, 128, 8, dtype=torch.uint8)
    q2k = torch.zeros(1, 4, 16, dtype=torch.int32)
    pt = torch.zeros(2, 4, dtype=torch.int32)
    su = torch.full((2,), 300, dtype=torch.int32)
    prep = lambda **kw: msa.prepare_msa_nvfp4_sparse_decode(
        kw.get("q", q), k, k, kw.get("q2k", q2k), k_scale=sc, v_scale=sc, page_table=pt,
        seqused_k=su, k_global_scale=kw.get("kgs", 0.5), v_global_scale=2.0,
        seqlen_q=kw.get("seqlen_q", 2))
    with pytest.raises(ValueError):
        prep(seqlen_q=33)                                   # seqlen_q past 32
    with pytest.raises(ValueError):
        prep(seqlen_q=1)                                    # 4 rows for 2 requests x 1 token
    with pytest.raises(ValueError):
        prep(q2k=torch.zeros(1, 4, 8, dtype=torch.int32))  # topk other than 16
    with pytest.raises(ValueError):
        prep(kgs=0.0)                                       # global scales must be positive
    with pytest.raises(ValueError):
        prep(q=torch.zeros(4, 32, 128, dtype=torch.bfloat16))   # 32 query heads on 1 KV head


def _plan(a):
    route, splits = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = msa.lib.msa_sparse_attention_plan(ctypes.byref(a), ctypes.byref(route),
                                           ctypes.byref(splits))
    return st, route.value, splits.value


@pytest.mark.parametrize("seqlen_q", [1, 4, 8, 32, 64])
@pytest.mark.parametrize("kv_dtype", [0, 1, 2])
def test_g16_short_queries_take_the_decode_route(seqlen_q, kv_dtype):
    # one token's 16 heads fill a row tile: each token of a short query is a
    # decode tile, whatever the format (no bf16 staging of the context)
    a = _attn(batch=128, total_q=128 * seqlen_q, num_qo_heads=16, num_kv_heads=1, topk=16,
              max_seqlen_q=seqlen_q, max_k_tiles=1024, page_table=FAKE, seqused_k=FAKE,
              page_table_width=1024, kv_dtype=kv_dtype)
    a.cu_seqlens_k = None
    if kv_dtype == 2:
        a.k_scale = a.v_scale = FAKE
    st, route, splits = _plan(a)
    assert st == 0 and route == 1 and splits >= 1
    st, n = _size(a)
    # split partials at most: far below the 8.6 GB a staged context would take
    assert st == 0 and n < 64 << 20


def test_long_queries_take_the_prefill_route():
    a = _attn(batch=1, total_q=128, num_qo_heads=16, num_kv_heads=1, topk=16, max_seqlen_q=128,
              max_k_tiles=64)
    assert _plan(a)[:2] == (0, 0)


@pytest.mark.parametrize("seqlen_q,topk,route", [(32, 16, 1), (33, 16, 0), (8, 64, 1), (9, 64, 0)])
def test_short_queries_whose_union_overflows_take_the_prefill_route(seqlen_q, topk, route):
    # G = 1: seqlen_q rows fit one decode tile, but seqlen_q x topk selections
    # must also fit its 512-entry union; past that the prefill tiles take them
    a = _attn(batch=2, total_q=2 * seqlen_q, num_qo_heads=2, num_kv_heads=2, topk=topk,
              max_seqlen_q=seqlen_q, max_k_tiles=64)
    st, r, _ = _plan(a)
    assert st == 0 and r == route
    assert _size(a)[0] == 0


@pytest.mark.parametrize("hq,hkv,temp", [(512, 1, False), (512, 1, True), (1024, 2, False)])
def test_group_larger_than_a_tile_is_rejected(hq, hkv, temp):
    kw = dict(num_qo_heads=hq, num_kv_heads=hkv, total_q=64, max_seqlen_q=32)
    if temp:
        kw.update(lse_t=FAKE, lse_temperature_scale=1.0)
    st, msg = _call(_attn(**kw))
    assert st == 2 and "prefill tile" in msg


def test_flat_e2m1_decode_stages_only_selected_blocks():
    # one token per request, flat E2M1: the workspace holds the selected
    # blocks (at most topk per request and KV head), not every visible block
    a = _attn(batch=64, total_q=64, num_qo_heads=16, num_kv_heads=1, topk=16, max_seqlen_q=1,
              max_k_tiles=1024, kv_dtype=2, k_scale=FAKE, v_scale=FAKE)
    st, route, splits = _plan(a)
    assert (st, route, splits) == (0, 0, 1)
    st, n = _size(a)
    page = 2 * 128 * 256                  # K and V, 128 rows of 256 bytes
    assert st == 0 and 64 * 16 * page <= n < 64 * 16 * page + (1 << 20)
    # long queries stage every visible block
    b = _attn(batch=2, total_q=4096, num_qo_heads=16, num_kv_heads=1, topk=16,
              max_seqlen_q=2048, max_k_tiles=16, kv_dtype=2, k_scale=FAKE, v_scale=FAKE)
    st, n = _size(b)
    assert st == 0 and 2 * 16 * page <= n < 2 * 16 * page + (1 << 20)


def test_noalloc_rejects_workspace_beyond_its_scratch():
    # fp8 prefill over 64 requests x 1024 blocks stages GBs: declined before
    # any device call, naming the limit
    a = _attn(batch=64, total_q=64 * 1024, num_qo_heads=16, num_kv_heads=2, topk=16,
              max_seqlen_q=1024, max_k_tiles=1024, kv_dtype=1)
    st = msa.lib.msa_sparse_attention_noalloc(ctypes.byref(a), None)
    msg = msa.lib.msa_last_error().decode()
    assert st == 6 and "33554432" in msg


def test_q_offset_modes_are_checked_on_the_host():
    st, msg = _call(_attn(q_offset_mode=3, causal=1))
    assert st == 5 and "q_offset_mode" in msg
    st, msg = _call(_attn(q_offset_mode=1, q_offset_value=(1 << 30) + 1, causal=1))
    assert st == 2 and "q_offset_value" in msg
    st, msg = _call(_attn(q_offset_mode=2, causal=1))          # no tensor
    assert st == 1 and "q_offset" in msg
    p = msa.ProxyArgs()
    p.batch, p.total_q, p.num_qo_heads, p.num_kv_heads = 1, 4, 4, 2
    p.head_dim, p.max_seqlen_q, p.max_k_tiles, p.kv_dtype = 128, 4, 2, 0
    p.q = p.k = p.out = p.cu_seqlens_q = p.cu_seqlens_k = FAKE
    p.q_offset_mode = 2
    assert msa.lib.msa_proxy_score(ctypes.byref(p), None) == 1


def test_proxy_topk_host_checks():
    p = msa.ProxyArgs()
    p.batch, p.total_q, p.num_qo_heads, p.num_kv_heads = 2, 8, 32, 2
    p.head_dim, p.max_seqlen_q, p.max_k_tiles, p.kv_dtype = 128, 4, 64, 1
    p.q = p.k = p.cu_seqlens_q = p.page_table = p.seqused_k = FAKE
    p.page_table_width, p.reduce_heads = 64, 1
    n = ctypes.c_size_t(0)
    assert msa.lib.msa_proxy_topk_workspace_size(ctypes.byref(p), 0, ctypes.byref(n)) == 2
    assert msa.lib.msa_proxy_topk_workspace_size(ctypes.byref(p), 16, ctypes.byref(n)) == 0
    # candidates: one shared selection x 8 queries x 2 KV heads x chunks x 16, score + id
    assert n.value >= 2 * 8 * 2 * 16 * 4
    assert msa.lib.msa_proxy_topk(ctypes.byref(p), 16, FAKE, None, 0, None) == 6
    assert msa.lib.msa_proxy_topk(ctypes.byref(p), 16, None, FAKE, n.value, None) == 1
    assert msa.lib.msa_proxy_topk(ctypes.byref(p), 16, FAKE, FAKE + 8, n.value, None) == 6
