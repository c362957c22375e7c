"""Edge cases of the HIP path against the fp64 oracle (GPU).

Largest top-K, the widest GQA group, requests with no queries or no keys
(and multi-token decode against fewer keys than queries),
a million-token paged context (page ids past the LDS read-ahead), the flat
layout on the decode-shaped kernel, non-causal multi-token decode and empty
batches.  Every call goes through the C ABI (via the ctypes binding).
"""
import pytest
import torch

import synth
from gpu_helpers import assert_attention_close, gpu_attention, oracle_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _check(msa, p, what):
    print(what, flush=True)
    out, lse = gpu_attention(msa, p.to("cuda"))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, what)
    return out, lse


def test_topk_64_prefill_and_decode(msa):
    p = synth.make_problem("topk64_prefill", q_lens=[200, 70], k_lens=[9000, 700], num_qo_heads=8,
                           num_kv_heads=1, topk=64, seed=31, selection="general")
    _check(msa, p, "topk 64 prefill")
    d = synth.make_problem("topk64_decode", q_lens=[1] * 3, k_lens=[9000, 20000, 300],
                           num_qo_heads=16, num_kv_heads=1, topk=64, paged=True, seed=32,
                           selection="decode")
    _check(msa, d, "topk 64 decode")


def test_group_64(msa):
    p = synth.make_problem("g64_prefill", q_lens=[37, 9], k_lens=[400, 130], num_qo_heads=64,
                           num_kv_heads=1, topk=3, seed=33, selection="general")
    _check(msa, p, "G 64 prefill")
    d = synth.make_problem("g64_decode", q_lens=[1] * 4, k_lens=[3000, 129, 700, 5000],
                           num_qo_heads=64, num_kv_heads=1, topk=8, paged=True, seed=34,
                           selection="decode", kv_dtype=synth.KV_FP8)
    _check(msa, d, "G 64 fp8 decode")


def test_requests_without_queries_or_keys(msa):
    # request 0 has no keys (every row empty: 0 / -inf); request 1 no queries
    p = synth.make_problem("zero_len", q_lens=[40, 0, 25], k_lens=[0, 300, 260], num_qo_heads=4,
                           num_kv_heads=2, topk=3, seed=35, selection="general")
    out, lse = _check(msa, p, "zero-length requests")
    assert (out[:40].float() == 0).all() and torch.isneginf(lse[:40]).all()


def test_million_token_paged_context(msa):
    # 7813 pages: more blocks than the decode kernel reads ahead into LDS
    d = synth.make_problem("long_ctx", q_lens=[1, 1], k_lens=[1_000_000, 150_000], num_qo_heads=16,
                           num_kv_heads=1, topk=16, paged=True, seed=36, selection="decode")
    _check(msa, d, "1M-token context decode")


def test_flat_layout_on_decode_kernel(msa):
    # seqlen_q x G <= 64 on the flat layout takes the decode-shaped kernel
    p = synth.make_problem("flat_decode", q_lens=[3, 5], k_lens=[700, 300], num_qo_heads=8,
                           num_kv_heads=1, topk=4, seed=37, selection="general")
    _check(msa, p, "flat decode-shaped")


def test_non_causal_multi_token_decode(msa):
    d = synth.make_problem("nc_decode", q_lens=[4] * 3, k_lens=[1000, 2000, 129], num_qo_heads=16,
                           num_kv_heads=1, topk=8, paged=True, causal=False, seed=38,
                           selection="decode")
    _check(msa, d, "non-causal MTP decode")


def test_empty_batches(msa):
    q = torch.empty(0, 8, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(0, 1, 128, dtype=torch.bfloat16, device="cuda")
    q2k = torch.empty(1, 0, 4, dtype=torch.int32, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = msa.sparse_attention(q, k, k, q2k, cu, cu, causal=True, return_softmax_lse=True,
                                    max_seqlen_q=0, max_k_tiles=0)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 128) and lse.shape == (0, 8)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8, synth.KV_E2M1])
def test_mtp_decode_with_fewer_keys_than_queries(msa, fmt):
    # 4 query tokens against 2, 3 and 0 keys: the leading tokens see no key
    # (0 / -inf), the rest a partial first page
    kw = dict(k_global_scale=0.5, v_global_scale=2.0) if fmt == synth.KV_E2M1 else {}
    d = synth.make_problem("short_kv_decode", q_lens=[4] * 4, k_lens=[2, 3, 0, 1000],
                           num_qo_heads=16, num_kv_heads=1, topk=4, paged=True, kv_dtype=fmt,
                           seed=39, selection="decode", **kw)
    out, lse = _check(msa, d, f"MTP decode with short KV, {fmt}")
    assert (out[:2].float() == 0).all() and torch.isneginf(lse[:2]).all()
    assert (out[8:12].float() == 0).all() and torch.isneginf(lse[8:12]).all()
