"""The allocation-free attention entry point (msa_sparse_attention_noalloc)
against msa_sparse_attention with a caller workspace (GPU).

Both launch the same kernels; the no-alloc call keeps its split-KV partials,
or its staged bf16 pages, in the library's per-GPU scratch array.  Two calls
in a row, the second smaller, each bitwise equal to the workspace call and
within the oracle's tolerance.
"""
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_attention_close, oracle_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _both(msa, p, splits):
    d = p.to("cuda")
    mq, T = max(p.q_lens), p.max_k_tiles
    kw = dict(causal=p.causal, softmax_scale=p.softmax_scale, page_table=d.page_table,
              seqused_k=d.seqused_k, k_scale=d.k_scale, v_scale=d.v_scale,
              k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale)
    route, nsplit = msa.attention_plan(d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k,
                                       page_table=d.page_table, seqused_k=d.seqused_k,
                                       k_scale=d.k_scale, v_scale=d.v_scale, max_seqlen_q=mq,
                                       max_k_tiles=T, splits=splits)
    need = msa.workspace_size(d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k,
                              page_table=d.page_table, seqused_k=d.seqused_k, k_scale=d.k_scale,
                              v_scale=d.v_scale, max_seqlen_q=mq, max_k_tiles=T, splits=splits)
    assert need > 0, "the case must use the scratch"
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full((p.total_q, p.num_qo_heads), float("nan"), device="cuda")
    msa.sparse_attention_noalloc(d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k,
                                 max_seqlen_q=mq, max_k_tiles=T, out=out, lse=lse, splits=splits,
                                 **kw)
    ref, ref_lse = msa.sparse_attention(d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k,
                                        return_softmax_lse=True, max_seqlen_q=mq, max_k_tiles=T,
                                        splits=splits, **kw)
    torch.cuda.synchronize()
    return out, lse, ref, ref_lse, route, nsplit


def test_noalloc_split_decode_twice(msa):
    # paged E2M1 decode with forced split-KV partials: a large call, then a
    # smaller one reusing the same scratch
    for i, (b, lo, hi) in enumerate(((40, 2000, 40000), (5, 130, 3000))):
        print(f"no-alloc split decode call {i}: batch {b}", flush=True)
        g = torch.Generator().manual_seed(90 + i)
        k_lens = torch.randint(lo, hi, (b,), generator=g).tolist()
        p = synth.make_problem("noalloc_dec", q_lens=[1] * b, k_lens=k_lens, num_qo_heads=16,
                               num_kv_heads=1, topk=16, paged=True, kv_dtype=synth.KV_E2M1,
                               seed=90 + i, selection="decode", k_global_scale=0.5,
                               v_global_scale=2.0)
        out, lse, ref, ref_lse, route, nsplit = _both(msa, p, splits=3)
        assert route == 1 and nsplit == 3
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
        ro, rl = oracle_attention(p)
        assert_attention_close(out, lse, ro, rl, f"no-alloc decode call {i}")


def test_noalloc_staged_fp8_prefill_twice(msa):
    # fp8 prefill: the visible blocks are staged to bf16 pages in the scratch
    # (700 x 2 x 3 q2k entries: every visible block is staged; 70 x 2 x 3:
    # only the selected blocks)
    for i, (ql, kl) in enumerate((([700, 200, 129], [900, 300, 129]), ([70], [260]))):
        print(f"no-alloc fp8 prefill call {i}", flush=True)
        p = synth.make_problem("noalloc_fp8", q_lens=ql, k_lens=kl, num_qo_heads=8,
                               num_kv_heads=2, topk=3, kv_dtype=synth.KV_FP8, seed=95 + i,
                               selection="general")
        out, lse, ref, ref_lse, route, _ = _both(msa, p, splits=0)
        assert route == 0
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
        ro, rl = oracle_attention(p)
        assert_attention_close(out, lse, ro, rl, f"no-alloc fp8 prefill call {i}")
