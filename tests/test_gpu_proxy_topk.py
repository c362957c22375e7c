"""msa_proxy_topk: proxy score -> head reduction -> top-K in one call (GPU).

On decode shapes the selection runs inside the proxy pass (per-chunk top-K
candidates, merged by block id); it must equal the two-call path
(msa_proxy_score then msa_topk_select) bit for bit, and the oracle's top-K on
the GPU's own fp32 scores, including exact ties.
"""
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _both(msa, d, topk, reduce, mq, T, q_offset=None):
    kw = dict(page_table=d.page_table, seqused_k=d.seqused_k, causal=True, max_seqlen_q=mq,
              max_k_tiles=T, reduce_heads=reduce, q_offset=q_offset)
    fused = msa.proxy_topk(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, topk=topk, **kw)
    scores = msa.proxy_score(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, **kw)
    two = msa.topk_select(scores, topk, d.k.shape[1])
    torch.cuda.synchronize()
    return fused.cpu(), two.cpu(), scores.cpu()


CASES = [
    # q_lens, k_lens, Hq, Hkv, fmt, paged, reduce, topk
    ([4, 4, 4], [9000, 600, 3000], 32, 2, synth.KV_FP8, True, True, 16),
    ([4, 4], [20000, 700], 16, 2, synth.KV_BF16, True, "group", 16),
    ([2, 2, 2], [5000, 129, 3000], 8, 2, synth.KV_BF16, True, False, 8),
    ([1, 1, 1, 1], [7000, 300, 128, 1], 16, 1, synth.KV_FP8, True, True, 48),
    ([3], [4000], 4, 1, synth.KV_F16, False, False, 64),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_select_matches_two_calls_and_oracle(msa, case):
    ql, kl, hq, hkv, fmt, paged, reduce, topk = CASES[case]
    print(f"proxy_topk case {case}", flush=True)
    p = synth.make_problem("ptk", q_lens=ql, k_lens=kl, num_qo_heads=hq, num_kv_heads=hkv,
                           topk=4, paged=paged, kv_dtype=fmt, seed=150 + case,
                           selection="general")
    d = p.to("cuda")
    fused, two, scores = _both(msa, d, topk, reduce, max(ql), p.max_k_tiles)
    assert torch.equal(fused, two)
    assert torch.equal(fused, oracle.topk_select(scores, topk, hkv))


def test_fused_select_exact_ties(msa):
    # every page holds the same keys: all blocks of a request score the same
    # (the partial last block too when it is full), so ties go to the lowest
    # block ids across chunks and KV heads
    print("proxy_topk ties", flush=True)
    p = synth.make_problem("ptk_tie", q_lens=[4, 4], k_lens=[128 * 70, 128 * 33 + 5],
                           num_qo_heads=32, num_kv_heads=2, topk=4, paged=True,
                           kv_dtype=synth.KV_FP8, seed=160, selection="general")
    p.k[:] = p.k[0:1].clone()
    d = p.to("cuda")
    for reduce in (True, "group"):
        fused, two, scores = _both(msa, d, 16, reduce, 4, p.max_k_tiles)
        assert torch.equal(fused, two)
        assert torch.equal(fused, oracle.topk_select(scores, 16, 2))


def test_fused_select_with_q_offset(msa):
    print("proxy_topk q_offset", flush=True)
    p = synth.make_problem("ptk_qo", q_lens=[4, 4, 4], k_lens=[6000, 3000, 900],
                           num_qo_heads=32, num_kv_heads=2, topk=4, paged=True,
                           kv_dtype=synth.KV_FP8, seed=161, selection="general")
    d = p.to("cuda")
    g = torch.Generator().manual_seed(4)
    qo = torch.randint(-50, 6100, (12,), generator=g, dtype=torch.int32).cuda()
    fused, two, scores = _both(msa, d, 16, True, 4, p.max_k_tiles, q_offset=qo)
    assert torch.equal(fused, two)
    assert torch.equal(fused, oracle.topk_select(scores, 16, 2))


def test_prefill_shapes_go_through_the_score_buffer(msa):
    print("proxy_topk prefill shape", flush=True)
    p = synth.make_problem("ptk_pf", q_lens=[300, 129], k_lens=[700, 400], num_qo_heads=2,
                           num_kv_heads=2, topk=4, seed=162, selection="general")
    d = p.to("cuda")
    fused, two, _ = _both(msa, d, 4, False, 300, p.max_k_tiles)
    assert torch.equal(fused, two)


def test_mtp_workload_fused_equals_two_calls(msa):
    p = synth.workload(synth.WORKLOADS[3], device="cuda")
    print("workload", p.name, flush=True)
    fused, two, _ = _both(msa, p, p.topk, True, 4, p.max_k_tiles)
    assert torch.equal(fused, two)
