"""The five synthetic workloads at full size, in the launch configuration
the benchmark times (GPU).

Inputs are generated on the GPU (seeded).  Every selection index is checked
bit-exactly (the oracle's top-K on the GPU's own fp32 scores, all rows);
proxy scores and attention outputs are checked on sampled query rows that the
oracle evaluates one by one: random rows plus the first and last row of each
request (ragged tails, the diagonal block).
"""
import pytest
import torch

import oracle
import synth
from gpu_helpers import (assert_attention_close, assert_proxy_close, gpu_attention,
                         oracle_attention)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _sample_rows(p, n, seed):
    g = torch.Generator().manual_seed(seed)
    cu = p.cu_seqlens_q.cpu().tolist()
    rows = set(int(x) for x in torch.randint(0, p.total_q, (n,), generator=g))
    for b in range(len(cu) - 1):
        rows.update({cu[b], cu[b + 1] - 1})
    return sorted(rows)


def _cpu(t):
    return None if t is None else t.cpu()


def test_workload_flat_prefill_tiny(msa):
    p = synth.workload(synth.WORKLOADS[0], device="cuda")
    print("workload", p.name, flush=True)
    out, lse = gpu_attention(msa, p)
    ref_out, ref_lse = oracle_attention(p.to("cpu"))
    assert_attention_close(out, lse, ref_out, ref_lse, p.name)


def test_workload_flat_prefill_pipeline(msa):
    p = synth.workload(synth.WORKLOADS[1], device="cuda")
    print("workload", p.name, flush=True)
    T = p.max_k_tiles
    scores = msa.proxy_score(p.proxy_q, p.k, p.cu_seqlens_q, p.cu_seqlens_k, causal=True,
                             max_seqlen_q=8192, max_k_tiles=T)
    q2k = msa.topk_select(scores, p.topk, p.num_kv_heads)
    out, lse = gpu_attention(msa, p, q2k=q2k)
    torch.cuda.synchronize()
    # top-K: every row, bit-exact on the GPU's own scores
    s_cpu = scores.cpu()
    assert torch.equal(q2k.cpu(), oracle.topk_select(s_cpu, p.topk, p.num_kv_heads))
    rows = _sample_rows(p, 48, seed=1)
    pc = p.to("cpu")
    ref_s = oracle.proxy_score(pc.proxy_q, pc.k, pc.cu_seqlens_q, cu_seqlens_k=pc.cu_seqlens_k,
                               causal=True, max_k_tiles=T, rows=rows)
    assert_proxy_close(s_cpu[:, :, rows], ref_s[:, :, rows], "pipeline proxy")
    ref_out, ref_lse = oracle_attention(pc, q2k=q2k.cpu(), rows=rows)
    assert_attention_close(out[rows], lse[rows], ref_out, ref_lse, "pipeline attention")
    # information only: rows whose fp64-score selection differs
    ref_sel = oracle.topk_select(ref_s[:, :, rows], p.topk, p.num_kv_heads)
    diff = int((ref_sel != q2k.cpu()[:, rows]).any(-1).sum())
    print(f"rows whose fp64-score selection differs: {diff} of {2 * len(rows)}", flush=True)


@pytest.mark.parametrize("idx", [2, 4])
def test_workload_paged_decode(msa, idx):
    p = synth.workload(synth.WORKLOADS[idx], device="cuda")
    print("workload", p.name, flush=True)
    out, lse = gpu_attention(msa, p)
    torch.cuda.synchronize()
    rows = _sample_rows(p, 24, seed=idx)
    ref_out, ref_lse = oracle_attention(p, rows=rows)
    assert_attention_close(out[rows], lse[rows], ref_out, ref_lse, p.name)


def test_workload_paged_fp8_mtp_pipeline(msa):
    p = synth.workload(synth.WORKLOADS[3], device="cuda")
    print("workload", p.name, flush=True)
    T = p.max_k_tiles
    scores = msa.proxy_score(p.q, p.k, p.cu_seqlens_q, page_table=p.page_table,
                             seqused_k=p.seqused_k, causal=True, max_seqlen_q=4,
                             max_k_tiles=T, reduce_heads=True)
    q2k = msa.topk_select(scores, p.topk, p.num_kv_heads)
    out, lse = gpu_attention(msa, p, q2k=q2k)
    torch.cuda.synchronize()
    s_cpu = scores.cpu()
    assert torch.equal(q2k.cpu(), oracle.topk_select(s_cpu, p.topk, p.num_kv_heads))
    assert torch.equal(q2k[0], q2k[1])  # one shared selection per query
    # proxy and attention on every token of three sampled requests
    reqs = [0, 13, 31]
    rows = [4 * b + t for b in reqs for t in range(4)]
    ref_s = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, page_table=p.page_table,
                               seqused_k=p.seqused_k, causal=True, max_k_tiles=T,
                               reduce_heads=True, kv_format=synth.KV_FP8, rows=rows)
    assert_proxy_close(s_cpu[:, :, rows], ref_s[:, :, rows], "mtp proxy")
    ref_out, ref_lse = oracle_attention(p, q2k=q2k, rows=rows)
    assert_attention_close(out[rows], lse[rows], ref_out, ref_lse, "mtp attention")
