"""The five synthetic workloads at full size, in the launch configuration
the benchmark times (GPU).

Inputs are generated on the GPU (seeded).  Every query row of every
workload is checked: selection indices bit-exactly (the oracle's top-K on the
GPU's own fp32 scores), proxy scores and attention outputs against the fp64
oracle to the stated tolerances.
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
    # proxy and attention: every query row
    pc = p.to("cpu")
    ref_s = oracle.proxy_score(pc.proxy_q, pc.k, pc.cu_seqlens_q, cu_seqlens_k=pc.cu_seqlens_k,
                               causal=True, max_k_tiles=T)
    assert_proxy_close(s_cpu, ref_s, "pipeline proxy")
    ref_out, ref_lse = oracle_attention(pc, q2k=q2k.cpu())
    assert_attention_close(out, lse, ref_out, ref_lse, "pipeline attention")
    # information only: rows whose fp64-score selection differs
    ref_sel = oracle.topk_select(ref_s, p.topk, p.num_kv_heads)
    diff = int((ref_sel != q2k.cpu()).any(-1).sum())
    print(f"rows whose fp64-score selection differs: {diff} of {q2k.shape[0] * q2k.shape[1]}",
          flush=True)


@pytest.mark.parametrize("idx", [2, 4])
def test_workload_paged_decode(msa, idx):
    p = synth.workload(synth.WORKLOADS[idx], device="cuda")
    print("workload", p.name, flush=True)
    out, lse = gpu_attention(msa, p)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_attention(p)          # every row
    assert_attention_close(out, lse, ref_out, ref_lse, p.name)


@pytest.fixture(scope="module")
def mtp(msa):
    """The fp8 MTP decode pipeline, run once: proxy (reduce_heads) -> top-K ->
    attention, results copied to the host."""
    p = synth.workload(synth.WORKLOADS[3], device="cuda")
    print("workload", p.name, flush=True)
    T = p.max_k_tiles
    scores = msa.proxy_score(p.q, p.k, p.cu_seqlens_q, page_table=p.page_table,
                             seqused_k=p.seqused_k, causal=True, max_seqlen_q=4,
                             max_k_tiles=T, reduce_heads=True)
    q2k = msa.topk_select(scores, p.topk, p.num_kv_heads)
    out, lse = gpu_attention(msa, p, q2k=q2k)
    torch.cuda.synchronize()
    return p, scores.cpu(), q2k.cpu(), out.cpu(), lse.cpu()


def test_workload_paged_fp8_mtp_pipeline(mtp):
    p, s_cpu, q2k, out, lse = mtp
    assert torch.equal(q2k, oracle.topk_select(s_cpu, p.topk, p.num_kv_heads))
    assert torch.equal(q2k[0], q2k[1])  # one shared selection per query
    ref_out, ref_lse = oracle_attention(p, q2k=q2k)   # every row
    assert_attention_close(out, lse, ref_out, ref_lse, "mtp attention")


@pytest.mark.parametrize("part", range(4))
def test_workload_paged_fp8_mtp_proxy(mtp, part):
    # every row of the head-reduced fp8 proxy, in four parts of 8 requests
    # (each part is ~25 GFLOP of fp64 oracle work)
    p, s_cpu, _, _, _ = mtp
    rows = list(range(32 * part, 32 * part + 32))
    print(f"mtp proxy rows {rows[0]}..{rows[-1]}", flush=True)
    ref_s = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, page_table=p.page_table,
                               seqused_k=p.seqused_k, causal=True, max_k_tiles=p.max_k_tiles,
                               reduce_heads=True, kv_format=synth.KV_FP8, rows=rows)
    assert_proxy_close(s_cpu[:, :, rows], ref_s[:, :, rows], "mtp proxy")
