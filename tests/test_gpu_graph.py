"""Decode steps captured as one HIP graph (block_sparse_top_msa_amd.graph):
every replay equals the eager step on the same inputs, bit for bit, with the
program's own eager work and synchronisations between replays and new
queries written into the bound tensors in place."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _graph(msa, p, **kw):
    from block_sparse_top_msa_amd.graph import DecodeGraph
    return DecodeGraph(p.q, p.k, p.v, p.cu_seqlens_q, max_seqlen_q=max(p.q_lens),
                       max_k_tiles=p.max_k_tiles, topk=p.topk, page_table=p.page_table,
                       seqused_k=p.seqused_k, cu_seqlens_k=p.cu_seqlens_k, k_scale=p.k_scale,
                       v_scale=p.v_scale, k_global_scale=p.k_global_scale,
                       v_global_scale=p.v_global_scale, **kw)


def _replays_match_eager(g, q_new, rounds=3):
    gen = torch.Generator(device="cuda").manual_seed(11)
    for r in range(rounds):
        # next step's queries, written in place; eager work and a sync between
        g.q.copy_(torch.randn(g.q.shape, generator=gen, device="cuda").to(g.q.dtype)
                  if q_new else g.q)
        torch.cuda.synchronize()
        out, lse = g.replay()
        got_out, got_lse = out.clone(), lse.clone()
        got_q2k = g.q2k.clone()
        torch.cuda.synchronize()
        ref_out, ref_lse = g.step()
        torch.cuda.synchronize()
        assert torch.equal(got_q2k, g.q2k), f"replay {r}: q2k"
        assert torch.equal(got_out, ref_out), f"replay {r}: out"
        assert torch.equal(got_lse, ref_lse), f"replay {r}: lse"


def test_fp8_mtp_pipeline_graph(msa):
    # proxy (fp8 K, reduce_heads) -> top-K -> attention, 4 tokens per request
    print("graph: fp8 MTP pipeline", flush=True)
    p = synth.make_problem("graph_mtp", q_lens=[4] * 5, k_lens=[9000, 130, 4000, 20000, 700],
                           num_qo_heads=32, num_kv_heads=2, topk=16, paged=True,
                           kv_dtype=synth.KV_FP8, seed=51, selection="proxy",
                           reduce_heads=True).to("cuda")
    g = _graph(msa, p, reduce_heads=True)
    _replays_match_eager(g, q_new=True)
    # the captured selection (proxy and top-K in one call) equals the proxy
    # scores followed by the separate select
    scores = msa.proxy_score(g.q, p.k, p.cu_seqlens_q, page_table=p.page_table,
                             seqused_k=p.seqused_k, causal=True, max_seqlen_q=max(p.q_lens),
                             max_k_tiles=p.max_k_tiles, reduce_heads=True)
    ref = msa.topk_select(scores, p.topk, p.num_kv_heads)
    torch.cuda.synchronize()
    assert torch.equal(g.q2k, ref)


@pytest.mark.parametrize("fmt,splits", [(synth.KV_BF16, 0), (synth.KV_E2M1, 3)])
def test_decode_graph_with_given_selection(msa, fmt, splits):
    print(f"graph: decode {fmt} splits {splits}", flush=True)
    kw = dict(k_global_scale=0.5, v_global_scale=2.0) if fmt == synth.KV_E2M1 else {}
    p = synth.make_problem("graph_dec", q_lens=[1] * 6, k_lens=[3000, 129, 7000, 900, 5000, 64],
                           num_qo_heads=16, num_kv_heads=1 if fmt == synth.KV_E2M1 else 2,
                           topk=8, paged=True, kv_dtype=fmt, seed=52, selection="decode",
                           **kw).to("cuda")
    g = _graph(msa, p, q2k=p.q2k, splits=splits)
    if splits > 1:
        assert g.workspace is not None          # split partials bound before capture
    _replays_match_eager(g, q_new=True)


@pytest.mark.parametrize("seqlen_q,given_ws", [(1, False), (4, True), (8, False), (32, True)])
def test_nvfp4_decode_runner(msa, seqlen_q, given_ws):
    # prepare once, call: equals the plain call bitwise and the oracle within
    # tolerance; a captured call replays the same result
    import oracle
    from gpu_helpers import assert_attention_close, gpu_attention
    print(f"nvfp4 runner seqlen_q {seqlen_q} workspace given {given_ws}", flush=True)
    p = synth.make_problem("nvfp4_runner", q_lens=[seqlen_q] * 3, k_lens=[5000, 700, 2600],
                           num_qo_heads=16, num_kv_heads=1, topk=16, paged=True,
                           kv_dtype=synth.KV_E2M1, seed=70 + seqlen_q, selection="decode",
                           k_global_scale=0.5, v_global_scale=2.0).to("cuda")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda") if given_ws else None
    run = msa.prepare_msa_nvfp4_sparse_decode(
        p.q, p.k, p.v, p.q2k, k_scale=p.k_scale, v_scale=p.v_scale, page_table=p.page_table,
        seqused_k=p.seqused_k, k_global_scale=0.5, v_global_scale=2.0, workspace_buffer=ws,
        seqlen_q=seqlen_q)
    assert run.splits >= 1
    # one token's 16 heads fill a row tile: every seqlen_q in the runner's
    # envelope takes the decode kernel (in-register E2M1, no staged context)
    assert run.decode_route == 1
    out = run().clone()
    lse = run.lse.clone()
    ref = gpu_attention(msa, p)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
    ref_out, ref_lse = oracle.sparse_attention(
        p.q, p.k, p.v, p.q2k.cpu(), p.cu_seqlens_q.cpu(), page_table=p.page_table.cpu(),
        seqused_k=p.seqused_k.cpu(), causal=True, kv_format=p.kv_dtype, k_scale=p.k_scale,
        v_scale=p.v_scale, k_global_scale=0.5, v_global_scale=2.0)
    assert_attention_close(out, lse, ref_out, ref_lse, "nvfp4 runner")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(3):
        run.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.out, out) and torch.equal(run.lse, lse)
