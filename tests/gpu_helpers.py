"""Shared helpers for the GPU parity tests: run the HIP path through the
Python binding, run the oracle on the same inputs, compare to the stated
tolerances.

Tolerances (fp64 oracle vs the HIP path):
  out   bf16, max |delta| <= 2e-2; rows with no attended key exactly 0
  lse   |delta| <= 1e-3 where finite; -inf exactly where the oracle has -inf
  proxy |delta| <= 1e-3 * max(1, |ref|); identical -inf pattern
  top-K bit-exact against the oracle's selection on the GPU's own fp32 scores
"""
import math

import torch

import oracle

OUT_TOL = 2e-2
LSE_TOL = 1e-3
PROXY_RTOL = 1e-3


def gpu_attention(msa, p, q2k=None, splits=0, lse=True, workspace=None):
    q2k = p.q2k if q2k is None else q2k
    return msa.sparse_attention(
        p.q, p.k, p.v, q2k, p.cu_seqlens_q, p.cu_seqlens_k, causal=p.causal,
        softmax_scale=p.softmax_scale, page_table=p.page_table, seqused_k=p.seqused_k,
        return_softmax_lse=lse, k_scale=p.k_scale, v_scale=p.v_scale,
        k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale,
        max_seqlen_q=max(p.q_lens), max_k_tiles=p.max_k_tiles, splits=splits,
        workspace=workspace)


def oracle_attention(p, q2k=None, rows=None):
    q2k = p.q2k if q2k is None else q2k
    return oracle.sparse_attention(
        p.q, p.k, p.v, q2k.cpu(), p.cu_seqlens_q.cpu(),
        cu_seqlens_k=None if p.cu_seqlens_k is None else p.cu_seqlens_k.cpu(),
        page_table=None if p.page_table is None else p.page_table.cpu(),
        seqused_k=None if p.seqused_k is None else p.seqused_k.cpu(),
        causal=p.causal, softmax_scale=p.softmax_scale, kv_format=p.kv_dtype,
        k_scale=p.k_scale, v_scale=p.v_scale, k_global_scale=p.k_global_scale,
        v_global_scale=p.v_global_scale, rows=rows)


def assert_attention_close(out, lse, ref_out, ref_lse, what=""):
    out = out.float().cpu().double()
    ref_lse = ref_lse.double()
    empty = torch.isneginf(ref_lse)
    d = (out - ref_out).abs()
    worst = float(d.max()) if d.numel() else 0.0
    assert worst <= OUT_TOL, f"{what}: max |out - ref| = {worst:.4g} > {OUT_TOL}"
    if empty.any():
        assert (out[empty] == 0).all(), f"{what}: rows with no attended key must be exactly 0"
    if lse is not None:
        lse = lse.double().cpu()
        assert torch.equal(torch.isneginf(lse), empty), f"{what}: -inf LSE pattern differs"
        fin = ~empty
        if fin.any():
            e = float((lse[fin] - ref_lse[fin]).abs().max())
            assert e <= LSE_TOL, f"{what}: max |lse - ref| = {e:.4g} > {LSE_TOL}"
    return worst


def assert_proxy_close(got, ref, what=""):
    got = got.double().cpu()
    ref = ref.double()
    assert got.shape == ref.shape, (got.shape, ref.shape)
    ninf_g, ninf_r = torch.isneginf(got), torch.isneginf(ref)
    assert torch.equal(ninf_g, ninf_r), f"{what}: -inf pattern differs ({int((ninf_g != ninf_r).sum())} entries)"
    fin = ~ninf_r
    if fin.any():
        err = ((got[fin] - ref[fin]).abs() / ref[fin].abs().clamp(min=1.0)).max()
        assert float(err) <= PROXY_RTOL, f"{what}: proxy relative error {float(err):.3g}"


def device():
    return torch.device("cuda", 0)
