"""A decode step bound to its tensors once and replayed as one HIP graph.

Serving loops run the same decode shapes every step; capturing the step
(optionally proxy score -> top-K select -> sparse attention, the MSA decode
pipeline of the msa_proxy_score and msa_sparse_attention pages) removes the
per-launch host work and gaps.  The library never allocates, never
synchronises and clears nothing with memset (its fills are kernels), so the
step captures as it is: this module only binds the buffers (outputs, q2k,
the proxy/top-K and split-KV workspaces) before capture and passes
every size explicitly, so that no call inside the graph reads a device
value on the host.

Replays read the bound tensors' current contents: write the next step's
queries (and, without the proxy, its q2k rows) into them in place.  Two
graphs that may run at the same time need their own workspaces, which each
DecodeGraph holds.
"""
from __future__ import annotations

import torch

from . import (Workspace, proxy_topk, proxy_topk_workspace_size, sparse_attention,
               workspace_size)


class DecodeGraph:
    """Capture of one decode step on the current device.

    With `q2k` given, the step is the sparse attention over those rows; with
    `q2k=None` it first scores every block with the proxy pass (`proxy_q`,
    default `q`, against `k`; `reduce_heads` as in proxy_score) and selects
    the top-`topk` blocks into `self.q2k` in the same call (proxy_topk: on
    decode shapes the selection runs inside the proxy pass).  `max_seqlen_q`
    and `max_k_tiles` are required (no host reads of device lengths).
    `replay()` returns (out, lse); lse is None unless `return_lse`."""

    def __init__(self, q, k, v, cu_seqlens_q, *, max_seqlen_q, max_k_tiles, topk,
                 page_table=None, seqused_k=None, cu_seqlens_k=None, q2k=None, proxy_q=None,
                 reduce_heads=True, k_scale=None, v_scale=None, k_global_scale=None,
                 v_global_scale=None, softmax_scale=None, causal=True, return_lse=True,
                 splits=0, warmup=2):
        self.q, self.k, self.v = q, k, v
        self.cu_seqlens_q, self.cu_seqlens_k = cu_seqlens_q, cu_seqlens_k
        self.page_table, self.seqused_k = page_table, seqused_k
        self.k_scale, self.v_scale = k_scale, v_scale
        self.k_global_scale, self.v_global_scale = k_global_scale, v_global_scale
        self.softmax_scale, self.causal, self.splits = softmax_scale, causal, splits
        self.max_seqlen_q, self.max_k_tiles, self.topk = int(max_seqlen_q), int(max_k_tiles), topk
        total_q, hq, _ = q.shape
        hkv = k.shape[1]
        dev = q.device
        self.select = q2k is None
        if self.select:
            self.proxy_q = q if proxy_q is None else proxy_q
            self.reduce_heads = reduce_heads
            self.q2k = torch.empty(hkv, total_q, topk, dtype=torch.int32, device=dev)
            self.select_workspace = Workspace(max(1, proxy_topk_workspace_size(
                self.proxy_q, k, cu_seqlens_q, cu_seqlens_k, topk=topk, page_table=page_table,
                seqused_k=seqused_k, causal=causal, max_seqlen_q=self.max_seqlen_q,
                max_k_tiles=self.max_k_tiles, reduce_heads=reduce_heads)), dev)
        else:
            self.q2k = q2k
        need = workspace_size(q, k, v, self.q2k, cu_seqlens_q, cu_seqlens_k,
                              page_table=page_table, seqused_k=seqused_k, k_scale=k_scale,
                              v_scale=v_scale, max_seqlen_q=self.max_seqlen_q,
                              max_k_tiles=self.max_k_tiles, splits=splits)
        self.workspace = Workspace(need, dev) if need else None
        self.out = torch.empty_like(q)
        self.lse = (torch.empty(total_q, hq, dtype=torch.float32, device=dev)
                    if return_lse else None)

        # warm up on a side stream (default priority), then capture
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(warmup):
                self.step()
        torch.cuda.current_stream(dev).wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.step()

    def step(self):
        """The step itself, launched eagerly on the current stream."""
        if self.select:
            proxy_topk(self.proxy_q, self.k, self.cu_seqlens_q, self.cu_seqlens_k,
                       topk=self.topk, page_table=self.page_table, seqused_k=self.seqused_k,
                       causal=self.causal, max_seqlen_q=self.max_seqlen_q,
                       max_k_tiles=self.max_k_tiles, reduce_heads=self.reduce_heads,
                       out=self.q2k, workspace=self.select_workspace)
        return sparse_attention(
            self.q, self.k, self.v, self.q2k, self.cu_seqlens_q, self.cu_seqlens_k,
            causal=self.causal, softmax_scale=self.softmax_scale, page_table=self.page_table,
            seqused_k=self.seqused_k, return_softmax_lse=self.lse is not None,
            k_scale=self.k_scale, v_scale=self.v_scale, k_global_scale=self.k_global_scale,
            v_global_scale=self.v_global_scale, max_seqlen_q=self.max_seqlen_q,
            max_k_tiles=self.max_k_tiles, workspace=self.workspace, out=self.out, lse=self.lse,
            splits=self.splits)

    def replay(self):
        self.graph.replay()
        return self.out, self.lse
