"""q_offset (msa_sparse_attention page and msa_proxy_score page, Parameters:
q_offset) through the C ABI against the oracle (GPU).

Reading (the pages leave it open; parity with the pages' own kernels is
unpinned): the queries' causal positions -- an int o puts query iq of every
request at KV position o + iq, a tensor gives each query row its own
position.  Right-aligned positions passed as a tensor must reproduce the
default bit for bit; other positions must match the oracle.
"""
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_attention_close, assert_proxy_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _right_aligned(p):
    pos = []
    for b in range(p.batch):
        lq, lk = p.q_lens[b], p.k_lens[b]
        pos += [lk - lq + i for i in range(lq)]
    return torch.tensor(pos, dtype=torch.int32)


def _random_positions(p, seed):
    g = torch.Generator().manual_seed(seed)
    pos = []
    for b in range(p.batch):
        lk = p.k_lens[b]
        pos += torch.randint(-40, lk + 60, (p.q_lens[b],), generator=g).tolist()
    return torch.tensor(pos, dtype=torch.int32)


def _attn(msa, p, q_offset, splits=0, temp=None):
    d = p.to("cuda")
    qo = q_offset.cuda() if isinstance(q_offset, torch.Tensor) else q_offset
    kw = {}
    if temp is not None:
        kw = dict(return_temperature_lse=True, lse_temperature_scale=temp)
    r = msa.sparse_attention(d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k, causal=True,
                             softmax_scale=p.softmax_scale, page_table=d.page_table,
                             seqused_k=d.seqused_k, return_softmax_lse=True, k_scale=d.k_scale,
                             v_scale=d.v_scale, k_global_scale=p.k_global_scale,
                             v_global_scale=p.v_global_scale, max_seqlen_q=max(p.q_lens),
                             max_k_tiles=p.max_k_tiles, splits=splits, q_offset=qo, **kw)
    torch.cuda.synchronize()
    return r


def _oracle(p, q_offset, temp=None):
    return oracle.sparse_attention(
        p.q, p.k, p.v, p.q2k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
        page_table=p.page_table, seqused_k=p.seqused_k, causal=True,
        softmax_scale=p.softmax_scale, kv_format=p.kv_dtype, k_scale=p.k_scale,
        v_scale=p.v_scale, k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale,
        q_offset=q_offset, lse_temperature_scale=temp)


PREFILL = [
    # q_lens, k_lens, Hq, Hkv, fmt, paged
    ([300, 77], [700, 129], 16, 2, synth.KV_BF16, False),
    ([260, 33], [400, 300], 8, 2, synth.KV_F16, False),
    ([200, 70], [700, 300], 8, 2, synth.KV_FP8, True),
    ([150], [500], 4, 1, synth.KV_E2M1, False),
]


@pytest.mark.parametrize("case", range(len(PREFILL)))
def test_prefill_q_offset(msa, case):
    ql, kl, hq, hkv, fmt, paged = PREFILL[case]
    print(f"q_offset prefill case {case} ({fmt})", flush=True)
    kw = dict(k_global_scale=0.5, v_global_scale=2.0) if fmt == synth.KV_E2M1 else {}
    p = synth.make_problem("qoff_pf", q_lens=ql, k_lens=kl, num_qo_heads=hq, num_kv_heads=hkv,
                           topk=4, paged=paged, kv_dtype=fmt, seed=110 + case,
                           selection="general", **kw)
    base = _attn(msa, p, None)
    same = _attn(msa, p, _right_aligned(p))
    assert torch.equal(base[0], same[0]) and torch.equal(base[1], same[1])
    for qo in (_random_positions(p, 7 + case), 100):
        out, lse = _attn(msa, p, qo)
        ro, rl = _oracle(p, qo)
        assert_attention_close(out, lse, ro, rl, f"prefill case {case} q_offset")


DECODE = [
    # q_lens, k_lens, Hq, Hkv, fmt, splits
    ([1, 1, 1], [3000, 129, 7000], 16, 2, synth.KV_BF16, 0),
    ([4, 4, 4], [2500, 600, 9000], 32, 2, synth.KV_FP8, 0),
    ([1, 1, 1, 1], [5000, 900, 3000, 200], 16, 1, synth.KV_E2M1, 3),
    ([3, 3], [2000, 700], 8, 2, synth.KV_BF16, 2),
]


@pytest.mark.parametrize("case", range(len(DECODE)))
def test_decode_q_offset(msa, case):
    ql, kl, hq, hkv, fmt, splits = DECODE[case]
    print(f"q_offset decode case {case} ({fmt}, splits {splits})", flush=True)
    kw = dict(k_global_scale=0.5, v_global_scale=2.0) if fmt == synth.KV_E2M1 else {}
    p = synth.make_problem("qoff_dec", q_lens=ql, k_lens=kl, num_qo_heads=hq, num_kv_heads=hkv,
                           topk=8, paged=True, kv_dtype=fmt, seed=120 + case,
                           selection="decode", **kw)
    assert msa.attention_plan(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q, page_table=p.page_table,
                              seqused_k=p.seqused_k, k_scale=p.k_scale, v_scale=p.v_scale,
                              max_seqlen_q=max(ql), max_k_tiles=p.max_k_tiles)[0] == 1
    base = _attn(msa, p, None, splits)
    same = _attn(msa, p, _right_aligned(p), splits)
    assert torch.equal(base[0], same[0]) and torch.equal(base[1], same[1])
    for qo in (_random_positions(p, 17 + case), 640):
        out, lse = _attn(msa, p, qo, splits)
        ro, rl = _oracle(p, qo)
        assert_attention_close(out, lse, ro, rl, f"decode case {case} q_offset")


def test_temperature_route_q_offset(msa):
    print("q_offset with the temperature LSE", flush=True)
    p = synth.make_problem("qoff_t", q_lens=[120, 9], k_lens=[400, 260], num_qo_heads=8,
                           num_kv_heads=2, topk=3, seed=131, selection="general")
    qo = _random_positions(p, 3)
    out, lse, lt = _attn(msa, p, qo, temp=0.7)
    ro, rl, rt = _oracle(p, qo, temp=0.7)
    assert_attention_close(out, lse, ro, rl, "temperature q_offset")
    f = torch.isfinite(rt)
    assert torch.equal(torch.isneginf(lt.cpu().double()), ~f)
    assert float((lt.cpu().double()[f] - rt[f]).abs().max()) <= 1e-3


PROXY = [
    # q_lens, k_lens, Hq, Hkv, fmt, paged, reduce
    ([300, 150], [700, 300], 4, 2, synth.KV_BF16, False, False),     # prefill-shaped kernel
    ([300, 150], [700, 300], 8, 2, synth.KV_BF16, False, "group"),
    ([4, 4, 4], [9000, 600, 3000], 32, 2, synth.KV_FP8, True, True),  # rows kernel
    ([2, 1], [3000, 260], 8, 2, synth.KV_BF16, True, False),
]


@pytest.mark.parametrize("case", range(len(PROXY)))
def test_proxy_q_offset(msa, case):
    ql, kl, hq, hkv, fmt, paged, reduce = PROXY[case]
    print(f"q_offset proxy case {case}", flush=True)
    p = synth.make_problem("qoff_px", q_lens=ql, k_lens=kl, num_qo_heads=hq, num_kv_heads=hkv,
                           topk=4, paged=paged, kv_dtype=fmt, seed=140 + case,
                           selection="general")
    d = p.to("cuda")

    def run(qo):
        qo = qo.cuda() if isinstance(qo, torch.Tensor) else qo
        s = msa.proxy_score(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, page_table=d.page_table,
                            seqused_k=d.seqused_k, causal=True, max_seqlen_q=max(ql),
                            max_k_tiles=p.max_k_tiles, reduce_heads=reduce, q_offset=qo)
        torch.cuda.synchronize()
        return s.cpu()

    assert torch.equal(run(None), run(_right_aligned(p)))
    for qo in (_random_positions(p, 27 + case), 90):
        got = run(qo)
        ref = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
                                 page_table=p.page_table, seqused_k=p.seqused_k, causal=True,
                                 max_k_tiles=p.max_k_tiles, reduce_heads=reduce is True,
                                 kv_format=fmt, q_offset=qo)
        if reduce == "group":
            ref = ref.view(hkv, hq // hkv, *ref.shape[1:]).amax(dim=1)
        assert_proxy_close(got, ref, f"proxy case {case} q_offset")
