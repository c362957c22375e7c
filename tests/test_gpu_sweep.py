"""Seeded random sweep of the attention, proxy and top-K calls against the
fp64 oracle (GPU).

Each seed draws a small problem: 1-5 requests (some with no queries or no
keys), G = Hq / Hkv from 1 to 32, bf16 / fp16 / fp8 / packed E2M1 K/V,
flat or paged, causal or not, prefill or decode-shaped queries, top-K 1-64,
split-KV 0-5, a softmax scale, global scales, the temperature LSE and
q_offset (an int or per-row positions).  Attention goes through whichever
route the library picks; the proxy (not E2M1) and the top-K follow on the
same inputs.  Tolerances as in the parity tests; outputs larger than 2 in
magnitude also get 2^-8 of the largest |out| (bf16's own spacing there is
1/64 to 1/32, and P enters the PV product in bf16).
"""
import random

import pytest
import torch

import oracle
import synth
import gpu_helpers
from gpu_helpers import assert_attention_close, assert_proxy_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _draw(seed):
    rng = random.Random(seed)
    hkv = rng.choice([1, 1, 2, 2, 3, 4, 8])
    G = rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16, 32])
    while G * hkv > 32:
        G = max(1, G // 2)
    fmt = rng.choice([synth.KV_BF16, synth.KV_BF16, synth.KV_F16, synth.KV_FP8, synth.KV_E2M1])
    c = dict(seed=seed, hkv=hkv, G=G, fmt=fmt, paged=rng.random() < 0.6,
             causal=rng.random() < 0.8, decode=rng.random() < 0.45)
    B = rng.randint(1, 5)
    if c["decode"]:
        lq = rng.choice([1, 1, 2, 4])
        c["q_lens"] = [lq] * B
        c["k_lens"] = [rng.choice([1, 127, 128, 129, rng.randint(1, 4000)]) for _ in range(B)]
    else:
        c["q_lens"] = [rng.choice([0, 1, 31, 32, 33, rng.randint(1, 200)]) for _ in range(B)]
        c["k_lens"] = [max(1, ql + rng.choice([0, 0, rng.randint(-20, 600)])) for ql in c["q_lens"]]
    c["topk"] = rng.choice([1, 3, 4, 8, 16, 33, 64])
    c["splits"] = rng.choice([0, 0, 1, 2, 3, 5])
    c["scale"] = rng.choice([None, None, 0.05, 0.2])
    if fmt == synth.KV_E2M1:
        c["gs"] = dict(k_global_scale=rng.choice([0.5, 1.0]), v_global_scale=rng.choice([1.0, 2.0]))
    else:
        c["gs"] = dict(v_global_scale=1.5) if rng.random() < 0.3 else {}
    c["tau"] = rng.choice([None, None, None, 0.5, 2.0, 8.0])
    c["q_offset"] = None
    if c["causal"] and rng.random() < 0.25:
        if rng.random() < 0.5:
            c["q_offset"] = rng.randint(-40, max(c["k_lens"]) + 40)
        else:
            c["q_offset"] = torch.tensor([rng.randint(-10, max(c["k_lens"]) + 10)
                                          for _ in range(sum(c["q_lens"]))], dtype=torch.int32)
    c["reduce"] = rng.choice([False, True, "group"])
    return c


@pytest.mark.parametrize("seed", range(5000, 5064))
def test_random_problem_matches_oracle(msa, seed):
    c = _draw(seed)
    hq, hkv = c["G"] * c["hkv"], c["hkv"]
    print(f"seed {seed}: q {c['q_lens']} k {c['k_lens']} Hq {hq} Hkv {hkv} {c['fmt']} "
          f"paged {c['paged']} causal {c['causal']} topk {c['topk']} splits {c['splits']} "
          f"tau {c['tau']} q_offset {type(c['q_offset']).__name__}", flush=True)
    p = synth.make_problem("sweep", q_lens=c["q_lens"], k_lens=c["k_lens"], num_qo_heads=hq,
                           num_kv_heads=hkv, topk=c["topk"], paged=c["paged"], kv_dtype=c["fmt"],
                           causal=c["causal"], seed=seed,
                           selection="decode" if c["decode"] else "general",
                           softmax_scale=c["scale"], **c["gs"])
    d = p.to("cuda")
    tau, qoff = c["tau"], c["q_offset"]
    res = msa.sparse_attention(
        d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k, causal=d.causal,
        softmax_scale=d.softmax_scale, page_table=d.page_table, seqused_k=d.seqused_k,
        return_softmax_lse=True, k_scale=d.k_scale, v_scale=d.v_scale,
        k_global_scale=d.k_global_scale, v_global_scale=d.v_global_scale,
        max_seqlen_q=max(c["q_lens"]), max_k_tiles=p.max_k_tiles, splits=c["splits"],
        return_temperature_lse=tau is not None, lse_temperature_scale=tau or 1.0,
        q_offset=qoff.cuda() if isinstance(qoff, torch.Tensor) else qoff)
    torch.cuda.synchronize()
    ref = oracle.sparse_attention(
        p.q, p.k, p.v, p.q2k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
        page_table=p.page_table, seqused_k=p.seqused_k, causal=p.causal,
        softmax_scale=p.softmax_scale, kv_format=p.kv_dtype, k_scale=p.k_scale,
        v_scale=p.v_scale, k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale,
        lse_temperature_scale=tau, q_offset=qoff)
    big = float(ref[0].abs().max()) if ref[0].numel() else 0.0
    tol = 2e-2 + (2.0 ** -8 * big if big > 2 else 0.0)
    saved, gpu_helpers.OUT_TOL = gpu_helpers.OUT_TOL, tol
    try:
        assert_attention_close(res[0], res[1], ref[0], ref[1], f"seed {seed}")
    finally:
        gpu_helpers.OUT_TOL = saved
    if tau is not None:
        lt, rlt = res[2].double().cpu(), ref[2]
        assert torch.equal(torch.isneginf(lt), torch.isneginf(rlt))
        fin = ~torch.isneginf(rlt)
        if fin.any():
            assert float((lt[fin] - rlt[fin]).abs().max()) <= 1e-3

    if c["fmt"] == synth.KV_E2M1 or sum(c["q_lens"]) == 0:
        return
    red, T = c["reduce"], p.max_k_tiles
    s = msa.proxy_score(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, page_table=d.page_table,
                        seqused_k=d.seqused_k, causal=c["causal"], max_seqlen_q=max(c["q_lens"]),
                        max_k_tiles=T, reduce_heads=red)
    torch.cuda.synchronize()
    rs = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
                            page_table=p.page_table, seqused_k=p.seqused_k, causal=c["causal"],
                            max_k_tiles=T, kv_format=c["fmt"])
    if red is True:
        rs = rs.amax(dim=0, keepdim=True)
    elif red == "group":
        rs = rs.view(hkv, c["G"], T, -1).amax(dim=1)
    assert_proxy_close(s, rs, f"seed {seed} proxy")
    mode = 1 if red is True else (0 if (red == "group" or hq == hkv) else 2)
    got = msa.topk_select(s, c["topk"], hkv, mode=mode)
    want = oracle.topk_select(s.cpu(), c["topk"], hkv, mode={0: "none", 1: "all", 2: "group"}[mode])
    assert torch.equal(got.cpu(), want)
