"""HIP path vs the fp64 oracle on small seeded problems (GPU).

Sizes are chosen so the oracle finishes in seconds while the kernels still
see several tiles, several KV blocks, ragged tails (partial last block, a
partial last query tile), empty selections and blocks above the causal
limit.  Every call goes through the C ABI (via the ctypes binding).
"""
import pytest
import torch

import gpu_helpers
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


def _dev(p):
    return p.to("cuda")


# ---------------------------------------------------------------------------
# sparse attention, prefill shape
# ---------------------------------------------------------------------------

PREFILL_CASES = [
    # q_lens, k_lens, Hq, Hkv, topk, causal
    ([1024], [1024], 4, 1, 4, True),
    ([300, 77], [300, 500], 16, 2, 5, True),      # ragged tiles, Lq != Lk
    ([200], [700], 8, 1, 6, False),               # non-causal
    ([129, 64, 1], [129, 640, 200], 32, 2, 3, True),  # G = 16
    ([90], [400], 2, 2, 4, True),                 # MHA, G = 1
    ([150, 40], [150, 300], 6, 3, 4, True),       # G = 2
    ([300, 50], [200, 50], 8, 2, 4, True),        # Lq > Lk: the first 100 queries see no key
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_bf16_matches_oracle(msa, case):
    ql, kl, hq, hkv, topk, causal = PREFILL_CASES[case]
    p = synth.make_problem("prefill", q_lens=ql, k_lens=kl, num_qo_heads=hq, num_kv_heads=hkv,
                           topk=topk, causal=causal, seed=100 + case, selection="general")
    print(f"prefill case {case}: q {ql} k {kl} Hq {hq} Hkv {hkv} topk {topk}", flush=True)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, f"prefill case {case}")


@pytest.mark.parametrize("hq,hkv", [(6, 2), (10, 2), (12, 2), (24, 2), (40, 8)])
def test_prefill_groups_not_dividing_a_slot(msa, hq, hkv):
    # G = 3, 5, 6, 12: a token's heads straddle two 32-row slots (and the
    # tile's last slot is partly empty)
    p = synth.make_problem("prefill_odd_g", q_lens=[200, 61], k_lens=[700, 61], num_qo_heads=hq,
                           num_kv_heads=hkv, topk=5, seed=200 + hq, selection="general")
    print(f"prefill G {hq // hkv}", flush=True)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, f"prefill G {hq // hkv}")


@pytest.mark.parametrize("hq,hkv,lq,fmt", [(6, 2, 4, synth.KV_BF16), (10, 2, 4, synth.KV_FP8),
                                          (12, 1, 4, synth.KV_E2M1), (40, 8, 1, synth.KV_BF16)])
def test_decode_groups_not_dividing_a_row_tile(msa, hq, hkv, lq, fmt):
    # a token's heads straddle two 16-row tiles of the decode kernel
    kw = dict(k_global_scale=0.5, v_global_scale=2.0) if fmt == synth.KV_E2M1 else {}
    p = synth.make_problem("decode_odd_g", q_lens=[lq] * 3, k_lens=[3000, 129, 900],
                           num_qo_heads=hq, num_kv_heads=hkv, topk=6, paged=True, kv_dtype=fmt,
                           seed=210 + hq, selection="decode", **kw)
    print(f"decode G {hq // hkv} x {lq} tokens, {fmt}", flush=True)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, f"decode G {hq // hkv}")


@pytest.mark.parametrize("q_lens,k_lens,hq,hkv,topk,fmt,paged", [
    ([33, 15], [214, 15], 8, 8, 16, synth.KV_E2M1, True),
    ([32], [32], 2, 2, 33, synth.KV_F16, False),
    ([33, 0], [589, 64], 1, 1, 64, synth.KV_BF16, True),
    ([40, 40], [700, 300], 2, 1, 16, synth.KV_FP8, True),
])
def test_short_queries_past_the_decode_union(msa, q_lens, k_lens, hq, hkv, topk, fmt, paged):
    # few enough rows for a decode tile, too many selections for its union:
    # the prefill tiles take the call
    kw = dict(k_global_scale=0.5, v_global_scale=2.0) if fmt == synth.KV_E2M1 else {}
    p = synth.make_problem("short_q_union", q_lens=q_lens, k_lens=k_lens, num_qo_heads=hq,
                           num_kv_heads=hkv, topk=topk, paged=paged, kv_dtype=fmt, seed=230 + hq,
                           selection="general", **kw)
    d = _dev(p)
    route, _ = msa.attention_plan(d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k,
                                  page_table=d.page_table, seqused_k=d.seqused_k,
                                  k_scale=d.k_scale, v_scale=d.v_scale, max_seqlen_q=max(q_lens),
                                  max_k_tiles=p.max_k_tiles)
    assert route == 0
    print(f"short queries past the decode union: {q_lens} topk {topk} {fmt}", flush=True)
    out, lse = gpu_attention(msa, d)
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "short queries past the decode union")


def test_prefill_fp8_and_scales(msa):
    p = synth.make_problem("prefill_fp8", q_lens=[260, 33], k_lens=[400, 33], num_qo_heads=8,
                           num_kv_heads=2, topk=3, kv_dtype=synth.KV_FP8, seed=7,
                           selection="general", softmax_scale=0.05, v_global_scale=1.5)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "prefill fp8")


@pytest.mark.parametrize("hkv,q_lens,k_lens,head_major", [
    (1, [200, 64], [300, 64], False),   # one KV head
    (2, [260, 33], [400, 34], False),   # (token, head) scale rows, Lq != Lk
    (2, [90, 40], [129, 300], True),    # a head-major view of the scales
])
def test_prefill_flat_e2m1(msa, hkv, q_lens, k_lens, head_major):
    print(f"flat E2M1 prefill Hkv {hkv} {q_lens} {k_lens} head-major {head_major}", flush=True)
    p = synth.make_problem("prefill_e2m1_flat", q_lens=q_lens, k_lens=k_lens, num_qo_heads=8,
                           num_kv_heads=hkv, topk=3, kv_dtype=synth.KV_E2M1, seed=9 + hkv,
                           selection="general", k_global_scale=0.5, v_global_scale=2.0)
    if head_major:
        hm = lambda t: t.permute(1, 0, 2).contiguous().permute(1, 0, 2)
        p.k_scale, p.v_scale = hm(p.k_scale), hm(p.v_scale)
        assert p.k_scale.stride() == (8, 8 * sum(k_lens), 1)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "prefill flat e2m1")


@pytest.mark.parametrize("fmt", [synth.KV_FP8, synth.KV_E2M1])
def test_prefill_paged_quantised_kv(msa, fmt):
    # prefill shapes over a paged fp8 / E2M1 cache: the blocks are staged to
    # bf16 pages in the workspace and read by the bf16 prefill kernel
    print(f"paged {fmt} prefill", flush=True)
    kw = dict(k_global_scale=0.5, v_global_scale=2.0) if fmt == synth.KV_E2M1 else {}
    p = synth.make_problem("prefill_paged_q", q_lens=[200, 70, 9], k_lens=[700, 300, 129],
                           num_qo_heads=8, num_kv_heads=2, topk=4, paged=True, kv_dtype=fmt,
                           seed=81, selection="general", extra_pages=5, **kw)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, f"paged {fmt} prefill")


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_flat_e2m1(msa, splits):
    print(f"flat E2M1 decode splits {splits}", flush=True)
    p = synth.make_problem("decode_e2m1_flat", q_lens=[1, 1, 1, 1], k_lens=[2000, 129, 700, 3001],
                           num_qo_heads=16, num_kv_heads=2, topk=6, kv_dtype=synth.KV_E2M1,
                           seed=31 + splits, selection="decode", k_global_scale=0.5,
                           v_global_scale=2.0)
    d = _dev(p)
    # flat E2M1 takes the prefill tiles over staged bf16 pages of only the
    # selected blocks; a requested split factor is not used there
    route = msa.attention_plan(d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k,
                               k_scale=d.k_scale, v_scale=d.v_scale, max_seqlen_q=1,
                               max_k_tiles=p.max_k_tiles, splits=splits)
    assert route == (0, 1)
    out, lse = gpu_attention(msa, d, splits=splits)
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "decode flat e2m1")


TEMPERATURE_CASES = [
    # q_lens, k_lens, Hq, Hkv, paged, fmt, tau, selection, splits, softmax_scale
    ([300, 77], [300, 500], 16, 2, False, synth.KV_BF16, 0.5, "general", 0, None),
    ([260, 33], [400, 33], 8, 2, False, synth.KV_FP8, 2.0, "general", 0, None),
    ([1, 1, 1], [2000, 129, 700], 16, 2, True, synth.KV_BF16, 1.5, "decode", 0, None),
    ([1, 1], [3000, 900], 16, 1, True, synth.KV_E2M1, 0.7, "decode", 0, None),
    ([4, 4], [2500, 600], 32, 2, True, synth.KV_FP8, 1.0, "decode", 0, None),
    # tau > 1 shrinks the rescale slack to 64 / tau; a large softmax scale
    # spreads the logits so the reference max moves
    ([300, 129], [700, 300], 8, 2, False, synth.KV_BF16, 10.0, "general", 0, 0.5),
    ([200, 64], [500, 300], 8, 1, False, synth.KV_F16, 4.0, "general", 0, 0.3),
    ([150, 40], [600, 300], 8, 2, True, synth.KV_E2M1, 0.1, "general", 0, None),
    ([1, 1, 1, 1], [9000, 129, 3000, 700], 16, 1, True, synth.KV_E2M1, 3.0, "decode", 3, 0.8),
    ([1, 1, 1], [5000, 300, 2000], 16, 2, True, synth.KV_BF16, 6.0, "decode", 2, 0.5),
    ([2, 2], [3000, 900], 16, 2, True, synth.KV_F16, 2.5, "decode", 0, 0.25),
]


@pytest.mark.parametrize("case", range(len(TEMPERATURE_CASES)))
def test_temperature_lse_matches_oracle(msa, case):
    ql, kl, hq, hkv, paged, fmt, tau, selection, splits, scale = TEMPERATURE_CASES[case]
    print(f"temperature LSE case {case}", flush=True)
    kw = dict(k_global_scale=0.5, v_global_scale=2.0) if fmt == synth.KV_E2M1 else {}
    p = synth.make_problem("temp", q_lens=ql, k_lens=kl, num_qo_heads=hq, num_kv_heads=hkv,
                           topk=6, paged=paged, kv_dtype=fmt, seed=60 + case,
                           selection=selection, softmax_scale=scale, **kw)
    d = _dev(p)
    # the temperature LSE keeps the tuned routes: decode shapes the decode
    # kernel (split as asked), prefill shapes the prefill tiles
    route, nsplit = msa.attention_plan(
        d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k, page_table=d.page_table,
        seqused_k=d.seqused_k, k_scale=d.k_scale, v_scale=d.v_scale, max_seqlen_q=max(ql),
        max_k_tiles=p.max_k_tiles, splits=splits, return_temperature_lse=True)
    assert route == (1 if selection == "decode" else 0)
    if splits:
        assert nsplit == splits
    out, lse, lse_t = msa.sparse_attention(
        d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k, causal=p.causal,
        softmax_scale=scale, page_table=d.page_table, seqused_k=d.seqused_k, k_scale=d.k_scale,
        v_scale=d.v_scale, k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale,
        max_seqlen_q=max(ql), max_k_tiles=p.max_k_tiles, return_temperature_lse=True,
        lse_temperature_scale=tau, splits=splits)
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_lt = oracle.sparse_attention(
        p.q, p.k, p.v, p.q2k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
        page_table=p.page_table, seqused_k=p.seqused_k, causal=p.causal, kv_format=fmt,
        softmax_scale=scale, k_scale=p.k_scale, v_scale=p.v_scale,
        k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale,
        lse_temperature_scale=tau)
    assert_attention_close(out, lse, ref_out, ref_lse, f"temperature case {case}")
    lt = lse_t.cpu().double()
    fin = torch.isfinite(ref_lt)
    assert torch.equal(torch.isfinite(lt), fin)
    assert float((lt[fin] - ref_lt[fin]).abs().max()) <= 1e-3
    # the same call without lse_t gives the same out and lse, bit for bit
    out2, lse2 = msa.sparse_attention(
        d.q, d.k, d.v, d.q2k, d.cu_seqlens_q, d.cu_seqlens_k, causal=p.causal,
        softmax_scale=scale, page_table=d.page_table, seqused_k=d.seqused_k, k_scale=d.k_scale,
        v_scale=d.v_scale, k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale,
        max_seqlen_q=max(ql), max_k_tiles=p.max_k_tiles, return_softmax_lse=True, splits=splits)
    torch.cuda.synchronize()
    if tau <= 1.0:   # (tau > 1 moves the reference max on its own slack)
        assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_prefill_without_lse_and_diagonal_selection(msa):
    p = synth.make_problem("prefill_diag", q_lens=[640], k_lens=[640], num_qo_heads=8,
                           num_kv_heads=1, topk=4, seed=8, selection="diagonal")
    out = gpu_attention(msa, _dev(p), lse=False)
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, None, ref_out, ref_lse, "prefill no lse")


def test_full_selection_is_dense_causal(msa):
    # every causally valid block selected: equals dense causal attention
    ql = kl = [384, 200]
    p = synth.make_problem("dense", q_lens=ql, k_lens=kl, num_qo_heads=8, num_kv_heads=2,
                           topk=3, seed=9, selection="proxy")
    rows = []
    for L in ql:
        for i in range(L):
            n = i // 128 + 1
            rows.append(list(range(n)) + [-1] * (3 - n))
    p.q2k = torch.tensor(rows, dtype=torch.int32).unsqueeze(0).repeat(2, 1, 1)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "dense")
    assert torch.isfinite(lse).all()


def test_empty_and_out_of_range_rows(msa):
    p = synth.make_problem("empty", q_lens=[64, 10], k_lens=[300, 10], num_qo_heads=4,
                           num_kv_heads=1, topk=4, seed=10, selection="general")
    q2k = p.q2k.clone()
    q2k[:, :20] = -1                 # nothing selected
    q2k[:, 20:30, 0] = 2             # block 2 holds keys 256..299; queries at
    q2k[:, 20:30, 1:] = -1           # positions 256..265 see some of it
    q2k[:, 30:40, 0] = 9             # past the sequence: ignored
    q2k[:, 30:40, 1:] = -1
    p.q2k = q2k
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "empty rows")
    assert (out[:20].float() == 0).all() and torch.isneginf(lse[:20]).all()
    assert (out[30:40].float() == 0).all()


# ---------------------------------------------------------------------------
# sparse attention, decode shape (paged, split-KV + LSE merge)
# ---------------------------------------------------------------------------

DECODE_CASES = [
    # batch, seqlen_q, Hq, Hkv, fmt, splits, kgs, vgs
    (5, 1, 64, 4, synth.KV_BF16, 0, None, None),
    (5, 1, 64, 4, synth.KV_BF16, 1, None, None),
    (3, 4, 32, 2, synth.KV_FP8, 0, None, None),
    (3, 4, 32, 2, synth.KV_FP8, 3, None, None),
    (6, 1, 16, 1, synth.KV_E2M1, 0, 0.5, 2.0),
    (6, 1, 16, 1, synth.KV_E2M1, 5, 0.5, 2.0),
    (4, 2, 8, 1, synth.KV_BF16, 2, None, None),     # 16 rows: 2 tokens x 8 heads
    (2, 3, 12, 1, synth.KV_FP8, 4, None, 1.25),     # 36 rows, 3 slots
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_paged_matches_oracle(msa, case):
    B, sq, hq, hkv, fmt, splits, kgs, vgs = DECODE_CASES[case]
    g = torch.Generator().manual_seed(200 + case)
    lens = [int(x) for x in torch.randint(200, 3000, (B,), generator=g)]
    lens[0] = 129  # a two-page request whose last page holds one key
    p = synth.make_problem("decode", q_lens=[sq] * B, k_lens=lens, num_qo_heads=hq,
                           num_kv_heads=hkv, topk=8, paged=True, kv_dtype=fmt, seed=300 + case,
                           selection="general", k_global_scale=kgs, v_global_scale=vgs,
                           extra_pages=3)
    print(f"decode case {case}: B {B} sq {sq} Hq {hq} Hkv {hkv} fmt {fmt} splits {splits}", flush=True)
    out, lse = gpu_attention(msa, _dev(p), splits=splits)
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, f"decode case {case}")


def test_decode_single_token_rows_out_of_order_and_repeated(msa):
    # one-token rows are used directly as the union only when ascending
    # without repeats; other rows go through the general union builder
    p = synth.make_problem("dec_perm", q_lens=[1] * 5, k_lens=[3000, 900, 4100, 128, 2500],
                           num_qo_heads=16, num_kv_heads=2, topk=8, paged=True, seed=21,
                           selection="decode")
    g = torch.Generator().manual_seed(5)
    q2k = p.q2k.clone()
    for h in range(q2k.shape[0]):
        for i in range(q2k.shape[1]):
            row = q2k[h, i]
            q2k[h, i] = row[torch.randperm(row.numel(), generator=g)]
    q2k[0, 0, 1] = q2k[0, 0, 0]      # a repeated id
    q2k[1, 2, :] = -1                # an empty row
    p.q2k = q2k
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "unsorted one-token rows")


COUNTER_BYTES = 64 * 1024   # the split arrival counters at the end of a workspace


def test_split_merge_in_kernel_many_launches(msa):
    # the last split of every unit merges the others' partials (device-scope
    # stores and loads, no fence): many launches with new queries each time,
    # split factors 2..5, and a staged fp8 prefill through the same cached
    # workspace in between, against the unsplit launch
    p = synth.make_problem("merge", q_lens=[1] * 40, k_lens=[int(x) for x in
                           torch.randint(300, 20000, (40,), generator=torch.Generator().manual_seed(3))],
                           num_qo_heads=16, num_kv_heads=1, topk=16, paged=True,
                           kv_dtype=synth.KV_E2M1, seed=33, selection="decode",
                           k_global_scale=0.5, v_global_scale=2.0)
    d = _dev(p)
    pf = _dev(synth.make_problem("merge_pf", q_lens=[300], k_lens=[700], num_qo_heads=8,
                                 num_kv_heads=2, topk=3, kv_dtype=synth.KV_FP8, seed=34,
                                 selection="general"))
    g = torch.Generator(device="cuda").manual_seed(5)
    for it in range(24):
        d.q.copy_(torch.randn(d.q.shape, generator=g, device="cuda").to(d.q.dtype))
        splits = 2 + it % 4
        a = gpu_attention(msa, d, splits=splits)
        ref = gpu_attention(msa, d, splits=1)
        if it % 6 == 0:
            gpu_attention(msa, pf)            # fp8 prefill: staged pages in the workspace
        torch.cuda.synchronize()
        assert (a[0].float() - ref[0].float()).abs().max() <= 2e-2, it
        assert (a[1] - ref[1]).abs().max() <= 1e-3, it


def test_decode_is_deterministic_and_workspace_carries_no_state(msa):
    # (apart from the split counters in the last 64 KiB, kept at zero)
    p = _dev(synth.make_problem("det", q_lens=[4] * 6, k_lens=[5000, 3000, 900, 4000, 128, 2000],
                                num_qo_heads=32, num_kv_heads=2, topk=16, paged=True,
                                kv_dtype=synth.KV_FP8, seed=11, selection="decode"))
    ws = msa.Workspace(msa.workspace_size(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q, page_table=p.page_table,
                                          seqused_k=p.seqused_k, max_seqlen_q=4,
                                          max_k_tiles=p.max_k_tiles, splits=4), "cuda")
    ws.view[:-COUNTER_BYTES].fill_(0xFF)   # NaN bytes: nothing may be read before it is written
    a = gpu_attention(msa, p, splits=4, workspace=ws)
    # a different shape through the same workspace in between
    small = _dev(synth.make_problem("det2", q_lens=[1, 1], k_lens=[700, 300], num_qo_heads=16,
                                    num_kv_heads=1, topk=4, paged=True, seed=12,
                                    selection="decode"))
    gpu_attention(msa, small, splits=2, workspace=ws)
    b = gpu_attention(msa, p, splits=4, workspace=ws)
    c = gpu_attention(msa, p, splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[0], c[0])
    assert torch.equal(a[1], b[1]) and torch.equal(a[1], c[1])
    ref_out, ref_lse = oracle_attention(p.to("cpu"))
    assert_attention_close(a[0], a[1], ref_out, ref_lse, "decode splits=4")
    assert not ws.view[-COUNTER_BYTES:].any()   # every merge reset its counter
    # split factors agree with each other within tolerance
    one = gpu_attention(msa, p, splits=1)
    assert float((one[0].float() - a[0].float()).abs().max()) <= 2e-2


def test_fp8_subnormals_and_e2m1_halves_decode_exactly(msa):
    # V made of E4M3 subnormal codes only, amplified through v_global_scale:
    # a flushed subnormal would move the output by ~100 x 2^-9
    p = synth.make_problem("sub", q_lens=[1, 1], k_lens=[256, 256], num_qo_heads=16,
                           num_kv_heads=1, topk=2, paged=True, kv_dtype=synth.KV_FP8, seed=12,
                           selection="decode", v_global_scale=100.0)
    codes = torch.tensor([1, 2, 3, 4, 5, 6, 7, 0x81, 0x82, 0x87], dtype=torch.uint8)
    idx = torch.randint(0, len(codes), p.v.shape, generator=torch.Generator().manual_seed(1))
    p.v = codes[idx].view(torch.float8_e4m3fn)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "fp8 subnormal V")
    # E2M1 with every nibble and subnormal E4M3 block scales
    pe = synth.make_problem("e2", q_lens=[1, 1], k_lens=[256, 200], num_qo_heads=16,
                            num_kv_heads=1, topk=2, paged=True, kv_dtype=synth.KV_E2M1, seed=13,
                            selection="decode", v_global_scale=64.0, k_global_scale=0.5)
    gen = torch.Generator().manual_seed(2)
    pe.v = torch.randint(0, 256, pe.v.shape, generator=gen, dtype=torch.int64).to(torch.uint8)
    pe.v_scale = torch.randint(1, 8, pe.v_scale.shape, generator=gen, dtype=torch.int64).to(torch.uint8)
    out, lse = gpu_attention(msa, _dev(pe))
    ref_out, ref_lse = oracle_attention(pe)
    assert_attention_close(out, lse, ref_out, ref_lse, "e2m1 all nibbles")


# ---------------------------------------------------------------------------
# proxy score
# ---------------------------------------------------------------------------

PROXY_CASES = [
    # q_lens, k_lens, Hq, Hkv, paged, fmt, causal, reduce
    ([300, 77], [300, 500], 2, 2, False, synth.KV_BF16, True, False),
    ([513], [513], 1, 1, False, synth.KV_BF16, True, False),
    ([200], [700], 4, 2, False, synth.KV_BF16, False, False),
    ([4, 4, 4], [3000, 129, 1000], 32, 2, True, synth.KV_FP8, True, True),
    ([4, 4], [700, 1300], 32, 2, True, synth.KV_FP8, True, False),
    ([1, 1, 1], [900, 128, 2000], 16, 1, True, synth.KV_BF16, True, True),
    ([3, 2], [1000, 500], 6, 2, True, synth.KV_BF16, True, True),  # G = 3 (atomic path)
    ([150, 90], [400, 300], 10, 2, False, synth.KV_BF16, True, True),  # wide, G = 5, all heads
    ([300, 50], [200, 50], 2, 2, False, synth.KV_BF16, True, False),   # Lq > Lk
]


@pytest.mark.parametrize("case", range(len(PROXY_CASES)))
def test_proxy_matches_oracle(msa, case):
    ql, kl, hq, hkv, paged, fmt, causal, reduce = PROXY_CASES[case]
    p = synth.make_problem("proxy", q_lens=ql, k_lens=kl, num_qo_heads=hq, num_kv_heads=hkv,
                           paged=paged, kv_dtype=fmt, causal=causal, seed=400 + case,
                           selection="proxy", reduce_heads=reduce)
    print(f"proxy case {case}", flush=True)
    d = _dev(p)
    T = p.max_k_tiles + 2  # extra columns past every sequence must be -inf
    got = msa.proxy_score(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, page_table=d.page_table,
                          seqused_k=d.seqused_k, causal=causal, max_seqlen_q=max(ql),
                          max_k_tiles=T, reduce_heads=reduce)
    ref = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
                             page_table=p.page_table, seqused_k=p.seqused_k, causal=causal,
                             max_k_tiles=T, reduce_heads=reduce, kv_format=fmt)
    assert_proxy_close(got, ref, f"proxy case {case}")


# Prefill-shaped proxy: every workgroup scores an equal piece of a reflected
# row-tile pair's visible blocks (pieces may span both tiles of the pair).
WIDE_PROXY_CASES = [
    # q_lens, k_lens, Hq, Hkv, paged, fmt, causal, reduce, extra columns
    ([1280], [1280], 1, 1, False, synth.KV_BF16, True, False, 0),        # 5 row tiles: the middle one alone
    ([600, 1100], [600, 1500], 2, 2, False, synth.KV_FP8, True, False, 3),   # fp8 K, ragged
    ([520, 260], [900, 700], 16, 2, True, synth.KV_BF16, True, "group", 1),  # paged, G = 8 reduced
    ([300, 300, 300, 129, 700], [300, 800, 301, 129, 700], 4, 2, False, synth.KV_BF16, True, True, 0),  # 10 (request, KV head) units
    ([700], [5000], 2, 1, True, synth.KV_FP8, False, False, 2),           # non-causal, 40 blocks per row
    ([2048], [2048], 1, 1, False, synth.KV_F16, True, False, 0),          # fp16 Q and K, 8 row tiles
]


@pytest.mark.parametrize("case", range(len(WIDE_PROXY_CASES)))
def test_wide_proxy_pieces_match_oracle(msa, case):
    ql, kl, hq, hkv, paged, fmt, causal, reduce, extra = WIDE_PROXY_CASES[case]
    p = synth.make_problem("wide_proxy", q_lens=ql, k_lens=kl, num_qo_heads=hq,
                           num_kv_heads=hkv, paged=paged, kv_dtype=fmt, causal=causal,
                           seed=430 + case, selection="proxy",
                           reduce_heads=reduce is True)
    print(f"wide proxy case {case}", flush=True)
    d = _dev(p)
    T = p.max_k_tiles + extra
    got = msa.proxy_score(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, page_table=d.page_table,
                          seqused_k=d.seqused_k, causal=causal, max_seqlen_q=max(ql),
                          max_k_tiles=T, reduce_heads=reduce)
    torch.cuda.synchronize()
    ref = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
                             page_table=p.page_table, seqused_k=p.seqused_k, causal=causal,
                             max_k_tiles=T, reduce_heads=reduce is True, kv_format=fmt)
    if reduce == "group":
        ref = ref.view(hkv, hq // hkv, T, -1).amax(dim=1)
    assert_proxy_close(got, ref, f"wide proxy case {case}")


# ---------------------------------------------------------------------------
# top-K select
# ---------------------------------------------------------------------------

def _adversarial_scores(hs, T, n, seed):
    g = torch.Generator().manual_seed(seed)
    s = torch.randn(hs, T, n, generator=g)
    k = n // 5
    s[:, :, :k] = torch.randint(-2, 3, (hs, T, k), generator=g).float()   # heavy ties
    s[:, :, k:2 * k] = 0.0
    s[:, ::2, k:2 * k] = -0.0                                              # +-0 ties
    s[:, 3:, 2 * k:3 * k] = float("-inf")                                  # few finite
    s[:, :, 3 * k] = float("-inf")                                         # none finite
    return s


@pytest.mark.parametrize("T,topk,hs,hkv,mode", [
    (64, 16, 2, 2, 0), (7, 16, 2, 2, 0), (1024, 16, 1, 2, 1), (130, 4, 8, 2, 2),
    (300, 33, 3, 1, 1), (64, 64, 1, 1, 0), (4096, 16, 1, 1, 0), (16384, 64, 1, 1, 0),
    (2000, 40, 2, 2, 0), (257, 16, 4, 2, 2),
])
def test_topk_bit_exact(msa, T, topk, hs, hkv, mode):
    s = _adversarial_scores(hs, T, 257, seed=T + topk)
    got = msa.topk_select(s.cuda(), topk, hkv, mode=mode)
    mode_name = {0: "none", 1: "all", 2: "group"}[mode]
    ref = oracle.topk_select(s, topk, hkv, mode=mode_name)
    assert torch.equal(got.cpu(), ref)


@pytest.mark.parametrize("T,topk,hs,hkv,mode", [
    (64, 16, 2, 2, 0), (50, 16, 3, 1, 1), (64, 8, 4, 2, 2),
])
def test_topk_many_rows(msa, T, topk, hs, hkv, mode):
    # a full-size row count (16387 queries) with the adversarial score mix
    s = _adversarial_scores(hs, T, 16387, seed=3 * T + mode)
    got = msa.topk_select(s.cuda(), topk, hkv, mode=mode)
    ref = oracle.topk_select(s, topk, hkv, mode={0: "none", 1: "all", 2: "group"}[mode])
    assert torch.equal(got.cpu(), ref)


@pytest.mark.parametrize("T", [64, 200])
def test_topk_shared_prefix_rows(msa, T):
    # rows whose finite scores agree in their leading bits (the search starts
    # below that prefix) or whose top-K is settled before the last bit
    rows = [
        torch.full((T,), 1.5),                                        # all equal
        torch.tensor([1.0 + i * 2.0 ** -23 for i in range(T)]),       # last bits only
        torch.where(torch.arange(T) % 4 == 1, 3.0, 2.0),              # exactly T/4 at the top
        torch.where(torch.arange(T) < 20, 7.0, -7.0),                 # 20 tied at the max
        torch.linspace(-1.0, 1.0, T),                                 # both signs
        torch.where(torch.arange(T) % 7 == 0, 0.25, float("-inf")),   # few finite
        torch.tensor([2.0 ** -(i % 30) for i in range(T)]),           # exponents only
    ]
    s = torch.stack(rows, dim=1).unsqueeze(0).contiguous()            # (1, T, rows)
    for topk in (1, 16, 17):
        got = msa.topk_select(s.cuda(), topk, 1, mode=0)
        ref = oracle.topk_select(s, topk, 1, mode="none")
        assert torch.equal(got.cpu(), ref), topk


# ---------------------------------------------------------------------------
# tile union
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tile_tokens", [1, 4, 16, 64])
def test_tile_union_bit_exact(msa, tile_tokens):
    p = synth.make_problem("union", q_lens=[300, 5, 64], k_lens=[2000, 900, 64 * 128],
                           num_qo_heads=2, num_kv_heads=2, topk=8, seed=tile_tokens,
                           selection="general")
    lens = torch.tensor(p.k_lens, dtype=torch.int32)
    T = p.max_k_tiles
    blocks, masks, counts = msa.tile_union(p.q2k.cuda(), p.cu_seqlens_q.cuda(), lens.cuda(),
                                           tile_tokens, T)
    blocks, masks, counts = blocks.cpu(), masks.cpu(), counts.cpu()
    cu = p.cu_seqlens_q.tolist()
    for g in range(2):
        for b in range(3):
            nblk = (p.k_lens[b] + 127) // 128
            for j in range(blocks.shape[2]):
                i0 = cu[b] + j * tile_tokens
                i1 = min(cu[b + 1], i0 + tile_tokens)
                if i0 >= cu[b + 1]:
                    assert int(counts[g, b, j]) == 0
                    continue
                ref_b, ref_m = oracle.tile_union(p.q2k[g, i0:i1], nblk)
                n = int(counts[g, b, j])
                assert blocks[g, b, j, :n].tolist() == ref_b
                assert [m % (1 << 64) for m in masks[g, b, j, :n].tolist()] == ref_m
                assert (blocks[g, b, j, n:] == -1).all()


@pytest.mark.parametrize("fmt,hq,hkv,splits", [
    (synth.KV_FP8, 32, 2, 0), (synth.KV_BF16, 32, 1, 2), (synth.KV_E2M1, 16, 1, 0),
    (synth.KV_FP8, 16, 1, 3),
])
def test_decode_per_token_tiles_with_uneven_query_lengths(msa, fmt, hq, hkv, splits):
    # G >= 16 puts every query token in a workgroup of its own; requests of
    # different lengths (one empty) start away from b * max_seqlen_q, so the
    # kernel re-reads their rows after the speculative first read
    q_lens = [4, 1, 0, 3, 4, 2]
    p = synth.make_problem("dec_uneven", q_lens=q_lens, k_lens=[2000, 129, 700, 5000, 300, 1500],
                           num_qo_heads=hq, num_kv_heads=hkv, topk=8, paged=True, kv_dtype=fmt,
                           seed=41 + hq + splits, selection="general",
                           k_global_scale=0.5 if fmt == synth.KV_E2M1 else None,
                           v_global_scale=2.0 if fmt == synth.KV_E2M1 else None)
    print(f"uneven decode fmt {fmt} Hq {hq} Hkv {hkv} splits {splits}", flush=True)
    out, lse = gpu_attention(msa, _dev(p), splits=splits)
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "uneven decode")


@pytest.mark.parametrize("ql,kl,hq,hkv,paged,fmt", [
    ([300, 200], [300, 456], 16, 2, False, synth.KV_BF16),     # > 64 rows: wide kernel
    ([4, 4, 4], [3000, 700, 129], 32, 2, True, synth.KV_FP8),   # <= 64 rows: rows kernel
    ([2, 1], [1000, 2000], 8, 1, True, synth.KV_BF16),
    ([150, 90], [400, 300], 10, 2, False, synth.KV_BF16),    # G = 5 (not a power of 2), wide
    ([4, 4], [2000, 700], 12, 2, True, synth.KV_FP8),         # G = 6, rows kernel
])
def test_proxy_group_reduction_in_kernel(msa, ql, kl, hq, hkv, paged, fmt):
    # reduce_heads="group": the max over each KV head's G query heads is taken
    # inside the proxy kernel; it must equal the per-head oracle maxed over
    # the group, and select exactly what the top-K's own group mode selects
    p = synth.make_problem("proxy_group", q_lens=ql, k_lens=kl, num_qo_heads=hq,
                           num_kv_heads=hkv, paged=paged, kv_dtype=fmt, causal=True, seed=77,
                           selection="proxy")
    print(f"proxy group ql {ql} Hq {hq} Hkv {hkv} paged {paged} fmt {fmt}", flush=True)
    d = _dev(p)
    T = p.max_k_tiles + 1
    kw = dict(page_table=d.page_table, seqused_k=d.seqused_k, causal=True,
              max_seqlen_q=max(ql), max_k_tiles=T)
    got = msa.proxy_score(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, reduce_heads="group", **kw)
    assert got.shape == (hkv, T, sum(ql))
    ref = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
                             page_table=p.page_table, seqused_k=p.seqused_k, causal=True,
                             max_k_tiles=T, kv_format=fmt)
    G = hq // hkv
    ref_group = ref.view(hkv, G, T, -1).amax(dim=1)
    assert_proxy_close(got, ref_group, "group-reduced proxy")
    per_head = msa.proxy_score(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, **kw)
    a = msa.topk_select(got, 4, hkv, mode=0)
    b = msa.topk_select(per_head, 4, hkv, mode=2)
    assert torch.equal(a.cpu(), b.cpu())


@pytest.mark.parametrize("B,sq,hq,hkv,paged,splits", [
    (5, 1, 64, 4, True, 0), (5, 1, 64, 4, True, 3), (3, 4, 32, 2, True, 0),
    (4, 2, 8, 1, False, 2),
])
def test_decode_fp16_matches_oracle(msa, B, sq, hq, hkv, paged, splits):
    # fp16 q, k, v and out (the page's "bf16/fp16"); P is fp16 too, so its
    # reference max moves once a score passes it by 15 (log2 units)
    g = torch.Generator().manual_seed(900 + B * sq)
    lens = [int(x) for x in torch.randint(200, 3000, (B,), generator=g)]
    lens[0] = 129
    p = synth.make_problem("dec16", q_lens=[sq] * B, k_lens=lens, num_qo_heads=hq,
                           num_kv_heads=hkv, topk=8, paged=paged, kv_dtype=synth.KV_F16,
                           seed=901 + B, selection="general")
    print(f"fp16 decode B {B} sq {sq} Hq {hq} Hkv {hkv} paged {paged} splits {splits}", flush=True)
    out, lse = gpu_attention(msa, _dev(p), splits=splits)
    assert out.dtype == torch.float16
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "fp16 decode")


def test_decode_fp16_large_score_spread(msa):
    # scores spread far beyond the fp16 slack: the rare rescale path runs
    p = synth.make_problem("dec16s", q_lens=[1] * 3, k_lens=[2000, 900, 3000], num_qo_heads=16,
                           num_kv_heads=1, topk=8, paged=True, kv_dtype=synth.KV_F16, seed=5,
                           selection="decode", softmax_scale=0.8)
    out, lse = gpu_attention(msa, _dev(p))
    ref_out, ref_lse = oracle_attention(p)
    assert torch.isfinite(out.float()).all()
    assert_attention_close(out, lse, ref_out, ref_lse, "fp16 decode, wide scores")


@pytest.mark.parametrize("hq,hkv,causal", [(16, 2, True), (4, 1, True), (8, 8, False)])
def test_prefill_fp16_matches_oracle(msa, hq, hkv, causal):
    # fp16 q, k, v and out through the prefill kernel: several tiles, a
    # ragged tail, irregular selections
    p = synth.make_problem("pf16", q_lens=[300, 77], k_lens=[300, 900], num_qo_heads=hq,
                           num_kv_heads=hkv, topk=4, causal=causal, kv_dtype=synth.KV_F16,
                           seed=31 + hq, selection="general")
    print(f"fp16 prefill Hq {hq} Hkv {hkv} causal {causal}", flush=True)
    out, lse = gpu_attention(msa, _dev(p))
    assert out.dtype == torch.float16
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "fp16 prefill")


def test_prefill_fp16_large_score_spread(msa):
    # a large softmax scale spreads scores far past the fp16 slack of 15
    # (log2 units): the reference max moves and O is rescaled, P stays finite
    p = synth.make_problem("pf16s", q_lens=[260], k_lens=[700], num_qo_heads=8, num_kv_heads=1,
                           topk=4, kv_dtype=synth.KV_F16, seed=77, selection="general",
                           softmax_scale=0.7)
    out, lse = gpu_attention(msa, _dev(p))
    assert torch.isfinite(out.float()).all()
    ref_out, ref_lse = oracle_attention(p)
    assert_attention_close(out, lse, ref_out, ref_lse, "fp16 prefill, wide scores")


@pytest.mark.parametrize("ql,kl,hq,hkv,paged,reduce", [
    ([300, 200], [300, 456], 8, 2, False, False),    # > 64 rows: wide kernel
    ([4, 4], [2000, 700], 32, 2, True, True),        # <= 64 rows: rows kernel, reduce_heads
    ([1, 1, 1], [900, 129, 3000], 16, 1, True, False),
])
def test_proxy_fp16_matches_oracle(msa, ql, kl, hq, hkv, paged, reduce):
    # the msa_proxy_score page: "q ... bf16 or fp16"; fp16 q with fp16 K
    p = synth.make_problem("proxy16", q_lens=ql, k_lens=kl, num_qo_heads=hq, num_kv_heads=hkv,
                           paged=paged, kv_dtype=synth.KV_F16, causal=True, seed=55,
                           selection="proxy", reduce_heads=reduce)
    print(f"fp16 proxy ql {ql} Hq {hq} Hkv {hkv} paged {paged} reduce {reduce}", flush=True)
    d = _dev(p)
    T = p.max_k_tiles + 1
    got = msa.proxy_score(d.q, d.k, d.cu_seqlens_q, d.cu_seqlens_k, page_table=d.page_table,
                          seqused_k=d.seqused_k, causal=True, max_seqlen_q=max(ql),
                          max_k_tiles=T, reduce_heads=reduce)
    ref = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k,
                             page_table=p.page_table, seqused_k=p.seqused_k, causal=True,
                             max_k_tiles=T, reduce_heads=reduce, kv_format=synth.KV_F16)
    assert_proxy_close(got, ref, "fp16 proxy")


@pytest.mark.parametrize("route", ["flat_selected", "flat_whole", "paged_decode"])
def test_e2m1_every_scale_byte(msa, route):
    # 256 one-key requests; request b's K and V block scales are the E4M3 byte
    # b and every E2M1 code is 1.0, so out = v_gs * decode(b) and lse = z of
    # that one key (the oracle gives NaN for the bytes 0x7F / 0xFF).  Covers the staged
    # flat route (selected blocks, and every visible block) and the paged
    # decode kernel.
    print(f"E2M1 scale bytes, {route}", flush=True)
    dev = torch.device("cuda", 0)
    n, hq = 256, 16
    byte = torch.arange(n, dtype=torch.int32).to(torch.uint8)
    q = torch.full((n, hq, 128), 0.01, dtype=torch.bfloat16)
    cu = torch.arange(n + 1, dtype=torch.int32)
    q2k = torch.zeros(1, n, 1, dtype=torch.int32)
    paged = route == "paged_decode"
    if paged:
        k = torch.full((n, 1, 128, 64), 0x22, dtype=torch.uint8)
        sc = byte.view(n, 1, 1, 1).expand(n, 1, 128, 8).contiguous()
        pt = torch.arange(n, dtype=torch.int32).view(n, 1)
        used = torch.ones(n, dtype=torch.int32)
        kw = dict(page_table=pt, seqused_k=used)
    else:
        k = torch.full((n, 1, 64), 0x22, dtype=torch.uint8)
        sc = byte.view(n, 1, 1).expand(n, 1, 8).contiguous()
        kw = dict(cu_seqlens_k=cu)
    v = k.clone()
    ref_out, ref_lse = oracle.sparse_attention(
        q, k, v, q2k, cu, causal=True, kv_format=synth.KV_E2M1, k_scale=sc, v_scale=sc.clone(),
        k_global_scale=0.5, v_global_scale=2.0, **kw)
    d = {key: val.to(dev) for key, val in kw.items()}
    out, lse = msa.sparse_attention(
        q.to(dev), k.to(dev), v.to(dev), q2k.to(dev), cu.to(dev), d.get("cu_seqlens_k"),
        causal=True, page_table=d.get("page_table"), seqused_k=d.get("seqused_k"),
        return_softmax_lse=True, k_scale=sc.to(dev), v_scale=sc.to(dev), k_global_scale=0.5,
        v_global_scale=2.0, max_seqlen_q=4096 if route == "flat_whole" else 1, max_k_tiles=1)
    torch.cuda.synchronize()
    out, lse = out.cpu().double(), lse.cpu().double()
    # NaN scale bytes are outside the caller contract (the attention kernels
    # are built without NaN semantics): the other 254 bytes must be exact
    nan = torch.isnan(ref_out)
    assert bool(nan[0x7F].all() and nan[0xFF].all()) and int(nan.any(-1).any(-1).sum()) == 2
    keep = torch.ones(n, dtype=torch.bool)
    keep[0x7F] = keep[0xFF] = False
    out, lse, ref_out, ref_lse = out[keep], lse[keep], ref_out[keep], ref_lse[keep]
    assert not torch.isnan(ref_out).any() and not torch.isnan(out).any()
    fin = torch.ones_like(out, dtype=torch.bool)
    # every E4M3 value is a bf16 value: the output is that value to within
    # the bf16 rounding of a softmax weight of one
    assert bool(((out[fin] - ref_out[fin]).abs() <= ref_out[fin].abs() * 2.0 ** -8).all())
    f = ~torch.isnan(ref_lse)
    assert float((lse[f] - ref_lse[f]).abs().max()) <= 1e-3


@pytest.mark.parametrize("hq,hkv,lq,lk,topk,scale,seed,paged", [
    (4, 1, 200, 3000, 4, None, 4, False),    # G = 4: a row's LSE here moved with its slot mates
    (8, 1, 130, 1500, 6, 1.5, 248, False),   # large logit spread: the rescale path
    (16, 2, 64, 1500, 6, 1.5, 256, True),
    (32, 2, 4, 1500, 6, 1.5, 272, True),     # decode tiles
])
def test_row_result_does_not_depend_on_its_slot_mates(msa, hq, hkv, lq, lk, topk, scale, seed,
                                                      paged):
    # the tokens that share a query row's MFMA tile (its slot, or a decode
    # tile) get other selections; every row of the other tokens must come out
    # bitwise unchanged (the first block of a row, and any move of its
    # reference max, send its whole wave down the rescale path)
    p = synth.make_problem("slot_mates", q_lens=[lq], k_lens=[lk], num_qo_heads=hq,
                           num_kv_heads=hkv, topk=topk, paged=paged, seed=seed,
                           softmax_scale=scale, selection="general")
    d = _dev(p)
    out_a, lse_a = gpu_attention(msa, d)
    q2k = p.q2k.clone()
    g = torch.Generator().manual_seed(7)
    nblk = (lk + 127) // 128
    changed = torch.arange(lq) % 2 == 1
    for h in range(hkv):
        for i in torch.nonzero(changed).flatten().tolist():
            ids = sorted(torch.randperm(nblk, generator=g)[:topk].tolist())
            q2k[h, i] = torch.tensor(ids, dtype=torch.int32)
    out_b, lse_b = gpu_attention(msa, d, q2k=q2k.cuda())
    torch.cuda.synchronize()
    keep = ~changed
    assert torch.equal(out_a[keep].cpu(), out_b[keep].cpu())
    assert torch.equal(lse_a[keep].cpu(), lse_b[keep].cpu())
    # outputs near a single V row reach |out| ~ 4 here, where bf16's spacing
    # is 1/32: the tolerance grows by 2^-8 of the largest |out|
    ref_out, ref_lse = oracle_attention(p, q2k=q2k)
    saved = gpu_helpers.OUT_TOL
    gpu_helpers.OUT_TOL = 2e-2 + 2.0 ** -8 * float(ref_out.abs().max())
    try:
        assert_attention_close(out_b, lse_b, ref_out, ref_lse, "changed slot mates")
    finally:
        gpu_helpers.OUT_TOL = saved


def _sub_problem(p, reqs):
    """The requests `reqs` of p (flat layout) as a problem of their own, with
    the same Q, K, V rows and selections."""
    cq = p.cu_seqlens_q.tolist()
    ck = p.cu_seqlens_k.tolist()
    qi = torch.cat([torch.arange(cq[r], cq[r + 1]) for r in reqs])
    ki = torch.cat([torch.arange(ck[r], ck[r + 1]) for r in reqs])
    ql = [cq[r + 1] - cq[r] for r in reqs]
    kl = [ck[r + 1] - ck[r] for r in reqs]
    cu = lambda lens: torch.tensor([0] + torch.cumsum(torch.tensor(lens), 0).tolist(),
                                   dtype=torch.int32)
    return dict(q=p.q[qi], k=p.k[ki], v=p.v[ki], q2k=p.q2k[:, qi].contiguous(),
                cu_q=cu(ql), cu_k=cu(kl), lq=max(ql), T=max((L + 127) // 128 for L in kl)), qi


@pytest.mark.parametrize("fmt,hq,hkv,q_lens,k_lens,splits", [
    (synth.KV_BF16, 16, 2, [100, 50, 7], [700, 300, 900], 0),   # prefill tiles
    (synth.KV_FP8, 8, 2, [100, 50, 7], [700, 300, 900], 0),     # staged fp8 prefill
    (synth.KV_BF16, 16, 1, [1, 1, 1], [3000, 129, 5000], 2),     # decode, fixed split count
    (synth.KV_FP8, 32, 2, [4, 4, 4], [2000, 700, 4000], 1),      # MTP decode
])
def test_request_result_does_not_depend_on_its_batch(msa, fmt, hq, hkv, q_lens, k_lens, splits):
    # a request computed alone, or in another order with other requests,
    # gives bitwise the same rows (decode at a fixed split count)
    p = synth.make_problem("batch_inv", q_lens=q_lens, k_lens=k_lens, num_qo_heads=hq,
                           num_kv_heads=hkv, topk=6, kv_dtype=fmt, seed=250 + hq,
                           selection="decode" if len(set(q_lens)) == 1 else "general")
    outs = {}
    for order in ([0, 1, 2], [0], [2, 0]):
        s, qi = _sub_problem(p, order)
        d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in s.items()}
        out, lse = msa.sparse_attention(d["q"], d["k"], d["v"], d["q2k"], d["cu_q"], d["cu_k"],
                                        causal=True, return_softmax_lse=True,
                                        max_seqlen_q=d["lq"], max_k_tiles=d["T"], splits=splits)
        torch.cuda.synchronize()
        n0 = q_lens[0]
        start = order.index(0)
        first = sum(q_lens[r] for r in order[:start])
        outs[tuple(order)] = (out[first:first + n0].cpu(), lse[first:first + n0].cpu())
    a = outs[(0, 1, 2)]
    for key in ((0,), (2, 0)):
        assert torch.equal(a[0], outs[key][0]) and torch.equal(a[1], outs[key][1]), key
