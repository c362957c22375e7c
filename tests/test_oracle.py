"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the oracle part it checks: a format definition,
an independent library routine, a closed form, brute force on tiny inputs,
or an invariance the method must satisfy.
"""
import itertools
import json
import math
import os
import random

import numpy as np
import pytest
import torch

import oracle
import synth

BLOCK = 128


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# P4: storage formats
# ---------------------------------------------------------------------------

def test_e2m1_table_matches_format_definition(golden_dir):
    ref = _load(golden_dir, "e2m1_table.json")["nibble_to_value"]
    got = oracle.decode_e2m1(torch.arange(16)).tolist()
    for n in range(16):
        assert got[n] == ref[n], n
        assert math.copysign(1.0, got[n]) == math.copysign(1.0, ref[n]) or ref[n] != 0.0


def test_e4m3fn_all_bytes_match_torch_cast():
    b = torch.arange(256, dtype=torch.uint8)
    mine = oracle.decode_e4m3fn(b)
    lib = b.view(torch.float8_e4m3fn).to(torch.float32).to(torch.float64)
    nan_m = torch.isnan(mine)
    assert torch.equal(nan_m, torch.isnan(lib))
    assert torch.equal(mine[~nan_m], lib[~nan_m])
    # signed zeros too
    assert math.copysign(1.0, float(mine[128])) == -1.0


def test_e4m3fn_spec_points(golden_dir):
    pts = _load(golden_dir, "e4m3fn_points.json")["points"]
    got = oracle.decode_e4m3fn(torch.tensor([p["byte"] for p in pts], dtype=torch.uint8))
    for p, g in zip(pts, got.tolist()):
        if p["value"] == "nan":
            assert math.isnan(g)
        else:
            assert g == p["value"] and math.copysign(1, g) == math.copysign(1, p["value"])


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(4096, generator=g) * 100).to(torch.bfloat16)
    x[:4] = torch.tensor([0.0, -0.0, float("inf"), -1e-40])
    assert torch.equal(oracle.decode_bf16(x), x.to(torch.float64))


def test_e2m1_packing_and_block_scale():
    # byte i holds element 2i in its low nibble, 2i+1 in its high nibble
    packed = torch.tensor([[0x21, 0xF7] + [0] * 6], dtype=torch.uint8)  # d = 16
    scale = torch.tensor([[0x38]], dtype=torch.uint8)                     # 1.0
    vals = oracle.dequant_e2m1(packed, scale)[0].tolist()
    assert vals[:4] == [0.5, 1.0, 6.0, -6.0]
    scale2 = torch.tensor([[0x40]], dtype=torch.uint8)                    # 2.0
    assert oracle.dequant_e2m1(packed, scale2)[0, :4].tolist() == [1.0, 2.0, 12.0, -12.0]
    # each 16-wide group uses its own scale
    p = torch.full((1, 16), 0x22, dtype=torch.uint8)                      # all 1.0
    s = torch.tensor([[0x38, 0x30]], dtype=torch.uint8)                   # 1.0, 0.5
    v = oracle.dequant_e2m1(p, s)[0]
    assert v[:16].eq(1.0).all() and v[16:].eq(0.5).all()


def test_quantizer_roundtrip_is_exact_on_grid():
    # values already on the E2M1 x scale grid survive the encoder exactly
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    x = torch.cat([grid, -grid]).view(1, 16) * 0.25
    packed, scl = synth.quantize_e2m1_blocks(x, 1.0)
    back = oracle.dequant_e2m1(packed, scl)
    assert torch.equal(back.to(torch.float32), x)


# ---------------------------------------------------------------------------
# P3: proxy score against brute force
# ---------------------------------------------------------------------------

def _bf(x):
    return [[float(v) for v in row] for row in x]


def _brute_proxy(q, k, q_lens, k_lens, causal):
    """Triple loop over (head, query, block), plain Python floats."""
    total_q, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    T = max((L + BLOCK - 1) // BLOCK for L in k_lens)
    qf = q.to(torch.float64).tolist()
    kf = k.to(torch.float64).tolist()
    out = [[[float("-inf")] * total_q for _ in range(T)] for _ in range(hq)]
    q0 = k0 = 0
    for Lq, Lk in zip(q_lens, k_lens):
        for iq in range(Lq):
            i = q0 + iq
            for h in range(hq):
                for t in range(T):
                    best = float("-inf")
                    for j in range(BLOCK * t, min(BLOCK * t + BLOCK, Lk)):
                        if causal and j > Lk - Lq + iq:
                            continue
                        s = math.fsum(qf[i][h][e] * kf[k0 + j][h // G][e] for e in range(d))
                        best = max(best, s)
                    out[h][t][i] = best
        q0 += Lq
        k0 += Lk
    return torch.tensor(out, dtype=torch.float64)


@pytest.mark.parametrize("causal", [True, False])
def test_proxy_matches_brute_force(causal):
    q_lens, k_lens = [7, 20], [300, 150]
    g = torch.Generator().manual_seed(11)
    d, hq, hkv = 8, 4, 2
    q = torch.randn(sum(q_lens), hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(sum(k_lens), hkv, d, generator=g).to(torch.bfloat16)
    cu_q = torch.tensor([0, 7, 27], dtype=torch.int32)
    cu_k = torch.tensor([0, 300, 450], dtype=torch.int32)
    got = oracle.proxy_score(q, k, cu_q, cu_seqlens_k=cu_k, causal=causal)
    ref = _brute_proxy(q, k, q_lens, k_lens, causal)
    assert got.shape == ref.shape == (hq, 3, 27)
    inf_g, inf_r = torch.isinf(got), torch.isinf(ref)
    assert torch.equal(inf_g, inf_r)
    assert torch.allclose(got[~inf_g], ref[~inf_r], rtol=1e-13, atol=1e-13)
    # request 1 (150 keys) has only 2 blocks: block 2 is -inf for its queries
    assert torch.isinf(got[:, 2, 7:]).all()
    if causal:
        # request 0 query 0 sits at position 293: all 3 blocks visible;
        # request 1 query 0 at 130: block 1 has 3 visible keys
        assert torch.isfinite(got[:, :, 0]).all()
        assert torch.isfinite(got[:, 1, 7]).all()


def test_proxy_paged_equals_flat_and_reduce_heads():
    p = synth.make_problem("t", q_lens=[3, 5], k_lens=[260, 384], num_qo_heads=4,
                           num_kv_heads=2, head_dim=16, paged=True, seed=5,
                           selection="proxy")
    # rebuild the same logical keys in the flat layout
    flat = []
    for b, L in enumerate(p.k_lens):
        pages = p.page_table[b, :(L + 127) // 128].long()
        flat.append(p.k[pages].permute(0, 2, 1, 3).reshape(-1, 2, 16)[:L])
    kf = torch.cat(flat)
    cu_k = torch.tensor([0, 260, 644], dtype=torch.int32)
    a = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, page_table=p.page_table,
                           seqused_k=p.seqused_k)
    b = oracle.proxy_score(p.q, kf, p.cu_seqlens_q, cu_seqlens_k=cu_k)
    assert torch.equal(a, b)
    r = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, page_table=p.page_table,
                           seqused_k=p.seqused_k, reduce_heads=True)
    assert torch.equal(r, a.max(dim=0, keepdim=True).values)
    # decode alignment: query 2 of request 0 sits at 259, sees block 2 key 256..259
    assert torch.isfinite(a[:, 2, 2]).all()


def test_proxy_is_unscaled():
    # the proxy never applies a softmax scale: doubling q doubles the score
    p = synth.make_problem("t", q_lens=[4], k_lens=[200], num_qo_heads=2,
                           num_kv_heads=1, head_dim=16, seed=2, selection="proxy")
    a = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k)
    b = oracle.proxy_score((p.q.float() * 2).to(torch.bfloat16), p.k, p.cu_seqlens_q,
                           cu_seqlens_k=p.cu_seqlens_k)
    fin = torch.isfinite(a)
    assert torch.equal(b[fin], 2 * a[fin]) and torch.equal(fin, torch.isfinite(b))


# ---------------------------------------------------------------------------
# P9: top-K selection
# ---------------------------------------------------------------------------

def _brute_topk(row, topk):
    """Rank counting with explicit comparisons: block t is selected iff fewer
    than topk finite blocks beat it (higher score, or equal score and lower
    id)."""
    T = len(row)
    sel = []
    for t in range(T):
        if not math.isfinite(row[t]):
            continue
        beat = 0
        for u in range(T):
            if u == t or not math.isfinite(row[u]):
                continue
            if row[u] > row[t] or (row[u] == row[t] and u < t):
                beat += 1
        if beat < topk:
            sel.append(t)
    return sel + [-1] * (topk - len(sel))


def test_topk_worked_example(golden_dir):
    ex = _load(golden_dir, "topk_worked.json")
    row = [float(x) for x in ex["scores"]]
    s = torch.tensor(row, dtype=torch.float32).view(1, -1, 1)
    for case in ex["cases"]:
        got = oracle.topk_select(s, case["topk"], 1)[0, 0].tolist()
        assert got == case["q2k"], case


@pytest.mark.parametrize("seed", range(4))
def test_topk_matches_rank_counting(seed):
    rng = random.Random(seed)
    T, n, topk = 37, 40, 8
    rows = []
    for r in range(n):
        kind = r % 4
        if kind == 0:
            row = [rng.gauss(0, 1) for _ in range(T)]
        elif kind == 1:        # heavy ties, signed zeros
            row = [rng.choice([0.0, -0.0, 1.0, -1.0, 2.0]) for _ in range(T)]
        elif kind == 2:        # few finite
            row = [float("-inf")] * T
            for t in rng.sample(range(T), rng.randint(0, 10)):
                row[t] = rng.gauss(0, 1)
        else:                  # all equal
            row = [0.5] * T
        rows.append(row)
    s = torch.tensor(rows, dtype=torch.float32).T.unsqueeze(0)  # (1, T, n)
    got = oracle.topk_select(s, topk, 1)[0]
    for i, row in enumerate(rows):
        r32 = [float(np.float32(x)) for x in row]
        assert got[i].tolist() == _brute_topk(r32, topk), (i, row)
    # all-equal rows pick 0..topk-1
    assert got[3].tolist() == list(range(topk))


def test_topk_modes_map_heads():
    g = torch.Generator().manual_seed(1)
    s = torch.randn(8, 10, 5, generator=g)
    a = oracle.topk_select(s, 3, 2, mode="group")
    ref = oracle.topk_select(s.view(2, 4, 10, 5).amax(dim=1), 3, 2, mode="none")
    assert torch.equal(a, ref)
    one = oracle.topk_select(s[:1], 3, 2)          # H_s == 1 -> shared selection
    assert torch.equal(one[0], one[1])
    assert torch.equal(one[0], oracle.topk_select(s[:1], 3, 1)[0])


# ---------------------------------------------------------------------------
# tile union
# ---------------------------------------------------------------------------

def test_tile_union_brute():
    rows = torch.tensor([[0, 3, -1], [3, 5, 7], [-1, -1, -1], [2, 3, 9]], dtype=torch.int32)
    blocks, masks = oracle.tile_union(rows, num_blocks=8)
    assert blocks == [0, 2, 3, 5, 7]            # 9 is out of range
    assert masks == [0b0001, 0b1000, 0b1011, 0b0010, 0b0010]


# ---------------------------------------------------------------------------
# attention: P1, P2, P5 .. P8, P10 .. P12
# ---------------------------------------------------------------------------

def _all_blocks_q2k(q_lens, k_lens, hkv, causal):
    """Every block a query may see (causally valid), ascending."""
    rows = []
    for Lq, Lk in zip(q_lens, k_lens):
        nblk = (Lk + BLOCK - 1) // BLOCK
        for iq in range(Lq):
            if causal:
                n = min(nblk, (Lk - Lq + iq) // BLOCK + 1)
            else:
                n = nblk
            rows.append(list(range(n)))
    width = max(len(r) for r in rows)
    t = torch.full((hkv, len(rows), width), -1, dtype=torch.int32)
    for i, r in enumerate(rows):
        t[:, i, :len(r)] = torch.tensor(r, dtype=torch.int32)
    return t


@pytest.mark.parametrize("causal", [True, False])
def test_full_selection_equals_dense_sdpa(causal):
    q_lens, k_lens = [130, 64], [300, 64]
    hq, hkv, d = 4, 2, 32
    p = synth.make_problem("t", q_lens=q_lens, k_lens=k_lens, num_qo_heads=hq,
                           num_kv_heads=hkv, head_dim=d, seed=7, selection="proxy")
    q2k = _all_blocks_q2k(q_lens, k_lens, hkv, causal)
    out, lse = oracle.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q,
                                       cu_seqlens_k=p.cu_seqlens_k, causal=causal)
    q0 = k0 = 0
    for Lq, Lk in zip(q_lens, k_lens):
        qq = p.q[q0:q0 + Lq].to(torch.float64).transpose(0, 1)            # (hq, Lq, d)
        kk = p.k[k0:k0 + Lk].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        vv = p.v[k0:k0 + Lk].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        iq = torch.arange(Lq).view(-1, 1)
        j = torch.arange(Lk).view(1, -1)
        mask = (j <= Lk - Lq + iq) if causal else torch.ones(Lq, Lk, dtype=torch.bool)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        logits = (qq @ kk.transpose(1, 2)) * d ** -0.5
        ref_lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
        assert torch.allclose(out[q0:q0 + Lq].transpose(0, 1), ref, atol=1e-12, rtol=1e-12)
        assert torch.allclose(lse[q0:q0 + Lq].T, ref_lse, atol=1e-12, rtol=1e-12)
        q0 += Lq
        k0 += Lk


@pytest.mark.parametrize("tau", [0.5, 2.0])
def test_temperature_lse_full_selection_equals_scaled_logsumexp(tau):
    # every valid block selected: lse_t = logsumexp(tau * z) of the dense
    # masked logits, computed here without the oracle
    q_lens, k_lens = [70, 33], [300, 33]
    hq, hkv, d = 4, 2, 32
    p = synth.make_problem("t", q_lens=q_lens, k_lens=k_lens, num_qo_heads=hq,
                           num_kv_heads=hkv, head_dim=d, seed=8, selection="proxy")
    q2k = _all_blocks_q2k(q_lens, k_lens, hkv, True)
    out, lse, lse_t = oracle.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q,
                                              cu_seqlens_k=p.cu_seqlens_k, causal=True,
                                              softmax_scale=0.3, k_global_scale=0.5,
                                              lse_temperature_scale=tau)
    q0 = k0 = 0
    for Lq, Lk in zip(q_lens, k_lens):
        qq = p.q[q0:q0 + Lq].to(torch.float64).transpose(0, 1)
        kk = p.k[k0:k0 + Lk].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        mask = torch.arange(Lk).view(1, -1) <= Lk - Lq + torch.arange(Lq).view(-1, 1)
        logits = (qq @ kk.transpose(1, 2)) * (0.3 * 0.5)
        ref = torch.logsumexp((tau * logits).masked_fill(~mask, float("-inf")), dim=-1)
        assert torch.allclose(lse_t[q0:q0 + Lq].T, ref, atol=1e-12, rtol=1e-12)
        q0 += Lq
        k0 += Lk
    # tau = 1 is the plain LSE; a single key gives tau * z_j; no key gives -inf
    _, lse1, lse_t1 = oracle.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q,
                                              cu_seqlens_k=p.cu_seqlens_k, causal=True,
                                              lse_temperature_scale=1.0)
    assert torch.allclose(lse1, lse_t1, atol=1e-12, rtol=0)
    one = synth.make_problem("t", q_lens=[1], k_lens=[1], num_qo_heads=2, num_kv_heads=1,
                             head_dim=16, seed=3, selection="proxy")
    q2k1 = torch.tensor([[[0]]], dtype=torch.int32)
    _, l1, lt1 = oracle.sparse_attention(one.q, one.k, one.v, q2k1, one.cu_seqlens_q,
                                         cu_seqlens_k=one.cu_seqlens_k, causal=True,
                                         lse_temperature_scale=tau)
    assert torch.allclose(lt1, tau * l1, atol=1e-12, rtol=0)
    _, _, lt0 = oracle.sparse_attention(one.q, one.k, one.v, -torch.ones_like(q2k1),
                                        one.cu_seqlens_q, cu_seqlens_k=one.cu_seqlens_k,
                                        causal=True, lse_temperature_scale=tau)
    assert torch.isneginf(lt0).all()


def test_empty_selection_gives_zero_and_neg_inf():
    p = synth.make_problem("t", q_lens=[40], k_lens=[500], num_qo_heads=2,
                           num_kv_heads=1, head_dim=16, seed=1, selection="general")
    q2k = p.q2k.clone()
    q2k[:, :10] = -1                       # nothing selected
    q2k[:, 10:20, 0] = 3                   # only block 3 (keys 384..499); query
    q2k[:, 10:20, 1:] = -1                 # positions 460..469 see some of it
    out, lse = oracle.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q,
                                       cu_seqlens_k=p.cu_seqlens_k, causal=True)
    assert (out[:10] == 0).all() and torch.isneginf(lse[:10]).all()
    assert torch.isfinite(lse[10:20]).all()
    # a selection lying entirely above the causal limit is empty too:
    # 1 query at position 99 of a 200-key sequence selecting only block 1
    p2 = synth.make_problem("t", q_lens=[1], k_lens=[100], num_qo_heads=2,
                            num_kv_heads=1, head_dim=16, seed=1, selection="general")
    k = torch.cat([p2.k, p2.k]); v = torch.cat([p2.v, p2.v])
    cu_k = torch.tensor([0, 200], dtype=torch.int32)
    q2k2 = torch.tensor([[[1]]], dtype=torch.int32)
    # Lq = 1 right-aligned at 199 sees block 1; to make it causally empty use
    # a longer query run whose first query sits at 100 -> block 1 starts at 128
    o2, l2 = oracle.sparse_attention(p2.q, k, v, q2k2, p2.cu_seqlens_q,
                                     cu_seqlens_k=cu_k, causal=True)
    assert torch.isfinite(l2).all()
    q3 = p2.q.repeat(100, 1, 1)            # 100 queries at positions 100..199
    cu_q3 = torch.tensor([0, 100], dtype=torch.int32)
    q2k3 = torch.ones((1, 100, 1), dtype=torch.int32)
    o3, l3 = oracle.sparse_attention(q3, k, v, q2k3, cu_q3, cu_seqlens_k=cu_k, causal=True)
    assert torch.isneginf(l3[:28]).all() and (o3[:28] == 0).all()   # positions 100..127
    assert torch.isfinite(l3[28:]).all()


def test_single_key_closed_form():
    # one allowed key j: out = v_gs * v_j, lse = z_j (closed form)
    p = synth.make_problem("t", q_lens=[1], k_lens=[129], num_qo_heads=3,
                           num_kv_heads=1, head_dim=16, seed=4, selection="general")
    # the query sits at position 128; block 1 holds exactly key 128
    q2k = torch.tensor([[[1, -1]]], dtype=torch.int32)
    out, lse = oracle.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q,
                                       cu_seqlens_k=p.cu_seqlens_k, causal=True,
                                       softmax_scale=0.3, k_global_scale=0.5,
                                       v_global_scale=2.0)
    kj = p.k[128, 0].to(torch.float64)
    vj = p.v[128, 0].to(torch.float64)
    for h in range(3):
        z = 0.3 * 0.5 * float(p.q[0, h].to(torch.float64) @ kj)
        assert abs(float(lse[0, h]) - z) < 1e-12
        assert torch.allclose(out[0, h], 2.0 * vj, atol=0, rtol=0)


def test_attention_worked_examples(golden_dir):
    ex = _load(golden_dir, "attention_worked.json")
    d = 8
    for case in ex["cases"]:
        n = len(case["logits"])
        q = torch.zeros(1, 1, d, dtype=torch.bfloat16); q[0, 0, 0] = 1
        k = torch.zeros(n, 1, d, dtype=torch.bfloat16)
        v = torch.zeros(n, 1, d, dtype=torch.bfloat16)
        for j, z in enumerate(case["logits"]):
            k[j, 0, 0] = z
            v[j, 0, j] = 1
        out, lse = oracle.sparse_attention(
            q, k, v, torch.zeros(1, 1, 1, dtype=torch.int32),
            torch.tensor([0, 1], dtype=torch.int32),
            cu_seqlens_k=torch.tensor([0, n], dtype=torch.int32),
            causal=False, softmax_scale=1.0)
        assert abs(float(lse[0, 0]) - case["lse"]) < 1e-15
        for j, w in enumerate(case["weights"]):
            assert abs(float(out[0, 0, j]) - w) < 1e-15


def _to_flat(p):
    """Same logical K/V in the flat layout."""
    ks, vs = [], []
    for b, L in enumerate(p.k_lens):
        pages = p.page_table[b, :(L + 127) // 128].long()
        hkv, d = p.k.shape[1], p.k.shape[3]
        ks.append(p.k[pages].permute(0, 2, 1, 3).reshape(-1, hkv, d)[:L])
        vs.append(p.v[pages].permute(0, 2, 1, 3).reshape(-1, hkv, d)[:L])
    cu = [0]
    for L in p.k_lens:
        cu.append(cu[-1] + L)
    return torch.cat(ks), torch.cat(vs), torch.tensor(cu, dtype=torch.int32)


def test_paged_equals_flat_under_two_page_tables():
    base = dict(q_lens=[3, 1, 4], k_lens=[700, 129, 256], num_qo_heads=4,
                num_kv_heads=2, head_dim=16, paged=True, selection="general")
    p1 = synth.make_problem("a", seed=8, **base)
    kf, vf, cu_k = _to_flat(p1)
    ref = oracle.sparse_attention(p1.q, kf, vf, p1.q2k, p1.cu_seqlens_q,
                                  cu_seqlens_k=cu_k, causal=True)
    got = oracle.sparse_attention(p1.q, p1.k, p1.v, p1.q2k, p1.cu_seqlens_q,
                                  page_table=p1.page_table, seqused_k=p1.seqused_k,
                                  causal=True)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    # a second, different page assignment of the same logical cache
    npg = p1.k.shape[0]
    perm = torch.randperm(npg, generator=torch.Generator().manual_seed(99))
    inv = torch.empty_like(perm); inv[perm] = torch.arange(npg)
    k2 = torch.empty_like(p1.k); v2 = torch.empty_like(p1.v)
    k2[perm] = p1.k; v2[perm] = p1.v
    pt2 = torch.where(p1.page_table >= 0, perm[p1.page_table.clamp(min=0).long()].to(torch.int32),
                      p1.page_table)
    got2 = oracle.sparse_attention(p1.q, k2, v2, p1.q2k, p1.cu_seqlens_q,
                                   page_table=pt2, seqused_k=p1.seqused_k, causal=True)
    assert torch.equal(ref[0], got2[0]) and torch.equal(ref[1], got2[1])


def test_gqa_equals_replicated_mha():
    p = synth.make_problem("t", q_lens=[50, 20], k_lens=[300, 200], num_qo_heads=6,
                           num_kv_heads=2, head_dim=16, seed=9, selection="general")
    G = 3
    a = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                cu_seqlens_k=p.cu_seqlens_k, causal=True)
    k6 = p.k.repeat_interleave(G, dim=1)
    v6 = p.v.repeat_interleave(G, dim=1)
    q2k6 = p.q2k.repeat_interleave(G, dim=0)
    b = oracle.sparse_attention(p.q, k6, v6, q2k6, p.cu_seqlens_q,
                                cu_seqlens_k=p.cu_seqlens_k, causal=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_scale_invariances():
    p = synth.make_problem("t", q_lens=[30], k_lens=[400], num_qo_heads=2,
                           num_kv_heads=1, head_dim=16, seed=10, selection="general")
    kw = dict(cu_seqlens_k=p.cu_seqlens_k, causal=True)
    base = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                   softmax_scale=0.2, k_global_scale=1.5, **kw)
    moved = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                    softmax_scale=0.2 * 3, k_global_scale=1.5 / 3, **kw)
    assert torch.allclose(base[0], moved[0], atol=1e-12)
    fin = torch.isfinite(base[1])
    assert torch.allclose(base[1][fin], moved[1][fin], atol=1e-12)
    vs = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                 softmax_scale=0.2, k_global_scale=1.5,
                                 v_global_scale=-2.5, **kw)
    assert torch.allclose(vs[0], -2.5 * base[0], atol=1e-12)
    assert torch.equal(torch.isfinite(vs[1]), fin)
    assert torch.equal(vs[1][fin], base[1][fin])
    # default softmax scale is head_dim ** -0.5
    dflt = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q, **kw)
    expl = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                   softmax_scale=0.25, **kw)
    assert torch.equal(dflt[0], expl[0])


def test_lse_merge_of_disjoint_splits_equals_unsplit():
    p = synth.make_problem("t", q_lens=[20], k_lens=[1000], num_qo_heads=2,
                           num_kv_heads=1, head_dim=16, seed=12, selection="general",
                           topk=8)
    kw = dict(cu_seqlens_k=p.cu_seqlens_k, causal=True)
    full = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q, **kw)
    rng = random.Random(5)
    for nsplit in (2, 3, 5):
        owner = {t: rng.randrange(nsplit) for t in range(8)}
        parts = []
        for s in range(nsplit):
            q2k_s = p.q2k.clone()
            for t, o in owner.items():
                if o != s:
                    q2k_s[q2k_s == t] = -1
            parts.append(oracle.sparse_attention(p.q, p.k, p.v, q2k_s, p.cu_seqlens_q, **kw))
        o, l = oracle.lse_merge(parts)
        fin = torch.isfinite(full[1])
        assert torch.equal(torch.isfinite(l), fin)
        assert torch.allclose(l[fin], full[1][fin], atol=1e-12)
        assert torch.allclose(o, full[0], atol=1e-12)


def test_decode_alignment_right_aligned():
    # 4 decode tokens at positions Lk-4+i: token i equals a one-token
    # request over the first Lk-3+i keys with the same selection
    p = synth.make_problem("t", q_lens=[4], k_lens=[300], num_qo_heads=2,
                           num_kv_heads=1, head_dim=16, paged=True, seed=13,
                           selection="decode", topk=3)
    full = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                   page_table=p.page_table, seqused_k=p.seqused_k,
                                   causal=True)
    for i in range(4):
        one = oracle.sparse_attention(
            p.q[i:i + 1], p.k, p.v, p.q2k[:, i:i + 1], torch.tensor([0, 1], dtype=torch.int32),
            page_table=p.page_table, seqused_k=torch.tensor([300 - 3 + i], dtype=torch.int32),
            causal=True)
        # same key set; only the summation order may differ
        assert torch.allclose(one[0][0], full[0][i], atol=1e-13, rtol=0)
        assert torch.allclose(one[1][0], full[1][i], atol=1e-13, rtol=0)
    # the four tokens differ (the last page gains one key per token)
    assert not torch.equal(full[0][0], full[0][3])


def test_q2k_is_read_as_a_set():
    p = synth.make_problem("t", q_lens=[25], k_lens=[600], num_qo_heads=2,
                           num_kv_heads=1, head_dim=16, seed=14, selection="general",
                           topk=4)
    kw = dict(cu_seqlens_k=p.cu_seqlens_k, causal=True)
    base = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q, **kw)
    perm = p.q2k.flip(-1)
    dup = torch.cat([p.q2k, p.q2k], dim=-1)
    for alt in (perm, dup):
        o, l = oracle.sparse_attention(p.q, p.k, p.v, alt, p.cu_seqlens_q, **kw)
        assert torch.equal(o, base[0]) and torch.equal(l, base[1])


def test_e2m1_paged_global_scales():
    # packed-E2M1 K/V: equal to bf16-free fp64 attention over the decoded
    # values with K's global scale folded into the logit scale
    p = synth.make_problem("t", q_lens=[1, 1], k_lens=[300, 140], num_qo_heads=4,
                           num_kv_heads=1, head_dim=32, paged=True, kv_dtype="e2m1x2",
                           seed=15, selection="decode", topk=2, k_global_scale=0.5,
                           v_global_scale=2.0)
    got = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                  page_table=p.page_table, seqused_k=p.seqused_k,
                                  causal=True, kv_format="e2m1x2", k_scale=p.k_scale,
                                  v_scale=p.v_scale, k_global_scale=0.5, v_global_scale=2.0)
    kd = oracle.dequant_e2m1(p.k, p.k_scale)
    vd = oracle.dequant_e2m1(p.v, p.v_scale)
    for b, L in enumerate(p.k_lens):
        sel = [t for t in p.q2k[0, b].tolist() if t >= 0]
        keys = torch.cat([kd[int(p.page_table[b, t]), 0] for t in sel])
        vals = torch.cat([vd[int(p.page_table[b, t]), 0] for t in sel])
        pos = torch.cat([torch.arange(128 * t, 128 * t + 128) for t in sel])
        ok = pos < L
        keys, vals = keys[ok], vals[ok]
        for h in range(4):
            z = (32 ** -0.5) * 0.5 * (p.q[b, h].to(torch.float64) @ keys.T)
            w = torch.softmax(z, dim=0)
            assert torch.allclose(got[0][b, h], 2.0 * (w @ vals), atol=1e-12)
            assert abs(float(got[1][b, h]) - float(torch.logsumexp(z, 0))) < 1e-12


def test_synthetic_selection_recipes():
    # flat prefill tiny workload: own block + up to 3 earlier, ascending
    p = synth.workload(synth.WORKLOADS[0])
    q2k = p.q2k[0]
    for i in (0, 127, 128, 300, 1023):
        row = q2k[i].tolist()
        c = i // 128
        valid = [x for x in row if x >= 0]
        assert valid == sorted(set(valid)) and c in valid and max(valid) == c
        assert len(valid) == min(4, c + 1)


# ---------------------------------------------------------------------------
# QSA indexed attention (qsa page)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hkv", [(12, 1), (24, 2)])
def test_qsa_causal_indices_equal_dense_causal_sdpa(hq, hkv):
    # the qsa page's example pattern (every earlier token of the query's own
    # packed sequence) must reproduce dense causal attention of each sequence
    lens = [9, 14]
    p = synth.make_qsa_problem("qsa", lens, hq, hkv, width=16, seed=3, mode="causal")
    out, lse = oracle.qsa_indexed_attention(p.q, p.k, p.v, p.indices)
    c = 0
    for L in lens:
        qq = p.q[c:c + L].to(torch.float64).transpose(0, 1)
        kk = p.k[c:c + L].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        vv = p.v[c:c + L].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        mask = torch.ones(L, L, dtype=torch.bool).tril()
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        logits = (qq @ kk.transpose(1, 2)) * 256 ** -0.5
        ref_lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
        assert torch.allclose(out[c:c + L].transpose(0, 1), ref, atol=1e-12, rtol=1e-12)
        assert torch.allclose(lse[:, c:c + L], ref_lse, atol=1e-12, rtol=1e-12)
        c += L


def test_qsa_empty_single_and_set_semantics():
    p = synth.make_qsa_problem("qsa", [12], 12, 1, width=8, seed=4)
    idx = p.indices.clone()
    idx[0] = -1                                        # empty: 0 and -inf
    idx[5] = torch.tensor([3, -1, -1, -1, -1, -1, -1, -1])   # one key: v_3, lse = z_3
    out, lse = oracle.qsa_indexed_attention(p.q, p.k, p.v, idx)
    assert (out[0] == 0).all() and torch.isneginf(lse[:, 0]).all()
    v3 = p.v[3, 0].to(torch.float64)
    for h in range(12):
        assert torch.equal(out[5, h], v3)
        z = (p.q[5, h].to(torch.float64) @ p.k[3, 0].to(torch.float64)) * 256 ** -0.5
        assert abs(float(lse[h, 5] - z)) < 1e-12
    # a row is a set: order and extra padding do not matter
    g = torch.Generator().manual_seed(9)
    perm = idx.clone()
    for i in range(perm.shape[0]):
        perm[i] = perm[i][torch.randperm(perm.shape[1], generator=g)]
    wide = torch.cat([perm, torch.full((perm.shape[0], 4), -1, dtype=torch.int32)], dim=1)
    out2, lse2 = oracle.qsa_indexed_attention(p.q, p.k, p.v, wide)
    assert torch.equal(out, out2) or torch.allclose(out, out2, atol=1e-14, rtol=0)
    assert torch.allclose(lse, lse2, atol=1e-14, rtol=0)


def test_f16_decode_all_bit_patterns_match_torch_cast():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.float16)
    got = oracle.decode_f16(x)
    ref = x.to(torch.float64)
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(got[~nan], ref[~nan])
    assert torch.equal(torch.signbit(got[~nan]), torch.signbit(ref[~nan]))   # -0 stays -0


def test_fp16_full_selection_equals_dense_sdpa():
    q_lens, k_lens = [70, 33], [200, 33]
    hq, hkv, d = 4, 2, 32
    p = synth.make_problem("t16", q_lens=q_lens, k_lens=k_lens, num_qo_heads=hq,
                           num_kv_heads=hkv, head_dim=d, seed=8, selection="proxy",
                           kv_dtype=synth.KV_F16)
    assert p.q.dtype == torch.float16 and p.k.dtype == torch.float16
    q2k = _all_blocks_q2k(q_lens, k_lens, hkv, True)
    out, lse = oracle.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q,
                                       cu_seqlens_k=p.cu_seqlens_k, causal=True,
                                       kv_format=synth.KV_F16)
    q0 = k0 = 0
    for Lq, Lk in zip(q_lens, k_lens):
        qq = p.q[q0:q0 + Lq].to(torch.float64).transpose(0, 1)
        kk = p.k[k0:k0 + Lk].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        vv = p.v[k0:k0 + Lk].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        iq = torch.arange(Lq).view(-1, 1)
        mask = torch.arange(Lk).view(1, -1) <= Lk - Lq + iq
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        assert torch.allclose(out[q0:q0 + Lq].transpose(0, 1), ref, atol=1e-12, rtol=1e-12)
        q0 += Lq
        k0 += Lk


def test_qsa_bitmap_full_map_equals_dense_sdpa():
    # every block selected: plain (non-causal) attention over all packed
    # tokens, including the partial last block
    p = synth.make_qsa_problem("qsab", [14], 12, 1, width=8, seed=6)
    bitmap = torch.ones(14, 4, dtype=torch.uint8)     # ceil(14 / 4) blocks
    out, lse = oracle.qsa_bitmap_attention(p.q, p.k, p.v, bitmap)
    qq = p.q.to(torch.float64).transpose(0, 1)
    kk = p.k.to(torch.float64).repeat_interleave(12, 1).transpose(0, 1)
    vv = p.v.to(torch.float64).repeat_interleave(12, 1).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)
    ref_lse = torch.logsumexp((qq @ kk.transpose(1, 2)) * 256 ** -0.5, dim=-1)
    assert torch.allclose(out.transpose(0, 1), ref, atol=1e-12, rtol=1e-12)
    assert torch.allclose(lse, ref_lse, atol=1e-12, rtol=1e-12)


def test_qsa_bitmap_indices_layout():
    bm = torch.tensor([[0, 1, 0, 1], [0, 0, 0, 0], [1, 0, 0, 0]], dtype=torch.uint8)
    idx = oracle.qsa_bitmap_indices(bm, num_kv_tokens=14)
    assert idx[0].tolist()[:6] == [4, 5, 6, 7, 12, 13] and (idx[0, 6:] == -1).all()
    assert (idx[1] == -1).all()
    assert idx[2].tolist()[:4] == [0, 1, 2, 3]


# ---------------------------------------------------------------------------
# head reduction and the score -> KV-head mapping (msa_proxy_score page,
# Parameters: reduce_heads; msa_sparse_attention page, Parameters: q2k_indices)
# ---------------------------------------------------------------------------

def test_reduce_heads_hand_built():
    # 3 heads, 2 blocks, 2 queries; the maximum sits in a different head for
    # every (block, query), so taking any single head, a mean, or the wrong
    # axis gives a different tensor
    s = torch.tensor([[[1.0, -5.0], [0.0, 2.0]],
                      [[3.0, -6.0], [float("-inf"), 1.0]],
                      [[2.0, -4.0], [-1.0, 7.0]]], dtype=torch.float64)
    want = torch.tensor([[[3.0, -4.0], [0.0, 7.0]]], dtype=torch.float64)
    assert torch.equal(oracle.reduce_heads(s), want)
    # all -inf across heads stays -inf
    z = torch.full((2, 1, 1), float("-inf"))
    assert oracle.reduce_heads(z).item() == float("-inf")


def _brute_group_topk(s, hkv, topk, heads_of):
    """Per KV head g: max over the score heads heads_of(g), then rank counting."""
    hs, T, n = len(s), len(s[0]), len(s[0][0])
    out = []
    for g in range(hkv):
        rows = []
        for i in range(n):
            row = []
            for t in range(T):
                m = float("-inf")
                for h in heads_of(g):
                    if s[h][t][i] > m:
                        m = s[h][t][i]
                row.append(m)
            rows.append(_brute_topk(row, topk))
        out.append(rows)
    return out


@pytest.mark.parametrize("G,hkv", [(4, 3), (2, 2), (3, 1)])
def test_group_and_all_modes_match_brute_force(G, hkv):
    rng = random.Random(G * 10 + hkv)
    hs, T, n, topk = G * hkv, 9, 6, 3
    s = [[[float(np.float32(rng.gauss(0, 1))) for _ in range(n)] for _ in range(T)]
         for _ in range(hs)]
    for h in range(hs):                           # some -inf blocks
        s[h][T - 1][0] = float("-inf")
    st = torch.tensor(s, dtype=torch.float32)
    got = oracle.topk_select(st, topk, hkv, mode="group").tolist()
    assert got == _brute_group_topk(s, hkv, topk, lambda g: range(g * G, g * G + G))
    got_all = oracle.topk_select(st, topk, hkv, mode="all").tolist()
    assert got_all == _brute_group_topk(s, hkv, topk, lambda g: range(hs))
    # auto picks "group" for H_s = G * Hkv > Hkv
    if G > 1:
        assert oracle.topk_select(st, topk, hkv).tolist() == got


def test_group_mode_uses_contiguous_heads():
    # Hq = 4, Hkv = 2: query heads 0, 1 belong to KV head 0 (h // G), not
    # heads 0, 2 (h % Hkv).  Head 1 alone scores block 2 highest, so KV head 0
    # must select block 2 and KV head 1 must not; taking one head per group
    # (the first) would not select it either.
    s = torch.full((4, 4, 1), 0.0)
    s[:, 0, 0] = 1.0                     # every head likes block 0
    s[1, 2, 0] = 9.0                     # only head 1 likes block 2
    s[3, 3, 0] = 5.0                     # only head 3 likes block 3
    got = oracle.topk_select(s, 2, 2, mode="group")[:, 0].tolist()
    assert got == [[0, 2], [0, 3]]
    # "all": the max over the four heads, shared by both KV heads
    got = oracle.topk_select(s, 2, 2, mode="all")[:, 0].tolist()
    assert got == [[2, 3], [2, 3]]


# ---------------------------------------------------------------------------
# q_offset (msa_proxy_score page, Parameters: q_offset; msa_sparse_attention
# page, Parameters: q_offset).  Reading: the queries' causal positions (an
# int o: o + iq; a tensor: each row's own position).  The reading itself is
# unpinned; these pin that the oracle applies it as stated.
# ---------------------------------------------------------------------------

def _positions(q_lens, k_lens, q_offset):
    pos = []
    for b, (Lq, Lk) in enumerate(zip(q_lens, k_lens)):
        q0 = sum(q_lens[:b])
        for iq in range(Lq):
            if q_offset is None:
                pos.append(Lk - Lq + iq)
            elif isinstance(q_offset, int):
                pos.append(q_offset + iq)
            else:
                pos.append(int(q_offset[q0 + iq]))
    return pos


def test_q_offset_right_alignment_tensor_is_the_default():
    q_lens, k_lens = [70, 5], [300, 260]
    p = synth.make_problem("t", q_lens=q_lens, k_lens=k_lens, num_qo_heads=4, num_kv_heads=2,
                           head_dim=16, seed=12, selection="general", topk=3)
    qo = torch.tensor(_positions(q_lens, k_lens, None), dtype=torch.int32)
    a = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                cu_seqlens_k=p.cu_seqlens_k, causal=True)
    b = oracle.sparse_attention(p.q, p.k, p.v, p.q2k, p.cu_seqlens_q,
                                cu_seqlens_k=p.cu_seqlens_k, causal=True, q_offset=qo)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    s0 = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k, causal=True)
    s1 = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q, cu_seqlens_k=p.cu_seqlens_k, causal=True,
                            q_offset=qo)
    assert torch.equal(s0, s1)


@pytest.mark.parametrize("form", ["int", "tensor"])
def test_q_offset_proxy_matches_brute_force(form):
    # queries at the given positions, including ones before every key (all
    # -inf) and past the sequence end (every key visible)
    q_lens, k_lens = [6, 9], [300, 150]
    g = torch.Generator().manual_seed(21)
    d, hq, hkv = 8, 4, 2
    q = torch.randn(sum(q_lens), hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(sum(k_lens), hkv, d, generator=g).to(torch.bfloat16)
    cu_q = torch.tensor([0, 6, 15], dtype=torch.int32)
    cu_k = torch.tensor([0, 300, 450], dtype=torch.int32)
    qo = 129 if form == "int" else torch.tensor([-1, 0, 127, 128, 290, 1000,
                                                  -5, 3, 40, 127, 128, 129, 140, 149, 700],
                                                 dtype=torch.int32)
    pos = _positions(q_lens, k_lens, qo)
    got = oracle.proxy_score(q, k, cu_q, cu_seqlens_k=cu_k, causal=True, q_offset=qo)
    G, T = hq // hkv, 3
    qf, kf = q.to(torch.float64).tolist(), k.to(torch.float64).tolist()
    q0 = k0 = 0
    for Lq, Lk in zip(q_lens, k_lens):
        for iq in range(Lq):
            i = q0 + iq
            for h in range(hq):
                for t in range(T):
                    best = float("-inf")
                    for j in range(BLOCK * t, min(BLOCK * t + BLOCK, Lk)):
                        if j <= pos[i]:
                            best = max(best, math.fsum(qf[i][h][e] * kf[k0 + j][h // G][e]
                                                       for e in range(d)))
                    ref = best
                    assert (got[h, t, i] == ref) if ref == float("-inf") else \
                        abs(float(got[h, t, i]) - ref) <= 1e-12, (h, t, i)
        q0 += Lq
        k0 += Lk
    if form == "tensor":
        assert torch.isinf(got[:, :, 0]).all() and torch.isinf(got[:, :, 6]).all()


def test_q_offset_full_selection_equals_dense_sdpa():
    # every block selected: attention equals SDPA with the mask j <= pos(i),
    # j < Lk built here; a row positioned before every key is empty (0, -inf)
    q_lens, k_lens = [40, 20], [300, 140]
    hq, hkv, d = 4, 2, 32
    p = synth.make_problem("t", q_lens=q_lens, k_lens=k_lens, num_qo_heads=hq,
                           num_kv_heads=hkv, head_dim=d, seed=23, selection="proxy")
    g = torch.Generator().manual_seed(5)
    qo = torch.randint(-3, 320, (sum(q_lens),), generator=g, dtype=torch.int32)
    qo[0] = -1
    q2k = _all_blocks_q2k(q_lens, k_lens, hkv, False)
    out, lse = oracle.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q,
                                       cu_seqlens_k=p.cu_seqlens_k, causal=True, q_offset=qo)
    q0 = k0 = 0
    for Lq, Lk in zip(q_lens, k_lens):
        qq = p.q[q0:q0 + Lq].to(torch.float64).transpose(0, 1)
        kk = p.k[k0:k0 + Lk].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        vv = p.v[k0:k0 + Lk].to(torch.float64).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        pos = qo[q0:q0 + Lq].to(torch.int64).view(-1, 1)
        mask = torch.arange(Lk).view(1, -1) <= pos
        nonempty = mask.any(dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq[:, nonempty], kk, vv, attn_mask=mask[nonempty])
        logits = (qq @ kk.transpose(1, 2)) * d ** -0.5
        ref_lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
        o = out[q0:q0 + Lq].transpose(0, 1)
        assert torch.allclose(o[:, nonempty], ref, atol=1e-12, rtol=1e-12)
        assert (o[:, ~nonempty] == 0).all()
        assert torch.allclose(lse[q0:q0 + Lq].T[:, nonempty], ref_lse[:, nonempty],
                              atol=1e-12, rtol=1e-12)
        assert torch.isneginf(lse[q0:q0 + Lq].T[:, ~nonempty]).all()
        q0 += Lq
        k0 += Lk
    assert torch.isneginf(lse[0]).all()
