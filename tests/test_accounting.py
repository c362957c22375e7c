"""Host-side work accounting used by bench.py, against brute-force counts on
small random problems (CPU only)."""
import random

import pytest
import torch

from block_sparse_top_msa_amd import accounting as acc


def _problem(seed, q_lens, k_lens, hkv, topk):
    rng = random.Random(seed)
    rows = []
    for g in range(hkv):
        for lq, lk in zip(q_lens, k_lens):
            nblk = (lk + 127) // 128
            for _ in range(lq):
                # some ids past the last block and some -1 padding
                n = rng.randint(0, topk)
                ids = sorted(rng.sample(range(nblk + 2), min(n, nblk + 2)))
                rows.append(ids + [-1] * (topk - len(ids)))
    q2k = torch.tensor(rows, dtype=torch.int32).view(hkv, sum(q_lens), topk)
    cu = torch.tensor([0] + list(torch.cumsum(torch.tensor(q_lens), 0).tolist()))
    return q2k, cu, torch.tensor(k_lens)


def _brute_slot_blocks(q2k, q_lens, k_lens, G, tile_tokens):
    hkv = q2k.shape[0]
    n = 0
    for g in range(hkv):
        q0 = 0
        for lq, lk in zip(q_lens, k_lens):
            nblk = (lk + 127) // 128
            for j in range(0, lq, tile_tokens):
                toks = range(j, min(lq, j + tile_tokens))
                n_slots = (tile_tokens * G + 31) // 32
                for s in range(n_slots):
                    blocks = set()
                    for t in toks:
                        t_in = t - j
                        if G * t_in <= 32 * s + 31 and G * t_in + G - 1 >= 32 * s:
                            blocks |= {x for x in q2k[g, q0 + t].tolist() if 0 <= x < nblk}
                    n += len(blocks)
            q0 += lq
    return n


@pytest.mark.parametrize("hq,hkv", [(8, 1), (16, 2), (4, 4), (32, 2), (64, 1), (6, 3), (128, 1)])
def test_prefill_slot_blocks_match_brute_force(hq, hkv):
    q_lens, k_lens = [70, 5, 129], [900, 130, 2000]
    q2k, cu, lk = _problem(hq + hkv, q_lens, k_lens, hkv, 6)
    G = hq // hkv
    tt = acc.prefill_tile_tokens(hq, hkv, 6)
    assert tt == max(1, min(64, 256 // G))
    got = acc.prefill_slot_blocks(q2k, cu, lk, hq, tt)
    assert got == _brute_slot_blocks(q2k, q_lens, k_lens, G, tt)


def test_prefill_slot_blocks_closed_forms():
    # every token of a request selects the same 5 blocks: each used slot of
    # each tile computes exactly those 5
    hq, hkv, lq = 16, 2, 100                       # G = 8: 4 tokens per slot, 32 per tile
    q2k = torch.tensor([0, 3, 4, 7, 9, -1], dtype=torch.int32).repeat(hkv, lq, 1)
    cu, lk = torch.tensor([0, lq]), torch.tensor([1280])
    slots = sum((min(32, lq - j) + 3) // 4 for j in range(0, lq, 32))   # 8 + 8 + 8 + 1
    assert acc.prefill_slot_blocks(q2k, cu, lk, hq, 32) == hkv * slots * 5
    assert acc.prefill_executed_flops(q2k, cu, lk, hq, 32) == hkv * slots * 5 * 32 * 128 * 128 * 4
    # a union never holds blocks past the request's last one
    assert acc.prefill_slot_blocks(q2k, cu, torch.tensor([700]), hq, 32) == hkv * slots * 3
    # the tile width shrinks when tokens x topk passes the union list
    assert acc.prefill_tile_tokens(16, 2, 64) == 8
    assert acc.prefill_tile_tokens(2, 2, 16) == 32


def test_attended_keys_and_flops_match_brute_force():
    q_lens, k_lens, hkv, hq = [40, 3, 90], [300, 129, 1000], 2, 8
    q2k, cu, lk = _problem(5, q_lens, k_lens, hkv, 5)
    got = acc.attended_keys(q2k, cu, lk, causal=True)
    ref = torch.zeros_like(got)
    q0 = 0
    for lq, L in zip(q_lens, k_lens):
        nblk = (L + 127) // 128
        for i in range(lq):
            pos = L - lq + i
            for g in range(hkv):
                n = 0
                for x in q2k[g, q0 + i].tolist():
                    if 0 <= x < nblk:
                        n += max(0, min(128 * x + 128, L, pos + 1) - 128 * x)
                ref[g, q0 + i] = n
        q0 += lq
    assert torch.equal(got, ref)
    assert acc.attention_flops(q2k, cu, lk, hq) == int(ref.sum()) * (hq // hkv) * 4 * 128


def test_decode_kv_bytes_match_brute_force():
    q_lens, k_lens, hkv, T = [1, 4, 2], [300, 129, 5000], 2, 40
    q2k, cu, lk = _problem(9, q_lens, k_lens, hkv, 7)
    ref = 0
    for g in range(hkv):
        q0 = 0
        for lq, L in zip(q_lens, k_lens):
            nblk = (L + 127) // 128
            used = {x for i in range(lq) for x in q2k[g, q0 + i].tolist() if 0 <= x < nblk}
            ref += sum(min(128, L - 128 * x) for x in used)
            q0 += lq
    for fmt, per in acc.BYTES_PER_TOKEN_SIDE.items():
        assert acc.decode_kv_bytes(q2k, cu, lk, fmt, T) == ref * 2 * per


def test_proxy_flops_match_brute_force():
    cu, lk = torch.tensor([0, 5, 5, 12]), torch.tensor([9, 4, 7])
    pairs = 0
    for b, (lq, L) in enumerate(zip([5, 0, 7], [9, 4, 7])):
        for i in range(lq):
            pairs += sum(1 for j in range(L) if j <= L - lq + i)
    assert acc.proxy_flops(cu, lk, 3, head_dim=128) == pairs * 3 * 2 * 128
    assert acc.proxy_flops(cu, lk, 3, head_dim=128, causal=False) == (5 * 9 + 7 * 7) * 3 * 2 * 128


def _qsa_brute(G, hkv, rows, chunks_per_token, bitmap_direct=False):
    """The QSA kernel's work by enumeration: rows = per-token sets of keys."""
    tt = min(16, 128 // G)
    total = 0
    for t0 in range(0, len(rows), tt):
        tile = rows[t0:t0 + tt]
        union = set().union(*tile)
        listed = sum(len(r) for r in tile)
        slots = -(-len(tile) * G // 16)
        base = 0 if bitmap_direct or not union else min(union)
        windows = {}
        for k in union:
            windows[(k - base) // 16384] = windows.get((k - base) // 16384, 0) + 1
        wide = bool(union) and (max(union) - base) // 16384 + 1 > 64
        if union and (wide or 5 * len(union) * -(-slots // 4) > 8 * listed):
            total += sum(chunks_per_token(i) for i in range(t0, t0 + len(tile))) * 16 * 32
        else:
            total += slots * sum(-(-n // 32) for n in windows.values()) * 16 * 32
    return total * 256 * 4 * hkv


@pytest.mark.parametrize("hq,hkv", [(12, 1), (24, 2), (16, 1), (4, 1), (5, 1)])
def test_qsa_executed_matches_enumeration(hq, hkv):
    rng = random.Random(hq * 10 + hkv)
    G = hq // hkv
    T, W = 45, 64
    rows, ind = [], torch.full((T, W), -1, dtype=torch.int32)
    for i in range(T):
        kind = rng.random()
        if kind < 0.1:
            r = []                                                 # empty row
        elif kind < 0.4:
            r = rng.sample(range(0, 20000 if i % 2 else 2000000), rng.randint(1, W))   # wide
        else:
            r = rng.sample(range(0, 80), rng.randint(1, W))        # dense, shared
        rows.append(set(r))
        ind[i, :len(r)] = torch.tensor(r, dtype=torch.int32)
    flops, shared, token = acc.qsa_executed(hq, hkv, indices=ind)
    assert flops == _qsa_brute(G, hkv, rows, lambda i: -(-W // 32))
    assert shared + token == -(-T // min(16, 128 // G))


def test_qsa_executed_bitmap_matches_enumeration():
    rng = random.Random(7)
    for tk in (517, 16384, 20001):
        nb = (tk + 3) // 4
        T = 33
        bm = torch.zeros(T, nb, dtype=torch.uint8)
        for i in range(T):
            pick = rng.sample(range(nb), rng.choice([0, 2, 40])) if i % 3 else list(range(min(12, nb)))
            bm[i, pick] = 1
        rows = [set(t for b in torch.nonzero(bm[i]).flatten().tolist()
                    for t in range(4 * b, min(4 * b + 4, tk))) for i in range(T)]
        nblocks = [int(bm[i].sum()) for i in range(T)]
        flops, _, _ = acc.qsa_executed(12, 1, bitmap=bm, num_kv_tokens=tk)
        assert flops == _qsa_brute(12, 1, rows, lambda i: -(-nblocks[i] // 8),
                                   bitmap_direct=tk <= 16384)


def test_qsa_executed_closed_forms():
    # ten tokens (G = 12: 120 rows, eight live 16-row slots) listing the same
    # 40 keys: one shared tile, 2 chunks x 8 slots
    ind = torch.arange(40, dtype=torch.int32).repeat(10, 1)
    assert acc.qsa_executed(12, 1, indices=ind) == (8 * 2 * 16 * 32 * 256 * 4, 1, 0)
    # ten tokens each listing one different key: U = 10 > 0.8 x 10 listed, so
    # each token runs ceil(W / 32) = 1 chunk of its own
    ind = torch.full((10, 4), -1, dtype=torch.int32)
    ind[:, 0] = torch.arange(10) * 100
    assert acc.qsa_executed(12, 1, indices=ind) == (10 * 16 * 32 * 256 * 4, 0, 1)
    # keys 0, 1, 2 and 16384 in one tile: two windows of one chunk each
    ind = torch.tensor([[0, 16384, 1, 2]] * 10, dtype=torch.int32)
    assert acc.qsa_executed(12, 1, indices=ind) == (8 * 2 * 16 * 32 * 256 * 4, 1, 0)
    # keys 0 and 64 * 16384: 65 windows, past the shared route's 64
    ind = torch.tensor([[0, 64 * 16384, 1, 2]] * 10, dtype=torch.int32)
    assert acc.qsa_executed(12, 1, indices=ind)[2] == 1
    # nothing listed: a shared tile with no chunks
    assert acc.qsa_executed(12, 1, indices=torch.full((3, 4), -1, dtype=torch.int32)) == (0, 1, 0)
