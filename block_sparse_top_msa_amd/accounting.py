"""Algorithmic work of an MSA call, for throughput and roofline reporting.

Counts only what the method must do:
  attention FLOPs = sum over (query, query head) of 4 * head_dim * |A(g, i)|,
      A(g, i) the keys of the query's selected blocks that exist (j < Lk) and
      are causally visible (2 * d for QK^T, 2 * d for PV per attended key);
      work on blocks a tile computes but a token did not select is not counted.
  decode KV bytes = sum over (request, KV head) of the valid tokens of every
      block in the union of the request's selections, times both sides, times
      the stored bytes per token per side (bf16 256, fp8 128, E2M1 64 + 8
      scale bytes); each block counts once per (request, KV head).
  proxy FLOPs = 2 * head_dim per (query head, visible key) pair.

torch ops on index tensors only; none of the attention arithmetic.
"""
from __future__ import annotations

import torch

BLOCK = 128
BYTES_PER_TOKEN_SIDE = {"bf16": 256, "fp8_e4m3": 128, "e2m1x2": 72}


def _row_geometry(cu_seqlens_q, lengths_k, total_q, device):
    cu = cu_seqlens_q.to(device=device, dtype=torch.int64)
    i = torch.arange(total_q, device=device)
    b = torch.searchsorted(cu[1:], i, right=True)
    lq = (cu[1:] - cu[:-1])[b]
    iq = i - cu[b]
    lk = lengths_k.to(device=device, dtype=torch.int64)[b]
    return b, lq, iq, lk


def attended_keys(q2k, cu_seqlens_q, lengths_k, causal=True):
    """|A(g, i)| as an int64 tensor (Hkv, total_q)."""
    hkv, total_q, topk = q2k.shape
    dev = q2k.device
    _, lq, iq, lk = _row_geometry(cu_seqlens_q, lengths_k, total_q, dev)
    t = q2k.to(torch.int64)
    start = BLOCK * t
    end = torch.minimum(start + BLOCK, lk.view(1, -1, 1))
    if causal:
        pos = (lk - lq + iq).view(1, -1, 1)
        end = torch.minimum(end, pos + 1)
    nblk = (lk + BLOCK - 1) // BLOCK
    valid = (t >= 0) & (t < nblk.view(1, -1, 1))
    n = torch.clamp(end - start, min=0) * valid
    return n.sum(-1)


def attention_flops(q2k, cu_seqlens_q, lengths_k, num_qo_heads, head_dim=128, causal=True):
    hkv = q2k.shape[0]
    G = num_qo_heads // hkv
    return int(attended_keys(q2k, cu_seqlens_q, lengths_k, causal).sum()) * G * 4 * head_dim


def decode_kv_bytes(q2k, cu_seqlens_q, lengths_k, kv_format, max_k_tiles):
    """Bytes of K and V the decode must read: union of selected blocks per
    (request, KV head), valid tokens only, both sides."""
    hkv, total_q, topk = q2k.shape
    dev = q2k.device
    b, _, _, lk = _row_geometry(cu_seqlens_q, lengths_k, total_q, dev)
    B = cu_seqlens_q.numel() - 1
    used = torch.zeros(hkv, B, max_k_tiles + 1, dtype=torch.bool, device=dev)
    t = q2k.to(torch.int64)
    nblk = ((lk + BLOCK - 1) // BLOCK).view(1, -1, 1)
    ok = (t >= 0) & (t < nblk)
    tt = torch.where(ok, t, torch.full_like(t, max_k_tiles))
    bb = b.view(1, -1, 1).expand_as(tt)
    gg = torch.arange(hkv, device=dev).view(-1, 1, 1).expand_as(tt)
    used[gg, bb, tt] = True
    used = used[:, :, :max_k_tiles]
    lkb = lengths_k.to(device=dev, dtype=torch.int64).view(1, -1, 1)
    starts = BLOCK * torch.arange(max_k_tiles, device=dev).view(1, 1, -1)
    tokens = torch.clamp(torch.minimum(starts + BLOCK, lkb) - starts, min=0)
    return int((used * tokens).sum()) * 2 * BYTES_PER_TOKEN_SIDE[kv_format]


def proxy_flops(cu_seqlens_q, lengths_k, num_qo_heads, head_dim=128, causal=True):
    cq = cu_seqlens_q.cpu().tolist()
    lks = lengths_k.cpu().tolist()
    pairs = 0
    for b in range(len(cq) - 1):
        lq, lk = cq[b + 1] - cq[b], int(lks[b])
        if causal:
            # query iq sees keys 0..lk-lq+iq
            first = lk - lq + 1
            pairs += sum(max(0, min(lk, first + iq)) for iq in range(lq))
        else:
            pairs += lq * lk
    return pairs * num_qo_heads * 2 * head_dim


# ---------------------------------------------------------------------------
# Executed MFMA work of the prefill tile kernel (a diagnostic beside the
# selected-work count above, not part of it)
# ---------------------------------------------------------------------------

SLOT_ROWS = 32
TILE_ROWS = 256


def prefill_tile_tokens(num_qo_heads, num_kv_heads, topk, max_union=512):
    """Query tokens per tile on the prefill route: 256 token-major rows of G
    heads each, at most 64 tokens (the per-block token masks) and at most
    `max_union` / topk tokens (the union list)."""
    G = num_qo_heads // num_kv_heads
    t = max(1, min(64, TILE_ROWS // G))
    if t * topk > max_union:
        t = max(1, max_union // topk)
    return t


def prefill_slot_blocks(q2k, cu_seqlens_q, lengths_k, num_qo_heads, tile_tokens):
    """Number of (32-row slot, KV block) pairs the prefill kernel computes.

    Tiles hold `tile_tokens` consecutive queries of one request and one KV
    head; their rows are token-major (row = G t + head), cut into 32-row
    slots.  A slot computes a block of its tile's union when a token with a
    row in the slot selected it (ids outside [0, ceil(Lk / 128)) are not in
    the union)."""
    hkv, total_q, topk = q2k.shape
    G = num_qo_heads // hkv
    dev = q2k.device
    b, _, iq, lk = _row_geometry(cu_seqlens_q, lengths_k, total_q, dev)
    B = cu_seqlens_q.numel() - 1
    t = q2k.to(torch.int64)
    nblk = ((lk + BLOCK - 1) // BLOCK).view(1, -1, 1)
    ok = (t >= 0) & (t < nblk)
    max_blk = int(nblk.max()) + 1 if nblk.numel() else 1
    tile = (iq // tile_tokens).view(1, -1, 1)
    tin = (iq % tile_tokens).view(1, -1, 1)
    s_lo = (G * tin) // SLOT_ROWS
    s_hi = (G * tin + G - 1) // SLOT_ROWS
    n_tiles = int(tile.max()) + 1 if tile.numel() else 1
    n_slots = (tile_tokens * G + SLOT_ROWS - 1) // SLOT_ROWS
    gg = torch.arange(hkv, device=dev).view(-1, 1, 1)
    bb = b.view(1, -1, 1)
    keys = []
    for k in range((G + SLOT_ROWS - 1) // SLOT_ROWS + 1):
        slot = s_lo + k
        use = ok & (slot <= s_hi)
        key = (((gg * B + bb) * n_tiles + tile) * n_slots + slot) * max_blk + t
        keys.append(key.expand_as(t)[use])
    return int(torch.unique(torch.cat(keys)).numel()) if keys else 0


def prefill_executed_flops(q2k, cu_seqlens_q, lengths_k, num_qo_heads, tile_tokens,
                           head_dim=128):
    """MFMA FLOPs of the prefill kernel: per computed (slot, block), S^T of
    32 rows x 128 keys and O^T += V^T P^T of the same size."""
    n = prefill_slot_blocks(q2k, cu_seqlens_q, lengths_k, num_qo_heads, tile_tokens)
    return n * SLOT_ROWS * BLOCK * head_dim * 4


# ---------------------------------------------------------------------------
# Executed MFMA work of the QSA tile kernel (a diagnostic beside the
# selected-token count, not part of it)
# ---------------------------------------------------------------------------

QSA_TILE_ROWS = 128      # eight 16-row slots
QSA_MAX_TOKENS = 16      # token bits of a key's mask word
QSA_WIN = 16384          # keys of one window of a tile's key range
QSA_MAX_WIN = 64         # windows a shared-route tile may span
QSA_SLOT_ROWS = 16


def qsa_tile_tokens(num_qo_heads, num_kv_heads):
    """Consecutive query tokens per QSA tile: 128 token-major rows of G heads,
    at most 16 tokens."""
    return min(QSA_MAX_TOKENS, QSA_TILE_ROWS // (num_qo_heads // num_kv_heads))


def qsa_executed(num_qo_heads, num_kv_heads, indices=None, bitmap=None, num_kv_tokens=None,
                 head_dim=256):
    """(MFMA FLOPs, shared tiles, per-token tiles) of the QSA kernel on index
    rows ([T, W] int32, negative = padding) or a block bitmap ([T, NB] uint8
    over num_kv_tokens keys).

    A tile of `qsa_tile_tokens` queries takes the shared route when its
    listed keys fall in at most 64 windows of 16384 keys (from its lowest
    key; a bitmap over at most 16384 keys is one window from key 0) and
    5 * U * ceil(S / 4) <= 8 * L, with U its key union, L its listed entries
    and S = ceil(tokens * G / 16) its live 16-row slots; then every live
    slot computes 32-key chunks over each window's union (ceil(U_w / 32)
    chunks per window).  Otherwise each token takes its own 16-row tile
    over its own keys: ceil(W / 32) chunks of index entries, or one chunk
    per eight selected blocks.  A 16-row slot's chunk costs 16 x 32 keys x
    head_dim x 4 FLOPs (S^T and O^T += V^T P^T), for every KV head."""
    G = num_qo_heads // num_kv_heads
    tt = qsa_tile_tokens(num_qo_heads, num_kv_heads)
    chunk = QSA_SLOT_ROWS * 32 * head_dim * 4
    if bitmap is not None:
        bm = bitmap.cpu() != 0
        T, nb = bm.shape
        blk = torch.arange(nb)
        size = torch.clamp(num_kv_tokens - 4 * blk, max=4)   # tokens per block
    else:
        ind = indices.cpu().to(torch.int64)
        T, W = ind.shape
    flops = shared = token = 0
    for t0 in range(0, T, tt):
        nt = min(tt, T - t0)
        slots = (nt * G + QSA_SLOT_ROWS - 1) // QSA_SLOT_ROWS
        if bitmap is not None:
            rows = bm[t0:t0 + nt]
            listed = int((rows.to(torch.int64) * size).sum())
            ub = rows.any(0)
            U = int(size[ub].sum())
            if U:
                lo, hi = 4 * int(blk[ub][0]), min(4 * int(blk[ub][-1]) + 3, num_kv_tokens - 1)
                base = 0 if num_kv_tokens <= QSA_WIN else lo
                tok = torch.arange(4 * nb).view(nb, 4)[ub].flatten()
                ukeys = tok[tok < num_kv_tokens]
            per_token = [(int(r.sum()) + 7) // 8 for r in rows]
        else:
            keys = ind[t0:t0 + nt]
            keys = keys[keys >= 0]
            listed = int(keys.numel())
            ukeys = torch.unique(keys)
            U = int(ukeys.numel())
            if U:
                lo, hi = int(keys.min()), int(keys.max())
                base = lo
            per_token = [(W + 31) // 32] * nt
        if U and ((hi - base) // QSA_WIN + 1 > QSA_MAX_WIN or
                  5 * U * ((slots + 3) // 4) > 8 * listed):
            token += 1
            flops += sum(per_token) * chunk
        else:
            shared += 1
            if U:
                per_win = torch.bincount((ukeys - base) // QSA_WIN)
                flops += slots * int(((per_win + 31) // 32).sum()) * chunk
    return flops * num_kv_heads, shared, token
