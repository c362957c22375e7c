"""Plain fp64 CPU oracle for the MiniMax Sparse Attention (MSA) hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
calls it, and it imports nothing from the HIP library: the two share no code.

Everything here is a direct, unblocked evaluation of the definitions on the
MSA documentation pages, in float64, with torch CPU ops (a matmul, a sort)
as library steps:

  decode_*          storage formats to exact values
                    (msa_sparse_attention page, Parameters: q / k / k_scale;
                     prepare_msa_nvfp4_sparse_decode page, Parameters: k, v,
                     k_scale, v_scale)
  proxy_score       per-KV-block max of unscaled, causally masked Q K^T
                    (msa_proxy_score page, summary and Parameters: causal,
                     max_k_tiles, reduce_heads)
  topk_select       top-K blocks per (kv head, query), ascending, -1 padded,
                    ties to the lower block id (msa_sparse_attention page,
                    Parameters: q2k_indices; prepare_msa_nvfp4_sparse_decode
                    page, Parameters: q2k_indices)
  tile_union        union of a query tile's selected blocks (msa_sparse_attention
                    page, summary)
  sparse_attention  dense attention masked down to each query's selected blocks
                    (msa_sparse_attention page, summary, Parameters and Returns)
  lse_merge         combining split partials by their LSE
                    (prepare_msa_nvfp4_sparse_decode page, Parameters:
                     workspace_buffer)
  qsa_indexed_attention, qsa_bitmap_attention
                    packed query sparse attention over caller-listed token
                    indices or a block bitmap (qsa page)

Readings of points the pages leave open are stated where they are used.
Every function is pinned by tests/test_oracle.py against something other than
itself (a library routine, a closed form, brute force, a format definition).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK = 128  # tokens per KV block / page

__all__ = [
    "BLOCK", "decode_bf16", "decode_f16", "decode_q", "decode_e4m3fn", "decode_e2m1",
    "unpack_e2m1x2", "qsa_indexed_attention", "qsa_bitmap_indices", "qsa_bitmap_attention",
    "dequant_e2m1", "decode_kv", "request_lengths", "logical_kv", "query_positions",
    "proxy_score",
    "reduce_heads", "selection_scores", "topk_select", "tile_union",
    "allowed_keys", "sparse_attention", "lse_merge",
]


# ---------------------------------------------------------------------------
# O0: storage formats -> exact float64 values
# ---------------------------------------------------------------------------

def decode_bf16(t: torch.Tensor) -> torch.Tensor:
    """bf16 -> float64, by placing the 16 stored bits on top of an fp32 word.

    bf16 is the top half of an IEEE binary32, so the value is exact.
    """
    bits = t.contiguous().view(torch.int16).to(torch.int32) & 0xFFFF
    return (bits << 16).view(torch.float32).to(torch.float64)


def decode_e4m3fn(b: torch.Tensor) -> torch.Tensor:
    """E4M3FN bytes -> float64.

    OCP 8-bit float E4M3, the `float8_e4m3fn` type named on the
    msa_sparse_attention page (Parameters: k_scale): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
    (2^-6 * m/8); no infinities; S.1111.111 is NaN.
    """
    b = b.contiguous().view(torch.uint8).to(torch.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = (b & 7).to(torch.float64)
    sign = 1.0 - 2.0 * s.to(torch.float64)
    normal = torch.pow(2.0, (e - 7).to(torch.float64)) * (1.0 + m / 8.0)
    sub = (2.0 ** -6) * (m / 8.0)
    val = sign * torch.where(e == 0, sub, normal)
    nan = (e == 15) & ((b & 7) == 7)
    return torch.where(nan, torch.full_like(val, float("nan")), val)


def decode_e2m1(nib: torch.Tensor) -> torch.Tensor:
    """E2M1 nibble -> float64.

    4-bit float: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0;
    exponent 0 is subnormal (m/2).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
    """
    n = nib.to(torch.int64) & 0xF
    s = (n >> 3) & 1
    e = (n >> 1) & 3
    m = (n & 1).to(torch.float64)
    sign = 1.0 - 2.0 * s.to(torch.float64)
    normal = torch.pow(2.0, (e - 1).to(torch.float64)) * (1.0 + m / 2.0)
    sub = m / 2.0
    return sign * torch.where(e == 0, sub, normal)


def unpack_e2m1x2(packed: torch.Tensor) -> torch.Tensor:
    """uint8 (..., d/2) -> nibbles (..., d).

    Reading (the pages say two values per byte but not which goes where):
    element 2i is the low nibble of byte i, element 2i+1 the high nibble.
    """
    p = packed.to(torch.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    return torch.stack([lo, hi], dim=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)


def dequant_e2m1(packed: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """Packed E2M1 (..., d/2) with E4M3 block scales (..., d/16) -> (..., d).

    Each group of 16 consecutive values along the head dimension shares one
    E4M3 scale (msa_sparse_attention page, Parameters: k_scale; reading: the
    scales are stored linearly for both K and V).  The per-side global scale
    is not applied here: K's folds into the softmax scale and V's multiplies
    the output.
    """
    vals = decode_e2m1(unpack_e2m1x2(packed))
    sc = decode_e4m3fn(scale)
    return vals * torch.repeat_interleave(sc, 16, dim=-1)


def decode_f16(t: torch.Tensor) -> torch.Tensor:
    """IEEE binary16 -> float64 from its fields: sign, 5-bit exponent (bias
    15), 10-bit fraction; exponent 0 is subnormal (2^-14 * f / 1024), 31 is
    inf / NaN (the msa_sparse_attention page, Parameters: q and k accept
    fp16)."""
    bits = t.contiguous().view(torch.int16).to(torch.int64) & 0xFFFF
    sign = torch.where((bits >> 15) == 1, -1.0, 1.0).to(torch.float64)
    e = (bits >> 10) & 0x1F
    f = (bits & 0x3FF).to(torch.float64)
    normal = torch.ldexp(1.0 + f / 1024.0, (e - 15).to(torch.float64).to(torch.int32))
    sub = torch.ldexp(f / 1024.0, torch.full_like(e, -14, dtype=torch.int32))
    val = torch.where(e == 0, sub, normal)
    val = torch.where(e == 31, torch.where(f == 0, torch.tensor(math.inf, dtype=torch.float64),
                                           torch.tensor(math.nan, dtype=torch.float64)), val)
    return sign * val


def decode_q(t: torch.Tensor) -> torch.Tensor:
    """Query storage (bf16 or fp16) -> float64."""
    return decode_f16(t) if t.dtype == torch.float16 else decode_bf16(t)


def decode_kv(data: torch.Tensor, kv_format: str, scale: Optional[torch.Tensor] = None):
    """K or V storage -> float64 values of the same logical shape (..., d)."""
    data = data.cpu()
    if kv_format == "bf16":
        return decode_bf16(data)
    if kv_format == "f16":
        return decode_f16(data)
    if kv_format == "fp8_e4m3":
        return decode_e4m3fn(data.view(torch.uint8))
    if kv_format == "e2m1x2":
        return dequant_e2m1(data.view(torch.uint8), scale.cpu().view(torch.uint8))
    raise ValueError(kv_format)


# ---------------------------------------------------------------------------
# O1, O2: addressing and causal positions
# ---------------------------------------------------------------------------

def request_lengths(cu_seqlens_q, cu_seqlens_k=None, seqused_k=None):
    """Per request: (first query row, Lq, Lk).  Flat KV length comes from
    cu_seqlens_k; paged from seqused_k (msa_sparse_attention page,
    Parameters: cu_seqlens_k, seqused_k)."""
    cq = [int(x) for x in torch.as_tensor(cu_seqlens_q).cpu()]
    out = []
    for b in range(len(cq) - 1):
        if seqused_k is not None:
            lk = int(torch.as_tensor(seqused_k).cpu()[b])
        else:
            ck = torch.as_tensor(cu_seqlens_k).cpu()
            lk = int(ck[b + 1]) - int(ck[b])
        out.append((cq[b], cq[b + 1] - cq[b], lk))
    return out


def _key_rows(b, blocks, lk, cu_seqlens_k, page_table):
    """For logical blocks of request b: per block, (storage selector, count
    of valid keys).  Flat: rows cu_k[b] + 128 t ...; paged: page
    page_table[b, t], slots 0..127 (msa_sparse_attention page, Parameters:
    k, page_table)."""
    res = []
    for t in blocks:
        n = min(BLOCK, lk - BLOCK * t)
        if n <= 0:
            continue
        if page_table is not None:
            res.append(("page", int(page_table[b, t]), t, n))
        else:
            start = int(cu_seqlens_k[b]) + BLOCK * t
            res.append(("rows", start, t, n))
    return res


def logical_kv(side, kv_format, scale, b, blocks, lk, cu_seqlens_k=None, page_table=None):
    """Decoded keys (or values) of request b restricted to `blocks`.

    Returns (positions int64 [n], values float64 [n, Hkv, d]) with key
    positions j = 128 t + slot, only j < Lk.
    """
    pt = None if page_table is None else torch.as_tensor(page_table).cpu()
    ck = None if cu_seqlens_k is None else torch.as_tensor(cu_seqlens_k).cpu()
    pos, vals = [], []
    for kind, where, t, n in _key_rows(b, blocks, lk, ck, pt):
        if kind == "page":
            raw = side[where, :, :n]                    # (Hkv, n, d')
            sc = None if scale is None else scale[where, :, :n]
            x = decode_kv(raw, kv_format, sc).permute(1, 0, 2)  # (n, Hkv, d)
        else:
            raw = side[where:where + n]                 # (n, Hkv, d')
            sc = None if scale is None else scale[where:where + n]
            x = decode_kv(raw, kv_format, sc)
        vals.append(x)
        pos.append(torch.arange(BLOCK * t, BLOCK * t + n, dtype=torch.int64))
    if not vals:
        return torch.zeros(0, dtype=torch.int64), None
    return torch.cat(pos), torch.cat(vals, dim=0)


def query_positions(q0: int, lq: int, lk: int, q_offset=None) -> torch.Tensor:
    """KV position of each local query iq of a request (int64 [Lq]).

    Default: right-aligned, Lk - Lq + iq (msa_proxy_score page, Parameters:
    causal; prepare_msa_nvfp4_sparse_decode page, Parameters: seqlen_q).
    With q_offset (msa_proxy_score page, Parameters: q_offset, a query
    position offset used by the causal alignment; msa_sparse_attention page,
    Parameters: q_offset, a per-query offset tensor).  Reading, since the
    pages define neither form further: an int o places query iq of every
    request at o + iq (o replaces the right alignment's Lk - Lq); a tensor
    holds each query row's own position, q_offset[q0 + iq].  Parity of this
    reading against the pages' kernels is unpinned.
    """
    iq = torch.arange(lq, dtype=torch.int64)
    if q_offset is None:
        return (lk - lq) + iq
    if isinstance(q_offset, int):
        return int(q_offset) + iq
    return torch.as_tensor(q_offset).cpu().to(torch.int64)[q0:q0 + lq].clone()


def allowed_keys(pos_keys: torch.Tensor, lq: int, lk: int, causal: bool,
                 qpos: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Bool [Lq, n]: key j may be seen by local query iq.

    Causal: query iq sees keys j <= its KV position, qpos[iq] (default the
    right alignment Lk - Lq + iq, see query_positions).  Reading for flat
    prefill with Lq != Lk: the same right alignment.  Keys j >= Lk never
    exist.
    """
    if qpos is None:
        qpos = (lk - lq) + torch.arange(lq, dtype=torch.int64)
    j = pos_keys.unsqueeze(0)
    ok = (j < lk).expand(lq, -1)
    if causal:
        ok = ok & (j <= qpos.unsqueeze(1))
    return ok


# ---------------------------------------------------------------------------
# O3, O4: proxy score and head reduction
# ---------------------------------------------------------------------------

def proxy_score(q, k, cu_seqlens_q, *, cu_seqlens_k=None, page_table=None,
                seqused_k=None, causal=True, max_k_tiles=None, reduce_heads=False,
                kv_format="bf16", rows: Optional[Sequence[int]] = None,
                chunk: int = 512, q_offset=None):
    """max_score[h, t, i]: max over keys j of block t (128 t <= j < 128 t + 128,
    j < Lk, j allowed by the causal rule) of the unscaled dot product
    q[i, h] . k[j, h // G]; -inf where no key qualifies or t is past the
    sequence (msa_proxy_score page, summary).  No softmax scale and no global
    scale enter.

    Returns float64 (Hq, max_k_tiles, total_q), or (1, ...) with
    reduce_heads (max over the query-head axis, msa_proxy_score page,
    Parameters: reduce_heads).  With `rows`, only those query rows are
    evaluated; the other columns stay -inf.
    """
    q = q.cpu()
    total_q, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    reqs = request_lengths(cu_seqlens_q, cu_seqlens_k, seqused_k)
    if max_k_tiles is None:
        max_k_tiles = max(((lk + BLOCK - 1) // BLOCK for _, _, lk in reqs), default=0)
    out = torch.full((hq, max_k_tiles, total_q), float("-inf"), dtype=torch.float64)
    want = None if rows is None else set(int(r) for r in rows)
    for b, (q0, lq, lk) in enumerate(reqs):
        local = [iq for iq in range(lq) if want is None or (q0 + iq) in want]
        if not local or lk <= 0:
            continue
        nblk = (lk + BLOCK - 1) // BLOCK
        pos, kv = logical_kv(k, kv_format, None, b, range(nblk), lk, cu_seqlens_k, page_table)
        tiles = min(nblk, max_k_tiles)
        pad = nblk * BLOCK - lk
        for c0 in range(0, len(local), chunk):
            li = torch.tensor(local[c0:c0 + chunk], dtype=torch.int64)
            qpos = query_positions(q0, lq, lk, q_offset)
            ok = allowed_keys(pos, lq, lk, causal, qpos)[li]      # (n, Lk)
            qb = decode_q(q[q0 + li])                           # (n, hq, d)
            for h in range(hq):
                z = qb[:, h, :] @ kv[:, h // G, :].T               # (n, Lk)
                z = torch.where(ok, z, torch.full_like(z, float("-inf")))
                z = torch.nn.functional.pad(z, (0, pad), value=float("-inf"))
                bm = z.view(len(li), nblk, BLOCK).max(dim=2).values  # (n, nblk)
                out[h, :tiles, q0 + li] = bm[:, :tiles].T
    if reduce_heads:
        out = _reduce_heads(out)   # the module-level reduce_heads below
    return out


def reduce_heads(scores: torch.Tensor) -> torch.Tensor:
    """amax over the query-head axis: (H, T, total_q) -> (1, T, total_q)."""
    return torch.as_tensor(scores).max(dim=0, keepdim=True).values


_reduce_heads = reduce_heads   # proxy_score's keyword argument shadows the name


def selection_scores(scores: torch.Tensor, num_kv_heads: int, mode: str = "auto"):
    """Scores used by each KV head's selection: (Hkv, T, total_q).

    mode "none": one score head per KV head (H_s == Hkv).
    mode "all":  the max over every score head (a reduce_heads output has
                 H_s == 1 already), copied to every KV head — reading of the
                 pages' "one shared block selection per query" for a
                 reduce_heads score feeding a per-KV-head q2k.
    mode "group": per-query-head scores (H_s == G * Hkv), max over the G
                 query heads of each KV head.  Not on the pages; the
                 per-group analogue of reduce_heads.
    mode "auto": "all" if H_s == 1, "none" if H_s == Hkv.
    """
    s = torch.as_tensor(scores)
    hs = s.shape[0]
    if mode == "auto":
        mode = "all" if hs == 1 else ("none" if hs == num_kv_heads else "group")
    if mode == "all":
        return s.max(dim=0, keepdim=True).values.expand(num_kv_heads, *s.shape[1:])
    if mode == "none":
        assert hs == num_kv_heads
        return s
    if mode == "group":
        assert hs % num_kv_heads == 0
        G = hs // num_kv_heads
        return s.reshape(num_kv_heads, G, *s.shape[1:]).max(dim=1).values
    raise ValueError(mode)


# ---------------------------------------------------------------------------
# O5: top-K block select
# ---------------------------------------------------------------------------

def topk_select(scores, topk: int, num_kv_heads: int, mode: str = "auto",
                rows: Optional[Sequence[int]] = None) -> torch.Tensor:
    """q2k_indices (Hkv, total_q, topk) int32 from max_score.

    For each (KV head g, query i): the candidates are the blocks t with a
    finite score; they are ordered by score, largest first, with equal scores
    (IEEE equality, so -0 == +0) ordered by lower block id; the first
    min(topk, #candidates) are kept and written ascending, -1 padded
    (msa_sparse_attention page, Parameters: q2k_indices).  -inf blocks are
    never selected, so a row with fewer finite blocks ends in -1.

    Comparisons happen in the precision of `scores` (fp32 scores stay fp32
    values; widening to float64 preserves their order).
    """
    s = selection_scores(torch.as_tensor(scores).cpu(), num_kv_heads, mode)
    s = s.to(torch.float64).numpy()                 # (Hkv, T, total_q)
    hkv, T, total_q = s.shape
    cols = np.arange(total_q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.full((hkv, total_q, topk), -1, dtype=np.int32)
    if T == 0 or cols.size == 0:
        return torch.from_numpy(out)
    tid = np.broadcast_to(np.arange(T), (cols.size, T))
    for g in range(hkv):
        sc = s[g][:, cols].T                        # (n, T)
        finite = np.isfinite(sc)
        key = np.where(finite, -sc, np.inf)         # excluded sort last
        order = np.lexsort((tid, key), axis=-1)     # primary: key, then block id
        kk = min(topk, T)
        top = order[:, :kk]
        keep = np.take_along_axis(finite, top, axis=1)
        chosen = np.where(keep, top, np.iinfo(np.int32).max)
        chosen = np.sort(chosen, axis=1)
        chosen = np.where(chosen == np.iinfo(np.int32).max, -1, chosen)
        out[g, cols, :kk] = chosen.astype(np.int32)
    return torch.from_numpy(out)


# ---------------------------------------------------------------------------
# a4: per-tile union of selected blocks
# ---------------------------------------------------------------------------

def tile_union(q2k_rows: torch.Tensor, num_blocks: int):
    """Union of the blocks a query tile selected (msa_sparse_attention page,
    summary: each tile runs one softmax over the union of its tokens' blocks).

    q2k_rows: (T, topk) int32 rows of the tile's tokens for one KV head.
    Returns (ascending list of blocks b with 0 <= b < num_blocks, and per
    listed block the bit mask of tile tokens that selected it).
    """
    rows = torch.as_tensor(q2k_rows).cpu().tolist()
    masks = {}
    for tok, row in enumerate(rows):
        for b in row:
            if 0 <= b < num_blocks:
                masks[b] = masks.get(b, 0) | (1 << tok)
    blocks = sorted(masks)
    return blocks, [masks[b] for b in blocks]


# ---------------------------------------------------------------------------
# O6: sparse attention
# ---------------------------------------------------------------------------

def sparse_attention(q, k, v, q2k, cu_seqlens_q, *, cu_seqlens_k=None,
                     page_table=None, seqused_k=None, causal=False,
                     softmax_scale=None, kv_format="bf16", k_scale=None,
                     v_scale=None, k_global_scale=None, v_global_scale=None,
                     rows: Optional[Sequence[int]] = None, chunk: int = 256,
                     lse_temperature_scale: Optional[float] = None, q_offset=None):
    """Dense attention masked down to each query's selected blocks.

    For query i of request b, query head h and its KV head g = h // G
    (G = Hq / Hkv), the attended keys are
        A(g, i) = { j : j // 128 in q2k[g, i, :] (entries >= 0),
                    j < Lk, j allowed by the right-aligned causal rule }
    (msa_sparse_attention page, summary and Parameters: q2k_indices, causal).
    Logits z_j = s_eff * q[i, h] . k[j, g] with
    s_eff = (softmax_scale or d^-0.5) * (k_global_scale or 1) (Parameters:
    softmax_scale, k_global_scale: the K global scale folds into the softmax
    scale).  lse = ln sum_j exp(z_j) (natural log, Returns) and
    out = (v_global_scale or 1) * sum_j exp(z_j - lse) v[j, g]
    (Parameters: v_global_scale, applied to the output).  An empty A gives a
    zero output and lse = -inf.  The entries of a q2k row are read as a set:
    duplicates, out-of-range blocks and -1 add nothing.

    Returns float64 (out [n, Hq, d], lse [n, Hq]) for all rows, or for
    `rows` in the given order.

    With `lse_temperature_scale` = tau also returns the temperature LSE
    lse_t [n, Hq] = ln sum_j exp(tau * z_j) over the same keys (-inf when A
    is empty).  Reading: the msa_sparse_attention page (Parameters:
    return_temperature_lse, lse_temperature_scale) says only that the scale
    multiplies the exponent; z_j are the logits whose LSE is lse, so tau = 1
    gives lse_t = lse.

    q_offset: the queries' causal positions (see query_positions).
    """
    q = q.cpu()
    q2k = torch.as_tensor(q2k).cpu()
    total_q, hq, d = q.shape
    hkv = q2k.shape[0]
    G = hq // hkv
    scale = (d ** -0.5) if softmax_scale is None else float(softmax_scale)
    s_eff = scale * (1.0 if k_global_scale is None else float(k_global_scale))
    vgs = 1.0 if v_global_scale is None else float(v_global_scale)
    reqs = request_lengths(cu_seqlens_q, cu_seqlens_k, seqused_k)

    row_list = list(range(total_q)) if rows is None else [int(r) for r in rows]
    where = {r: n for n, r in enumerate(row_list)}
    out = torch.zeros((len(row_list), hq, d), dtype=torch.float64)
    lse = torch.full((len(row_list), hq), float("-inf"), dtype=torch.float64)
    tau = None if lse_temperature_scale is None else float(lse_temperature_scale)
    lse_t = torch.full((len(row_list), hq), float("-inf"), dtype=torch.float64)

    for b, (q0, lq, lk) in enumerate(reqs):
        local = [iq for iq in range(lq) if (q0 + iq) in where]
        nblk = (lk + BLOCK - 1) // BLOCK
        for c0 in range(0, len(local), chunk):
            li = torch.tensor(local[c0:c0 + chunk], dtype=torch.int64)
            qi = decode_q(q[q0 + li])                             # (n, hq, d)
            dst = torch.tensor([where[q0 + int(x)] for x in li])
            for g in range(hkv):
                sel = q2k[g, q0 + li]                                # (n, topk)
                blocks = sorted({int(x) for x in sel.flatten().tolist() if 0 <= x < nblk})
                if not blocks:
                    continue
                pos, kk = logical_kv(k, kv_format, k_scale, b, blocks, lk, cu_seqlens_k, page_table)
                _, vv = logical_kv(v, kv_format, v_scale, b, blocks, lk, cu_seqlens_k, page_table)
                kblk = pos // BLOCK
                chosen = (sel.unsqueeze(2) == kblk.view(1, 1, -1)).any(dim=1)  # (n, nkeys)
                qpos = query_positions(q0, lq, lk, q_offset)
                ok = chosen & allowed_keys(pos, lq, lk, causal, qpos)[li]
                any_ok = ok.any(dim=1)
                for hh in range(G):
                    h = g * G + hh
                    z = s_eff * (qi[:, h, :] @ kk[:, g, :].T)          # (n, nkeys)
                    z = torch.where(ok, z, torch.full_like(z, float("-inf")))
                    m = z.max(dim=1, keepdim=True).values
                    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
                    e = torch.exp(z - m)                             # exp(-inf) = 0
                    ssum = e.sum(dim=1, keepdim=True)
                    l_h = (m + torch.log(ssum)).squeeze(1)
                    p = e / torch.where(ssum > 0, ssum, torch.ones_like(ssum))
                    o_h = vgs * (p @ vv[:, g, :])
                    l_h = torch.where(any_ok, l_h, torch.full_like(l_h, float("-inf")))
                    o_h = torch.where(any_ok.unsqueeze(1), o_h, torch.zeros_like(o_h))
                    out[dst, h] = o_h
                    lse[dst, h] = l_h
                    if tau is not None:
                        zt = torch.where(ok, tau * z, torch.full_like(z, float("-inf")))
                        mt = zt.max(dim=1, keepdim=True).values
                        mt = torch.where(torch.isfinite(mt), mt, torch.zeros_like(mt))
                        lt = (mt + torch.log(torch.exp(zt - mt).sum(dim=1, keepdim=True))).squeeze(1)
                        lse_t[dst, h] = torch.where(any_ok, lt, torch.full_like(lt, float("-inf")))
    return (out, lse) if tau is None else (out, lse, lse_t)


# ---------------------------------------------------------------------------
# a8: combining split partials
# ---------------------------------------------------------------------------

def lse_merge(parts):
    """Merge attention partials computed over disjoint key subsets.

    parts: sequence of (o_s, lse_s) with o_s normalised over its own subset
    (o_s = sum exp(z - lse_s) v) and lse_s its natural-log normaliser.
    lse = ln sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s.  All-empty
    parts (lse_s = -inf everywhere) give o = 0, lse = -inf.  This is how
    split-KV partials combine (prepare_msa_nvfp4_sparse_decode page,
    Parameters: workspace_buffer).
    """
    os_ = torch.stack([torch.as_tensor(o, dtype=torch.float64) for o, _ in parts])
    ls = torch.stack([torch.as_tensor(l, dtype=torch.float64) for _, l in parts])
    m = ls.max(dim=0).values
    m_safe = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    w = torch.exp(ls - m_safe)                                   # (S, ...)
    tot = w.sum(dim=0)
    lse = torch.where(tot > 0, m_safe + torch.log(torch.where(tot > 0, tot, torch.ones_like(tot))),
                      torch.full_like(tot, float("-inf")))
    wn = w / torch.where(tot > 0, tot, torch.ones_like(tot))
    o = (wn.unsqueeze(-1) * os_).sum(dim=0)
    return o, lse


# ---------------------------------------------------------------------------
# QSA: packed query sparse attention from token indices (qsa page)
# ---------------------------------------------------------------------------

def qsa_indexed_attention(q, k, v, indices, softmax_scale=None):
    """Packed query sparse attention over caller-selected tokens (qsa page:
    the indexed API, its output and LSE description and its example).

    q: bf16 [T, Hq, d]; k, v: bf16 [Tk, Hkv, d]; indices: int32 [T, W], the
    absolute packed token ids (rows of k / v) query i attends, in groups of
    four with -1 padding.  Query head h reads KV head h // (Hq / Hkv).
    Readings: an index row is a set (negative entries are padding; entries
    are distinct by the caller contract, so repeats are ignored); the
    softmax scale defaults to d^-0.5 as on the MSA pages; causality is the
    caller's, carried by the indices themselves.
    Returns (out [T, Hq, d], lse [Hq, T]) in float64; a query with no index
    gets out = 0 and lse = -inf.
    """
    qd = decode_bf16(q)
    kd = decode_bf16(k)
    vd = decode_bf16(v)
    T, Hq, d = qd.shape
    Hkv = kd.shape[1]
    G = Hq // Hkv
    scale = float(softmax_scale) if softmax_scale else d ** -0.5
    out = torch.zeros(T, Hq, d, dtype=torch.float64)
    lse = torch.full((Hq, T), -math.inf, dtype=torch.float64)
    for i in range(T):
        ids = sorted({int(x) for x in indices[i].tolist() if int(x) >= 0})
        if not ids:
            continue
        sel = torch.tensor(ids, dtype=torch.long)
        for h in range(Hq):
            z = scale * (kd[sel, h // G] @ qd[i, h])          # [n]
            m = z.max()
            w = torch.exp(z - m)
            s = w.sum()
            lse[h, i] = m + torch.log(s)
            out[i, h] = (w / s) @ vd[sel, h // G]
    return out, lse



def qsa_bitmap_indices(bitmap, num_kv_tokens: int):
    """Index rows equivalent to a QSA block bitmap (qsa page: the bitmap API).

    Reading (the page names a uint8 block bitmap and its int32 [T, NB]
    compact-index counterpart, nothing more): bitmap[i, b] != 0 selects the
    four packed tokens 4 b .. 4 b + 3 (those below num_kv_tokens) for query
    i.  Returns int32 [T, 4 * NB], ascending, -1 padded."""
    T, NB = bitmap.shape
    out = torch.full((T, 4 * NB), -1, dtype=torch.int32)
    for i in range(T):
        blocks = torch.nonzero(bitmap[i].cpu() != 0).flatten()
        tok = (4 * blocks.view(-1, 1) + torch.arange(4).view(1, -1)).reshape(-1)
        tok = tok[tok < num_kv_tokens]
        out[i, :tok.numel()] = tok.to(torch.int32)
    return out


def qsa_bitmap_attention(q, k, v, bitmap, softmax_scale=None):
    """QSA over a block bitmap: the indexed definition applied to the tokens
    of every selected block (qsa page: the bitmap API and its outputs)."""
    return qsa_indexed_attention(q, k, v, qsa_bitmap_indices(bitmap, k.shape[0]),
                                 softmax_scale=softmax_scale)
