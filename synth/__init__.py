"""Seeded synthetic inputs for the MSA sparse-attention path.

This module only draws random numbers and lays them out in the tensor formats
that the MiniMax Sparse Attention pages define (msa_sparse_attention page,
Parameters; msa_proxy_score page, Parameters; prepare_msa_nvfp4_sparse_decode
page, Parameters).  It holds none of the method's arithmetic: no proxy score,
no selection by score, no softmax.  Both the fp64 oracle and the HIP path
consume the same tensors built here.

Random draws happen in a fixed order per problem: sequence lengths, page
permutation, Q, K, V, proxy Q, selection randomness.  A problem is fully
determined by (recipe, seed, device): torch's CPU generator and its GPU
generator give different streams, so a test builds its inputs once and hands
the same tensors to both sides.
"""
from __future__ import annotations

import dataclasses
import itertools
import math
from typing import Optional

import torch

BLOCK = 128  # KV block / page size in tokens (msa_sparse_attention page, Parameters: k)

KV_BF16 = "bf16"
KV_FP8 = "fp8_e4m3"
KV_E2M1 = "e2m1x2"
KV_F16 = "f16"      # fp16 Q, K and V


@dataclasses.dataclass
class Problem:
    """One synthetic MSA problem.  Tensors live on `device`.

    q            (total_q, Hq, d) bf16
    k, v         flat (total_k, Hkv, d') or paged (num_pages, Hkv, 128, d');
                 d' = d for bf16 / fp8, d // 2 bytes for packed E2M1
    k_scale, v_scale  E2M1 only: (num_pages, Hkv, 128, d // 16) uint8 E4M3 bytes,
                 flat (total_k, Hkv, d // 16) in (token, head) order
    q2k          (Hkv, total_q, topk) int32, ascending, -1 padded, or None
                 when the selection is to come from the proxy pass
    proxy_q      (total_q, Hp, d) bf16 or None (the proxy reuses q then)
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens_q: torch.Tensor
    kv_dtype: str = KV_BF16
    cu_seqlens_k: Optional[torch.Tensor] = None
    page_table: Optional[torch.Tensor] = None
    seqused_k: Optional[torch.Tensor] = None
    q2k: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    causal: bool = True
    softmax_scale: Optional[float] = None
    k_global_scale: Optional[float] = None
    v_global_scale: Optional[float] = None
    topk: int = 16
    proxy_q: Optional[torch.Tensor] = None
    reduce_heads: bool = False
    max_k_tiles: int = 0
    # host copies of the per-request lengths (small)
    q_lens: tuple = ()
    k_lens: tuple = ()

    @property
    def paged(self) -> bool:
        return self.page_table is not None

    @property
    def batch(self) -> int:
        return len(self.q_lens)

    @property
    def num_qo_heads(self) -> int:
        return self.q.shape[1]

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    @property
    def total_q(self) -> int:
        return self.q.shape[0]

    def to(self, device) -> "Problem":
        out = dataclasses.replace(self)
        for f in dataclasses.fields(self):
            val = getattr(self, f.name)
            if isinstance(val, torch.Tensor):
                setattr(out, f.name, val.to(device))
        return out


# --------------------------------------------------------------------------
# generator helpers
# --------------------------------------------------------------------------

def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device, chunk_elems=1 << 27):
    """N(0,1) fp32 drawn chunk by chunk (bounded transient memory)."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        out[s:e] = torch.randn(e - s, generator=g, device=device)
    return out.view(shape)


def _randn_cast(shape, g, device, dtype, chunk_elems=1 << 26):
    """N(0,1) cast to `dtype` (bf16 round-to-nearest-even, or fp8 e4m3fn)."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=dtype, device=device)
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        out[s:e] = torch.randn(e - s, generator=g, device=device).to(dtype)
    return out.view(shape)


def _randint(lo, hi, n, g) -> list:
    """n integers uniform in [lo, hi] inclusive, drawn on the CPU generator."""
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


# --------------------------------------------------------------------------
# E2M1 + E4M3 block-scale encoder (input tooling: produces stored bytes)
# --------------------------------------------------------------------------

# E2M1 magnitudes by 3-bit code (sign is bit 3 of the nibble).
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _e2m1_encode_rne(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 values to E2M1 codes (nibbles), ties to the even code,
    saturating at +-6.  Returns uint8 nibbles (0..15)."""
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=x.device)
    mag = x.abs().clamp(max=6.0)
    mids = (grid[1:] + grid[:-1]) * 0.5  # 7 midpoints
    # index of the nearest grid point, ties resolved below
    code = torch.bucketize(mag, mids, right=False)  # mag <= mid -> lower
    # at an exact midpoint bucketize(right=False) picks the lower code;
    # ties go to the even code instead
    at_mid = torch.zeros_like(mag, dtype=torch.bool)
    for i in range(7):
        at_mid |= (mag == mids[i]) & (code == i)
    odd_low = (code % 2) == 1
    code = torch.where(at_mid & odd_low, code + 1, code)
    sign = (x < 0) & (code > 0)
    return (code | (sign.to(code.dtype) << 3)).to(torch.uint8)


def quantize_e2m1_blocks(x: torch.Tensor, global_scale: float):
    """x (..., d) fp32 -> (packed uint8 (..., d//2), E4M3 scale bytes (..., d//16)).

    Per 16-value block: scale = E4M3_RNE(amax / (6 * global_scale)),
    code = E2M1_RNE(x / (scale * global_scale)); an all-zero block (or one
    whose scale rounds to zero) gets scale 0 and zero codes.  Element 2i is
    the low nibble of byte i.
    """
    *lead, d = x.shape
    xb = x.reshape(*lead, d // 16, 16)
    amax = xb.abs().amax(dim=-1)
    scale_f8 = (amax / (6.0 * global_scale)).to(torch.float8_e4m3fn)
    scale_f = scale_f8.to(torch.float32)
    denom = (scale_f * global_scale).unsqueeze(-1)
    safe = torch.where(denom > 0, denom, torch.ones_like(denom))
    codes = _e2m1_encode_rne(torch.where(denom > 0, xb / safe, torch.zeros_like(xb)))
    codes = codes.reshape(*lead, d)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).to(torch.uint8)
    return packed, scale_f8.view(torch.uint8)


# --------------------------------------------------------------------------
# layouts
# --------------------------------------------------------------------------

def _page_table(k_lens, g_cpu, device):
    """Pages of ceil(len/128) per request, assigned as consecutive slices of
    one random permutation of all pages; padded with -1."""
    npg = [(L + BLOCK - 1) // BLOCK for L in k_lens]
    total = sum(npg)
    perm = torch.randperm(total, generator=g_cpu).to(torch.int32)
    width = max(npg) if npg else 0
    pt = torch.full((len(k_lens), max(width, 1)), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(npg):
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt.to(device), total


def _cu(lens, device):
    c = [0]
    for L in lens:
        c.append(c[-1] + L)
    return torch.tensor(c, dtype=torch.int32, device=device)


def _kv_pool(shape, dtype_name, g, device, global_scale=1.0):
    """K or V storage: bf16 / fp8 e4m3fn (unit scale) / packed E2M1 + scales."""
    if dtype_name == KV_BF16:
        return _randn_cast(shape, g, device, torch.bfloat16), None
    if dtype_name == KV_F16:
        return _randn_cast(shape, g, device, torch.float16), None
    if dtype_name == KV_FP8:
        return _randn_cast(shape, g, device, torch.float8_e4m3fn), None
    if dtype_name == KV_E2M1:
        *lead, d = shape
        data = torch.empty((*lead, d // 2), dtype=torch.uint8, device=device)
        scl = torch.empty((*lead, d // 16), dtype=torch.uint8, device=device)
        flat_d = data.view(-1, d // 2)
        flat_s = scl.view(-1, d // 16)
        rows = flat_d.shape[0]
        step = max(1, (1 << 24) // d)
        for s in range(0, rows, step):
            e = min(rows, s + step)
            x = torch.randn((e - s, d), generator=g, device=device)
            pd, ps = quantize_e2m1_blocks(x, global_scale)
            flat_d[s:e] = pd
            flat_s[s:e] = ps
        return data, scl
    raise ValueError(dtype_name)


# --------------------------------------------------------------------------
# selections (synthetic q2k, not from scores)
# --------------------------------------------------------------------------

def _select_with_diagonal(n_valid, extra, topk, g_cpu):
    """The block of the token itself (n_valid - 1) plus `extra` distinct
    uniform blocks from [0, n_valid - 1), ascending, -1 padded."""
    last = n_valid - 1
    k = min(extra, last)
    row = [last]
    if k > 0:
        perm = torch.randperm(last, generator=g_cpu)[:k]
        row += [int(x) for x in perm]
    row.sort()
    return row + [-1] * (topk - len(row))


def random_q2k_diagonal(q_lens, k_lens, num_kv_heads, topk, g_cpu, extra=None,
                        causal=True):
    """Per (kv head, token): the causally-last block the token may see, plus
    min(topk - 1, available) distinct uniform earlier blocks."""
    extra = topk - 1 if extra is None else extra
    rows = []
    for g in range(num_kv_heads):
        per_g = []
        for Lq, Lk in zip(q_lens, k_lens):
            nblk = (Lk + BLOCK - 1) // BLOCK
            for iq in range(Lq):
                pos = Lk - Lq + iq if causal else Lk - 1
                n_valid = min(nblk, pos // BLOCK + 1) if pos >= 0 else 0
                if n_valid <= 0:
                    per_g.append([-1] * topk)
                else:
                    per_g.append(_select_with_diagonal(n_valid, extra, topk, g_cpu))
        rows.append(per_g)
    return torch.tensor(rows, dtype=torch.int32).reshape(num_kv_heads, sum(q_lens), topk)


def random_q2k_general(q_lens, k_lens, num_kv_heads, topk, g_cpu, p_empty=0.05,
                       p_short=0.2, allow_noncausal_blocks=True):
    """Irregular selections for parity tests: some rows empty, some shorter
    than topk, some selecting blocks above the causal limit (they must then
    contribute nothing); ascending, -1 padded, distinct."""
    rows = []
    for g in range(num_kv_heads):
        for Lq, Lk in zip(q_lens, k_lens):
            nblk = (Lk + BLOCK - 1) // BLOCK
            for iq in range(Lq):
                u = float(torch.rand((), generator=g_cpu))
                if nblk == 0 or u < p_empty:
                    rows.append([-1] * topk)
                    continue
                n = min(topk, nblk)
                if float(torch.rand((), generator=g_cpu)) < p_short:
                    n = int(torch.randint(1, n + 1, (), generator=g_cpu))
                if allow_noncausal_blocks:
                    pool = nblk
                else:
                    pos = Lk - Lq + iq
                    pool = max(1, min(nblk, pos // BLOCK + 1))
                    n = min(n, pool)
                sel = sorted(int(x) for x in torch.randperm(pool, generator=g_cpu)[:n])
                rows.append(sel + [-1] * (topk - len(sel)))
    return torch.tensor(rows, dtype=torch.int32).reshape(num_kv_heads, sum(q_lens), topk)


def decode_q2k_last_plus_random(k_lens, q_per_req, num_kv_heads, topk, g_cpu):
    """Decode selection: the last (partial) page plus topk-1 distinct uniform
    pages from [0, npg - 1), ascending; the same row for every token of a
    request."""
    rows = torch.full((num_kv_heads, len(k_lens) * q_per_req, topk), -1, dtype=torch.int32)
    for g in range(num_kv_heads):
        for b, Lk in enumerate(k_lens):
            npg = (Lk + BLOCK - 1) // BLOCK
            sel = _select_with_diagonal(npg, topk - 1, topk, g_cpu)
            for t in range(q_per_req):
                rows[g, b * q_per_req + t] = torch.tensor(sel, dtype=torch.int32)
    return rows


# --------------------------------------------------------------------------
# generic builder
# --------------------------------------------------------------------------

def make_problem(name, *, q_lens, k_lens, num_qo_heads, num_kv_heads, head_dim=128,
                 topk=16, paged=False, kv_dtype=KV_BF16, causal=True, seed=0,
                 device="cpu", selection="general", proxy_heads=0,
                 reduce_heads=False, softmax_scale=None, k_global_scale=None,
                 v_global_scale=None, extra_pages=0, max_k_tiles=None, g_cpu=None):
    """Build a Problem.  Draw order: lengths (given), page permutation, Q, K, V,
    proxy Q, selection randomness.

    selection: "general" (irregular rows), "diagonal" (own block + random
    earlier ones), "decode" (last page + random pages), or "proxy" (none:
    q2k comes from the proxy and top-K passes).
    """
    if g_cpu is None:
        g_cpu = _gen(seed, "cpu")
    g_dev = g_cpu if str(device) == "cpu" else _gen(seed, device)
    q_lens = tuple(int(x) for x in q_lens)
    k_lens = tuple(int(x) for x in k_lens)
    B = len(q_lens)
    total_q = sum(q_lens)
    d = head_dim
    cu_q = _cu(q_lens, device)

    page_table = seqused = cu_k = None
    if paged:
        page_table, npages = _page_table(k_lens, g_cpu, device)
        npages += extra_pages
        seqused = torch.tensor(k_lens, dtype=torch.int32, device=device)
        kv_shape = (npages, num_kv_heads, BLOCK, d)
    else:
        cu_k = _cu(k_lens, device)
        kv_shape = (sum(k_lens), num_kv_heads, d)

    qdt = torch.float16 if kv_dtype == KV_F16 else torch.bfloat16
    q = _randn_cast((total_q, num_qo_heads, d), g_dev, device, qdt)
    kgs = 1.0 if k_global_scale is None else k_global_scale
    vgs = 1.0 if v_global_scale is None else v_global_scale
    k, k_scale = _kv_pool(kv_shape, kv_dtype, g_dev, device, kgs)
    v, v_scale = _kv_pool(kv_shape, kv_dtype, g_dev, device, vgs)
    proxy_q = None
    if proxy_heads:
        proxy_q = _randn_cast((total_q, proxy_heads, d), g_dev, device, qdt)

    q2k = None
    if selection == "general":
        q2k = random_q2k_general(q_lens, k_lens, num_kv_heads, topk, g_cpu)
    elif selection == "diagonal":
        q2k = random_q2k_diagonal(q_lens, k_lens, num_kv_heads, topk, g_cpu)
    elif selection == "decode":
        assert len(set(q_lens)) == 1
        q2k = decode_q2k_last_plus_random(k_lens, q_lens[0], num_kv_heads, topk, g_cpu)
    elif selection == "proxy":
        q2k = None
    else:
        raise ValueError(selection)
    if q2k is not None:
        q2k = q2k.to(device)

    if max_k_tiles is None:
        max_k_tiles = max(((L + BLOCK - 1) // BLOCK for L in k_lens), default=0)
    return Problem(name=name, q=q, k=k, v=v, cu_seqlens_q=cu_q, kv_dtype=kv_dtype,
                   cu_seqlens_k=cu_k, page_table=page_table, seqused_k=seqused,
                   q2k=q2k, k_scale=k_scale, v_scale=v_scale, causal=causal,
                   softmax_scale=softmax_scale, k_global_scale=k_global_scale,
                   v_global_scale=v_global_scale, topk=topk, proxy_q=proxy_q,
                   reduce_heads=reduce_heads, max_k_tiles=max_k_tiles,
                   q_lens=q_lens, k_lens=k_lens)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------

WORKLOADS = (
    "flat_prefill_1x1024_h4kv1_top4",
    "flat_prefill_2x8192_h16kv2_top16_pipeline",
    "paged_decode_bf16_b64_h64kv4_top16",
    "paged_decode_fp8_mtp4_b32_h32kv2_top16",
    "paged_decode_e2m1_b128_h16kv1_top16",
)


def workload(name: str, device="cpu", seed=None) -> Problem:
    """The five synthetic workloads, each seeded with its 1-based position."""
    idx = WORKLOADS.index(name)
    seed = idx + 1 if seed is None else seed
    g_len = _gen(seed, "cpu")  # lengths first, then the rest of the stream
    if idx == 0:
        # 1 x 1024 causal prefill, 4 q heads / 1 kv head, topk 4; each token
        # selects its own block plus up to 3 distinct earlier blocks.
        return make_problem(name, q_lens=[1024], k_lens=[1024], num_qo_heads=4,
                            num_kv_heads=1, topk=4, seed=seed, device=device,
                            selection="diagonal", g_cpu=g_len)
    if idx == 1:
        # 2 x 8192 causal prefill; proxy Q with one indexer head per kv head.
        return make_problem(name, q_lens=[8192, 8192], k_lens=[8192, 8192],
                            num_qo_heads=16, num_kv_heads=2, topk=16, seed=seed,
                            device=device, selection="proxy", proxy_heads=2,
                            g_cpu=g_len)
    if idx == 2:
        lens = _randint(16384, 65536, 64, g_len)
        return make_problem(name, q_lens=[1] * 64, k_lens=lens, num_qo_heads=64,
                            num_kv_heads=4, topk=16, paged=True, seed=seed,
                            device=device, selection="decode", g_cpu=g_len)
    if idx == 3:
        lens = _randint(65536, 131072, 32, g_len)
        return make_problem(name, q_lens=[4] * 32, k_lens=lens, num_qo_heads=32,
                            num_kv_heads=2, topk=16, paged=True, kv_dtype=KV_FP8,
                            seed=seed, device=device, selection="proxy",
                            reduce_heads=True, g_cpu=g_len)
    if idx == 4:
        lens = _randint(32768, 131072, 128, g_len)
        return make_problem(name, q_lens=[1] * 128, k_lens=lens, num_qo_heads=16,
                            num_kv_heads=1, topk=16, paged=True, kv_dtype=KV_E2M1,
                            seed=seed, device=device, selection="decode",
                            k_global_scale=0.5, v_global_scale=2.0, g_cpu=g_len)
    raise ValueError(name)


# --------------------------------------------------------------------------
# QSA (packed query sparse attention over 4-token groups) inputs
# --------------------------------------------------------------------------

class QsaProblem:
    """q [T, Hq, d], k / v [T, Hkv, d] bf16 (packed sequences), indices
    [T, W] int32: per query, absolute token ids in groups of four, -1 padded;
    or (bitmap problems) bitmap uint8 [T, ceil(T / 4)] over 4-token blocks."""

    def __init__(self, name, q, k, v, indices, seq_lens, bitmap=None):
        self.name, self.q, self.k, self.v, self.indices = name, q, k, v, indices
        self.seq_lens = list(seq_lens)
        self.bitmap = bitmap

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device)
        return QsaProblem(self.name, mv(self.q), mv(self.k), mv(self.v), mv(self.indices),
                          self.seq_lens, mv(self.bitmap))


def qsa_indices(seq_lens, width, g_cpu, mode="random"):
    """Index rows of 4-token groups for packed causal sequences.

    Query at position p of a sequence starting at row c sees groups
    [4 j, 4 j + 3] of its sequence with 4 j <= p; its own group is the
    partial causal tail (entries past p are -1).  mode "causal": every
    visible group (the qsa page's example pattern, up to `width` entries:
    the latest groups); "random": the tail group plus distinct uniformly
    drawn earlier groups, ascending, up to width / 4 groups.
    """
    assert width % 4 == 0
    ng_max = width // 4
    T = sum(seq_lens)
    out = torch.full((T, width), -1, dtype=torch.int32)
    four = torch.arange(4)
    c = 0
    for L in seq_lens:
        for p in range(L):
            own = p // 4
            if mode == "causal":
                groups = torch.arange(max(0, own - ng_max + 1), own + 1)
            else:
                k = min(own, ng_max - 1)
                earlier = torch.randperm(own, generator=g_cpu)[:k] if own else torch.zeros(0, dtype=torch.long)
                groups = torch.cat([torch.sort(earlier).values, torch.tensor([own])])
            tok = (4 * groups.view(-1, 1) + four.view(1, -1)).reshape(-1)
            ids = torch.where(tok <= p, tok + c, torch.full_like(tok, -1))
            out[c + p, :ids.numel()] = ids.to(torch.int32)
        c += L
    return out


def make_qsa_problem(name, seq_lens, num_qo_heads, num_kv_heads, width, seed, head_dim=256,
                     device="cpu", mode="random"):
    """Seeded QSA inputs: lengths given; draws in the order indices (CPU
    generator), then Q, K, V (generator on `device`), N(0,1) cast to bf16."""
    g_cpu = _gen(seed, "cpu")
    indices = qsa_indices(seq_lens, width, g_cpu, mode)
    g = _gen(seed, device)
    T = sum(seq_lens)
    q = _randn_cast((T, num_qo_heads, head_dim), g, device, torch.bfloat16)
    k = _randn_cast((T, num_kv_heads, head_dim), g, device, torch.bfloat16)
    v = _randn_cast((T, num_kv_heads, head_dim), g, device, torch.bfloat16)
    return QsaProblem(name, q, k, v, indices.to(device), seq_lens)


QSA_WORKLOAD = "qsa_indexed_1x8192_h12kv1_d256_w2048"


def qsa_workload(device="cpu", seed=6):
    """One packed 8192-token sequence, 12 query heads / 1 KV head, head dim
    256, 2048-wide index rows (the tail group plus up to 511 random earlier
    groups per query)."""
    return make_qsa_problem(QSA_WORKLOAD, [8192], 12, 1, 2048, seed, device=device)


def qsa_bitmap(seq_lens, g_cpu, density, mode="random"):
    """uint8 [T, ceil(T / 4)] block maps over the packed tokens.

    mode "random": every block selected with probability `density`;
    "causal": blocks overlapping the query's own sequence up to its position,
    each with probability `density`, its own block always."""
    T = sum(seq_lens)
    nb = (T + 3) // 4
    draw = torch.rand(T, nb, generator=g_cpu) < density
    if mode == "random":
        return draw.to(torch.uint8)
    start = torch.cat([torch.full((L,), c, dtype=torch.long)
                       for L, c in zip(seq_lens, [0] + list(itertools.accumulate(seq_lens))[:-1])])
    pos = torch.arange(T)
    b = torch.arange(nb).view(1, -1)
    inside = (b >= (start // 4).view(-1, 1)) & (b <= (pos // 4).view(-1, 1))
    own = b == (pos // 4).view(-1, 1)
    return ((draw & inside) | own).to(torch.uint8)


def make_qsa_bitmap_problem(name, seq_lens, num_qo_heads, num_kv_heads, density, seed,
                            head_dim=256, device="cpu", mode="random"):
    """Seeded QSA bitmap inputs: the bitmap (CPU generator), then Q, K, V
    (generator on `device`), N(0,1) cast to bf16."""
    g_cpu = _gen(seed, "cpu")
    bitmap = qsa_bitmap(seq_lens, g_cpu, density, mode)
    g = _gen(seed, device)
    T = sum(seq_lens)
    q = _randn_cast((T, num_qo_heads, head_dim), g, device, torch.bfloat16)
    k = _randn_cast((T, num_kv_heads, head_dim), g, device, torch.bfloat16)
    v = _randn_cast((T, num_kv_heads, head_dim), g, device, torch.bfloat16)
    return QsaProblem(name, q, k, v, None, seq_lens, bitmap.to(device))


QSA_BITMAP_WORKLOAD = "qsa_bitmap_1x8192_h12kv1_d256_causal_q25"


def qsa_bitmap_workload(device="cpu", seed=9):
    """One packed 8192-token sequence, 12 query heads / 1 KV head, head dim
    256; each query's block map holds its own 4-token block plus a random
    quarter of its earlier blocks."""
    return make_qsa_bitmap_problem(QSA_BITMAP_WORKLOAD, [8192], 12, 1, 0.25, seed, device=device,
                                   mode="causal")
