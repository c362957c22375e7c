"""QSA indexed forward (qsa page) through the C ABI against the fp64 oracle."""
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _check(p, out, out_f32, lse, what, rows=None):
    ref_out, ref_lse = oracle.qsa_indexed_attention(p.q.cpu(), p.k.cpu(), p.v.cpu(),
                                                    p.indices.cpu()) if rows is None else rows
    o = out.float().cpu().double()
    f = out_f32.cpu().double()
    l = lse.cpu().double()
    assert float((o - ref_out).abs().max()) <= 2e-2, what
    assert float((f - ref_out).abs().max()) <= 2e-2, what
    fin = torch.isfinite(ref_lse)
    assert torch.equal(torch.isfinite(l), fin), what
    assert float((l[fin] - ref_lse[fin]).abs().max()) <= 1e-3, what
    empty = torch.isneginf(ref_lse).T      # [T, Hq]
    assert (o[empty] == 0).all() and (f[empty] == 0).all(), what


@pytest.mark.parametrize("lens,hq,hkv,width,mode", [
    ([37, 50], 12, 1, 32, "random"),      # several chunks, ragged rows, packed ids
    ([70], 24, 2, 64, "causal"),          # 24/2: two KV heads, the page's pattern
    ([9, 3, 20], 12, 1, 2052, "random"),  # the widest rows, mostly padding
    ([33], 16, 2, 36, "random"),          # G = 8, width not a multiple of 32
    ([45, 20], 16, 1, 96, "random"),      # G = 16: every row of the MFMA tile live
    ([50], 16, 4, 64, "causal"),          # G = 4, four KV heads
])
def test_qsa_indexed_matches_oracle(msa, lens, hq, hkv, width, mode):
    print(f"qsa {lens} Hq {hq} Hkv {hkv} W {width} {mode}", flush=True)
    p = synth.make_qsa_problem("qsa", lens, hq, hkv, width, seed=len(lens) + width, mode=mode)
    d = p.to("cuda")
    out, out_f32, lse = msa.qsa_indexed_forward(d.q, d.k, d.v, d.indices)
    torch.cuda.synchronize()
    _check(p, out, out_f32, lse, f"qsa {lens} {hq}/{hkv} W {width}")


def test_qsa_empty_rows_strided_kv_and_repeatability(msa):
    p = synth.make_qsa_problem("qsa_edge", [40], 12, 1, 16, seed=5)
    idx = p.indices.clone()
    idx[3] = -1            # no key at all
    idx[7, 4:] = -1        # one group only
    p.indices = idx
    # K and V as views of one [Tk, 2, Hkv, 256] buffer (token stride 1 KiB)
    kv = torch.stack([p.k, p.v], dim=1).cuda()
    k, v = kv[:, 0], kv[:, 1]
    q, ind = p.q.cuda(), idx.cuda()
    a = msa.qsa_indexed_forward(q, k, v, ind)
    b = msa.qsa_indexed_forward(q, k, v, ind)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    _check(p, *a, "qsa edges")
    assert (a[0][3].float() == 0).all() and torch.isneginf(a[2][:, 3]).all()


def test_qsa_workload_every_row(msa):
    # the benchmark workload at full size, every query row against the oracle
    p = synth.qsa_workload(device="cpu")
    d = p.to("cuda")
    out, out_f32, lse = msa.qsa_indexed_forward(d.q, d.k, d.v, d.indices)
    torch.cuda.synchronize()
    o_all, of_all, l_all = out.float().cpu().double(), out_f32.cpu().double(), lse.cpu().double()
    for r0 in range(0, p.q.shape[0], 2048):
        rows = list(range(r0, min(r0 + 2048, p.q.shape[0])))
        print(f"qsa workload rows {rows[0]}..{rows[-1]}", flush=True)
        ref_out, ref_lse = oracle.qsa_indexed_attention(p.q[rows], p.k, p.v, p.indices[rows])
        assert float((o_all[rows] - ref_out).abs().max()) <= 2e-2
        assert float((of_all[rows] - ref_out).abs().max()) <= 2e-2
        fin = torch.isfinite(ref_lse)
        assert torch.equal(torch.isfinite(l_all[:, rows]), fin)
        assert float((l_all[:, rows][fin] - ref_lse[fin]).abs().max()) <= 1e-3


def _bitmap_rows(p):
    return oracle.qsa_bitmap_attention(p.q, p.k, p.v, p.bitmap)


@pytest.mark.parametrize("lens,hq,hkv,density,mode", [
    ([37, 50], 12, 1, 0.5, "random"),     # Tk = 87: the last block is cut at 3 tokens
    ([300], 24, 2, 0.4, "causal"),        # 75 blocks: two 64-block scan windows
    ([1000], 12, 1, 0.02, "random"),      # few blocks spread over 250: long empty scans
    ([9, 3, 20], 16, 2, 1.0, "random"),   # every block: the dense map
    ([130], 32, 2, 0.3, "causal"),        # G = 16
])
def test_qsa_bitmap_matches_oracle(msa, lens, hq, hkv, density, mode):
    print(f"qsa bitmap {lens} Hq {hq} Hkv {hkv} density {density} {mode}", flush=True)
    p = synth.make_qsa_bitmap_problem("qsa_bm", lens, hq, hkv, density, seed=len(lens) + 7,
                                      mode=mode)
    d = p.to("cuda")
    out, out_f32, lse = msa.qsa_bitmap_forward(d.q, d.k, d.v, d.bitmap)
    torch.cuda.synchronize()
    _check(p, out, out_f32, lse, f"qsa bitmap {lens} {hq}/{hkv}", rows=_bitmap_rows(p))


@pytest.mark.parametrize("tk,spread", [(517, False), (17000, False), (17000, True)])
def test_qsa_bitmap_hand_rows_and_indexed_equivalence(msa, tk, spread):
    # rows that exercise the block compaction: exactly 8 and 9 selected
    # blocks, hits at scan-window edges (63, 64, 127), an empty row, one
    # block.  Tk = 517 (130 blocks, the last one token long): shared-key
    # tiles; Tk = 17000: the tiles' keys fall in two 16384-key windows (row
    # 7 takes every block, row 11 the last one), still shared; spread: each
    # hand row alone in its 10-token tile (the others empty), so every tile
    # takes the per-token route and each token scans its own row
    T = 12
    p = synth.make_qsa_bitmap_problem("qsa_bm_hand", [T], 12, 1, 0.0, seed=3)
    k = synth._randn_cast((tk, 1, 256), synth._gen(4, "cpu"), "cpu", torch.bfloat16)
    v = synth._randn_cast((tk, 1, 256), synth._gen(5, "cpu"), "cpu", torch.bfloat16)
    bm = torch.zeros(T, (tk + 3) // 4, dtype=torch.uint8)
    bm[0, :8] = 1
    bm[1, :9] = 1
    bm[2, [63, 64, 127, 129]] = 1
    bm[4, 129] = 1                               # only the one-token block
    bm[5, ::2] = 7                               # any non-zero byte selects
    bm[6, 56:72] = 1                             # a run across the window edge
    bm[7] = 1
    bm[8, [0, 1, 2, 3, 4, 5, 6, 62, 63]] = 1
    bm[9, 120:] = 1
    bm[10, 64] = 1
    bm[11, [5, 70, 100]] = 1
    if tk > 16384:
        bm[11, -1] = 1
    q = p.q
    if spread:
        wide = torch.zeros(10 * T, bm.shape[1], dtype=torch.uint8)
        wide[::10] = bm
        bm = wide
        q = synth._randn_cast((10 * T, 12, 256), synth._gen(6, "cpu"), "cpu", torch.bfloat16)
        rows = [[int(x) for x in r if x >= 0] for r in oracle.qsa_bitmap_indices(bm, tk)]
        # (the empty row's tile lists nothing: the shared route's 0 / -inf)
        assert _qsa_routes(rows, 12) == ["token" if rows[10 * i] else "shared" for i in range(T)]
    T = bm.shape[0]
    p = synth.QsaProblem("qsa_bm_hand", q, k, v, None, [T], bm)
    d = p.to("cuda")
    out, out_f32, lse = msa.qsa_bitmap_forward(d.q, d.k, d.v, d.bitmap)
    torch.cuda.synchronize()
    _check(p, out, out_f32, lse, "qsa bitmap hand rows", rows=_bitmap_rows(p))
    empty = 30 if spread else 3
    assert torch.isneginf(lse[:, empty]).all() and (out[empty].float() == 0).all()
    if tk > 2052:
        return   # rows longer than the indexed entry point's widest
    # the indexed entry point over the same key lists (ascending, -1 padded)
    # consumes the same 32-token chunks: bitwise equal results
    ind = oracle.qsa_bitmap_indices(bm, tk).cuda()
    b = msa.qsa_indexed_forward(d.q, d.k, d.v, ind)
    torch.cuda.synchronize()
    assert torch.equal(out, b[0]) and torch.equal(out_f32, b[1]) and torch.equal(lse, b[2])


def test_qsa_bitmap_full_size_every_row(msa):
    # one 8192-token sequence, 12/1 heads, causal maps with a quarter of the
    # visible blocks: every query row against the oracle
    p = synth.make_qsa_bitmap_problem("qsa_bm_8192", [8192], 12, 1, 0.25, seed=8, mode="causal")
    d = p.to("cuda")
    out, out_f32, lse = msa.qsa_bitmap_forward(d.q, d.k, d.v, d.bitmap)
    torch.cuda.synchronize()
    o_all, l_all = out.float().cpu().double(), lse.cpu().double()
    for r0 in range(0, 8192, 2048):
        rows = list(range(r0, r0 + 2048))
        print(f"qsa bitmap rows {rows[0]}..{rows[-1]}", flush=True)
        ref_out, ref_lse = oracle.qsa_bitmap_attention(p.q[rows], p.k, p.v, p.bitmap[rows])
        assert float((o_all[rows] - ref_out).abs().max()) <= 2e-2
        fin = torch.isfinite(ref_lse)
        assert torch.equal(torch.isfinite(l_all[:, rows]), fin)
        assert float((l_all[:, rows][fin] - ref_lse[fin]).abs().max()) <= 1e-3


def test_qsa_bitmap_without_kv_tokens(msa):
    # Tk = 0: every query is empty (0 output, -inf LSE); nothing is read
    p = synth.make_qsa_problem("qsa_nokv", [5], 12, 1, 4, seed=2)
    q = p.q.cuda()
    k = torch.empty(0, 1, 256, dtype=torch.bfloat16, device="cuda")
    bm = torch.empty(5, 0, dtype=torch.uint8, device="cuda")
    out, out_f32, lse = msa.qsa_bitmap_forward(q, k, k, bm)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and (out_f32 == 0).all() and torch.isneginf(lse).all()


def _qsa_routes(rows, G):
    """The route each tile takes by the kernel's rule: tiles of
    min(16, 128 // G) consecutive tokens; the shared-key route unless the
    tile's listed keys fall in more than 64 windows of 16384 keys (from its
    lowest key) or 5 * union * ceil(live 16-row slots / 4) > 8 * listed
    entries."""
    tt = min(16, 128 // G)
    routes = []
    for t0 in range(0, len(rows), tt):
        tile = rows[t0:t0 + tt]
        keys = [k for r in tile for k in r if k >= 0]
        if not keys:
            routes.append("shared")
        elif (max(keys) - min(keys)) // 16384 + 1 > 64:
            routes.append("token")
        else:
            slots = (len(tile) * G + 15) // 16
            ok = 5 * len(set(keys)) * ((slots + 3) // 4) <= 8 * len(keys)
            routes.append("shared" if ok else "token")
    return routes


def _mixed_rows(tk, seed):
    # 10-token tiles (G = 12): tile 0 lists 48 of the same 64 keys per token
    # (shared keys), tile 1 eight random keys of 8000 per token (sparse: per
    # token), tile 2 64 keys spread over all tk rows (sparse over two key windows)
    g = torch.Generator().manual_seed(seed)
    rows = [sorted(torch.randperm(64, generator=g)[:48].tolist()) for _ in range(10)]
    rows += [torch.randperm(8000, generator=g)[:8].tolist() for _ in range(10)]
    rows += [torch.randperm(tk, generator=g)[:64].tolist() for _ in range(7)]
    return rows


@pytest.mark.parametrize("hq,hkv", [(12, 1), (24, 2)])
def test_qsa_shared_and_per_token_tiles_in_one_launch(msa, hq, hkv):
    tk = 20000
    rows = _mixed_rows(tk, seed=11 + hkv)
    assert _qsa_routes(rows, hq // hkv) == ["shared", "token", "token"]
    ind = torch.full((len(rows), 64), -1, dtype=torch.int32)
    for i, r in enumerate(rows):
        ind[i, :len(r)] = torch.tensor(r, dtype=torch.int32)
    g = synth._gen(21, "cpu")
    q = synth._randn_cast((len(rows), hq, 256), g, "cpu", torch.bfloat16)
    k = synth._randn_cast((tk, hkv, 256), g, "cpu", torch.bfloat16)
    v = synth._randn_cast((tk, hkv, 256), g, "cpu", torch.bfloat16)
    p = synth.QsaProblem("qsa_mixed", q, k, v, ind, [len(rows)])
    print(f"qsa mixed routes {hq}/{hkv} Tk {tk}", flush=True)
    d = p.to("cuda")
    a = msa.qsa_indexed_forward(d.q, d.k, d.v, d.indices)
    b = msa.qsa_indexed_forward(d.q, d.k, d.v, d.indices)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    _check(p, *a, f"qsa mixed routes {hq}/{hkv}")


def test_qsa_bitmap_shared_and_per_token_tiles(msa):
    # the same three kinds of tile through the bitmap entry point (Tk = 20001:
    # the last block one token long), then the indexed entry point over the
    # equivalent ascending rows: the same routes and chunks, bitwise equal
    tk, T = 20001, 27
    g = torch.Generator().manual_seed(5)
    nb = (tk + 3) // 4
    bm = torch.zeros(T, nb, dtype=torch.uint8)
    for i in range(10):
        bm[i, torch.randperm(16, generator=g)[:12]] = 1
    for i in range(10, 20):
        bm[i, torch.randperm(2000, generator=g)[:2]] = 1
    for i in range(20, T):
        bm[i, torch.randperm(nb, generator=g)[:16]] = 1
    bm[26, nb - 1] = 1
    full = oracle.qsa_bitmap_indices(bm, tk)
    rows = [[int(x) for x in r if x >= 0] for r in full]
    assert _qsa_routes(rows, 12) == ["shared", "token", "token"]
    gq = synth._gen(22, "cpu")
    q = synth._randn_cast((T, 12, 256), gq, "cpu", torch.bfloat16)
    k = synth._randn_cast((tk, 1, 256), gq, "cpu", torch.bfloat16)
    v = synth._randn_cast((tk, 1, 256), gq, "cpu", torch.bfloat16)
    p = synth.QsaProblem("qsa_bm_mixed", q, k, v, None, [T], bm)
    print("qsa bitmap mixed routes", flush=True)
    d = p.to("cuda")
    out, out_f32, lse = msa.qsa_bitmap_forward(d.q, d.k, d.v, d.bitmap)
    torch.cuda.synchronize()
    _check(p, out, out_f32, lse, "qsa bitmap mixed routes", rows=_bitmap_rows(p))
    w = (max(len(r) for r in rows) + 3) // 4 * 4
    b = msa.qsa_indexed_forward(d.q, d.k, d.v, full[:, :w].contiguous().cuda())
    torch.cuda.synchronize()
    assert torch.equal(out, b[0]) and torch.equal(out_f32, b[1]) and torch.equal(lse, b[2])


def test_qsa_24_2_full_size_sampled_rows(msa):
    # the page's other head configuration at the workload's size: 8192
    # packed tokens in two sequences, 24 query / 2 KV heads, 2048-wide random
    # rows; every 8th token (all 24 heads) against the oracle
    p = synth.make_qsa_problem("qsa_24_2", [5000, 3192], 24, 2, 2048, seed=31)
    d = p.to("cuda")
    out, out_f32, lse = msa.qsa_indexed_forward(d.q, d.k, d.v, d.indices)
    torch.cuda.synchronize()
    rows = list(range(0, 8192, 8))
    print("qsa 24/2 full size, sampled rows", flush=True)
    ref_out, ref_lse = oracle.qsa_indexed_attention(p.q[rows], p.k, p.v, p.indices[rows])
    o = out.float().cpu().double()[rows]
    f = out_f32.cpu().double()[rows]
    l = lse.cpu().double()[:, rows]
    assert float((o - ref_out).abs().max()) <= 2e-2
    assert float((f - ref_out).abs().max()) <= 2e-2
    fin = torch.isfinite(ref_lse)
    assert torch.equal(torch.isfinite(l), fin)
    assert float((l[fin] - ref_lse[fin]).abs().max()) <= 1e-3


@pytest.mark.parametrize("hq,hkv", [(12, 1), (24, 2)])
def test_qsa_shared_tiles_over_several_key_windows(msa, hq, hkv):
    # keys over 40 000 tokens, three 16384-key windows per tile: tile 0
    # lists the same 1500 keys spread over every window, tile 1 the same 600
    # keys in the first and last windows only (the middle one empty), tile 2
    # a dense run in the first window; all three share keys
    tk = 40000
    g = torch.Generator().manual_seed(hkv)
    spread = torch.randperm(tk, generator=g)[:1500]
    ends = torch.cat([torch.randperm(300, generator=g), tk - 1 - torch.randperm(300, generator=g)])
    rows = [torch.sort(spread).values.tolist()] * 10
    rows += [ends.tolist()] * 10
    rows += [list(range(i, 512 + i, 2)) for i in range(7)]
    assert _qsa_routes(rows, hq // hkv) == ["shared"] * 3
    ind = torch.full((len(rows), 1500), -1, dtype=torch.int32)
    for i, r in enumerate(rows):
        ind[i, :len(r)] = torch.tensor(r, dtype=torch.int32)
    gq = synth._gen(40 + hkv, "cpu")
    q = synth._randn_cast((len(rows), hq, 256), gq, "cpu", torch.bfloat16)
    k = synth._randn_cast((tk, hkv, 256), gq, "cpu", torch.bfloat16)
    v = synth._randn_cast((tk, hkv, 256), gq, "cpu", torch.bfloat16)
    p = synth.QsaProblem("qsa_windows", q, k, v, ind, [len(rows)])
    print(f"qsa shared windows {hq}/{hkv} Tk {tk}", flush=True)
    d = p.to("cuda")
    a = msa.qsa_indexed_forward(d.q, d.k, d.v, d.indices)
    b = msa.qsa_indexed_forward(d.q, d.k, d.v, d.indices)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    _check(p, *a, f"qsa shared windows {hq}/{hkv}")


def test_qsa_bitmap_dense_map_over_several_windows(msa):
    # a half-density random map over 40 001 tokens (10 001 blocks, the last
    # one token long): three windows per tile, shared keys; an empty row
    tk, T = 40001, 25
    g = torch.Generator().manual_seed(9)
    nb = (tk + 3) // 4
    bm = (torch.rand(T, nb, generator=g) < 0.5).to(torch.uint8)
    bm[4] = 0
    bm[5, nb - 1] = 1
    full = oracle.qsa_bitmap_indices(bm, tk)
    rows = [[int(x) for x in r if x >= 0] for r in full]
    assert _qsa_routes(rows, 12) == ["shared"] * 3
    gq = synth._gen(23, "cpu")
    q = synth._randn_cast((T, 12, 256), gq, "cpu", torch.bfloat16)
    k = synth._randn_cast((tk, 1, 256), gq, "cpu", torch.bfloat16)
    v = synth._randn_cast((tk, 1, 256), gq, "cpu", torch.bfloat16)
    p = synth.QsaProblem("qsa_bm_windows", q, k, v, None, [T], bm)
    print("qsa bitmap windows", flush=True)
    d = p.to("cuda")
    out, out_f32, lse = msa.qsa_bitmap_forward(d.q, d.k, d.v, d.bitmap)
    torch.cuda.synchronize()
    _check(p, out, out_f32, lse, "qsa bitmap windows", rows=_bitmap_rows(p))
    assert torch.isneginf(lse[:, 4]).all() and (out[4].float() == 0).all()
