"""Device-side check of the sparse attention caller contracts
(msa_validate_attention, and MSA_VALIDATE=1 in front of msa_sparse_attention).

Every broken input here goes to the check alone, which never launches the
attention; the one call that runs the attention under MSA_VALIDATE uses a
violation the attention kernels tolerate (a row out of order)."""
import pytest
import torch

import synth
from gpu_helpers import gpu_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_top_msa_amd as m
    return m


def _validate(msa, p, q2k=None, cu_seqlens_q=None, cu_seqlens_k=None, page_table=None,
              seqused_k=None, max_seqlen_q=None):
    pick = lambda x, y: y if x is None else x
    msa.validate_attention(
        p.q, p.k, p.v, pick(q2k, p.q2k), pick(cu_seqlens_q, p.cu_seqlens_q),
        pick(cu_seqlens_k, p.cu_seqlens_k), causal=p.causal,
        page_table=pick(page_table, p.page_table), seqused_k=pick(seqused_k, p.seqused_k),
        k_scale=p.k_scale, v_scale=p.v_scale,
        max_seqlen_q=pick(max_seqlen_q, max(p.q_lens)), max_k_tiles=p.max_k_tiles)


def _broken(msa, p, text, **kw):
    with pytest.raises(msa.MsaError) as e:
        _validate(msa, p, **kw)
    assert e.value.status == 8, str(e.value)
    assert text in str(e.value), str(e.value)


@pytest.fixture(scope="module")
def flat(msa):
    return synth.make_problem("val_flat", q_lens=[300, 77], k_lens=[300, 500], num_qo_heads=8,
                              num_kv_heads=2, topk=5, seed=41).to("cuda")


@pytest.fixture(scope="module")
def paged(msa):
    return synth.make_problem("val_paged", q_lens=[1, 1, 1], k_lens=[2000, 129, 700],
                              num_qo_heads=16, num_kv_heads=2, topk=8, paged=True, seed=42,
                              selection="decode").to("cuda")


def test_valid_inputs_pass(msa, flat, paged):
    print("validate: valid flat and paged inputs", flush=True)
    _validate(msa, flat)
    _validate(msa, paged)
    e2m1 = synth.make_problem("val_e2m1", q_lens=[1, 1], k_lens=[256, 200], num_qo_heads=16,
                              num_kv_heads=1, topk=4, paged=True, kv_dtype=synth.KV_E2M1,
                              seed=43, selection="decode").to("cuda")
    _validate(msa, e2m1)
    torch.cuda.synchronize()


def test_q2k_order_and_padding(msa, flat):
    print("validate: q2k order and padding", flush=True)
    q2k = flat.q2k.clone()
    row = q2k[1, 200]
    n = int((row >= 0).sum())
    assert n >= 2
    q2k[1, 200, 0], q2k[1, 200, 1] = row[1].item(), row[0].item()
    _broken(msa, flat, "q2k[g=1, i=200] entry 1 is not above", q2k=q2k)
    q2k = flat.q2k.clone()
    q2k[0, 7, 1] = q2k[0, 7, 0]
    if int(q2k[0, 7, 0]) >= 0:
        _broken(msa, flat, "q2k[g=0, i=7] entry 1 is not above", q2k=q2k)
    q2k = flat.q2k.clone()
    q2k[0, 5, :] = -1
    q2k[0, 5, 3] = 0
    _broken(msa, flat, "q2k[g=0, i=5] entry 3 follows -1 padding", q2k=q2k)
    # block ids past the sequence are ignored by the attention, not a violation
    q2k = flat.q2k.clone()
    assert q2k[0, 0].tolist() == [0, 1, 2, -1, -1]
    q2k[0, 0, 3] = 1000
    _validate(msa, flat, q2k=q2k)


def test_sequence_offsets_and_lengths(msa, flat, paged):
    print("validate: cu_seqlens, KV lengths", flush=True)
    cu = flat.cu_seqlens_q.clone()
    cu[2] = cu[2] - 1                                  # ends before total_q
    _broken(msa, flat, "cu_seqlens_q at request 2", cu_seqlens_q=cu)
    cu = flat.cu_seqlens_q.clone()
    cu[1] = cu[2] + 5                                  # a negative second length
    _broken(msa, flat, "cu_seqlens_q at request", cu_seqlens_q=cu)
    _broken(msa, flat, "cu_seqlens_q at request 0", max_seqlen_q=200)   # 300 > 200
    cuk = flat.cu_seqlens_k.clone()
    cuk[1] = cuk[2] + 1
    _broken(msa, flat, "cu_seqlens_k decreases after request 1", cu_seqlens_k=cuk)
    su = paged.seqused_k.clone()
    su[1] = 128 * paged.page_table.shape[1] + 1        # more keys than the table holds
    _broken(msa, paged, "KV length of request 1", seqused_k=su)
    su = paged.seqused_k.clone()
    su[2] = -3
    _broken(msa, paged, "KV length of request 2", seqused_k=su)


def test_page_table_entries(msa, paged):
    print("validate: page ids", flush=True)
    pt = paged.page_table.clone()
    sel = set(int(x) for x in paged.q2k[:, 0].flatten().tolist() if x >= 0)
    t = next(t for t in range((2000 + 127) // 128) if t not in sel)
    pt[0, t] = -1                                      # a hole inside request 0's pages
    _broken(msa, paged, f"page_table[0, {t}] is negative", page_table=pt)
    pt = paged.page_table.clone()
    pt[1, 5] = -7                                      # past request 1's two pages: padding
    _validate(msa, paged, page_table=pt)


def test_env_switch_checks_before_the_attention(msa, flat, monkeypatch):
    print("validate: MSA_VALIDATE=1", flush=True)
    ref = gpu_attention(msa, flat)
    monkeypatch.setenv("MSA_VALIDATE", "1")
    got = gpu_attention(msa, flat)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    q2k = flat.q2k.clone()
    q2k[1, 200] = q2k[1, 200].flip(0)                 # out of order (tolerated by the kernels)
    out = torch.full_like(flat.q, 7.0)
    with pytest.raises(msa.MsaError) as e:
        msa.sparse_attention(flat.q, flat.k, flat.v, q2k, flat.cu_seqlens_q, flat.cu_seqlens_k,
                             causal=flat.causal, max_seqlen_q=max(flat.q_lens),
                             max_k_tiles=flat.max_k_tiles, out=out)
    assert e.value.status == 8 and "q2k[g=1, i=200]" in str(e.value)
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()                  # nothing was launched
