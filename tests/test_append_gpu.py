"""GPU cache append (mla_cache_append) against the fp64 oracle: the written [c_KV | k_R] rows
within half a bf16 ulp (plus fp32 summation noise) of the exact values, every other cache byte
unchanged, tokens past the page-table row not written, and the decode reading what was
appended."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import check_against_oracle, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

SHAPES = {"deepseek": dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128, hidden=7168),
          "mha2mla": dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128, hidden=4096)}


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _case(shape, lens, T, seed, max_pages=None):
    c = SHAPES[shape]
    # the cache holds room for the T new tokens of every sequence
    inp = W.make_inputs(len(lens), c["H"], c["d_n"], c["d_c"], c["d_R"], c["d_v"],
                        [s + T for s in lens], seed, max_pages=max_pages)
    g = torch.Generator().manual_seed(seed + 1)
    B, hidden = len(lens), c["hidden"]
    x = torch.randn(B, T, hidden, generator=g).to(torch.bfloat16)
    Wd = (torch.randn(c["d_c"], hidden, generator=g) / hidden ** 0.5).to(torch.bfloat16)
    Wr = (torch.randn(c["d_R"], hidden, generator=g) / hidden ** 0.5).to(torch.bfloat16)
    before = torch.tensor(lens, dtype=torch.int32)
    return inp, x, Wd, Wr, before


def _append_and_check(M, shape, lens, T, seed):
    inp, x, Wd, Wr, before = _case(shape, lens, T, seed)
    say("append", shape, "B=%d T=%d" % (len(lens), T))
    kv0 = inp["kv_pages"].clone()
    kv = inp["kv_pages"].cuda()
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, inp["page_table"].cuda(), before.cuda())
    torch.cuda.synchronize()
    got = kv.cpu()
    rows, where = oracle.cache_append(W.u16(x), W.u16(Wd), W.u16(Wr), inp["page_table"].numpy(),
                                      before.numpy())
    written = np.zeros(got.shape[:2], dtype=bool)
    for b in range(len(lens)):
        for i in range(T):
            page, slot = where[b, i]
            g = got[page, slot].double().numpy()
            ref = rows[b, i]
            err = np.abs(g - ref)
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), (b, i, float(err.max()))
            written[page, slot] = True
    same = got.view(torch.int16).numpy()[~written] == kv0.view(torch.int16).numpy()[~written]
    assert np.all(same), "a cache slot other than the new tokens' changed"
    return inp, kv, before


@pytest.mark.parametrize("shape,lens,T", [("deepseek", [62, 64, 500], 2),
                                          ("deepseek", [1 + 37 * i for i in range(16)], 1),
                                          ("mha2mla", [1, 63, 64, 1000], 3)])
def test_append_matches_oracle(M, shape, lens, T):
    _append_and_check(M, shape, lens, T, 41)


def test_tokens_past_the_page_table_row_are_not_written(M):
    c = SHAPES["deepseek"]
    inp = W.make_inputs(2, c["H"], c["d_n"], c["d_c"], c["d_R"], c["d_v"], [64, 64], 42)
    g = torch.Generator().manual_seed(43)
    x = torch.randn(2, 3, c["hidden"], generator=g).to(torch.bfloat16)
    Wd = (torch.randn(c["d_c"], c["hidden"], generator=g) / 85).to(torch.bfloat16)
    Wr = (torch.randn(c["d_R"], c["hidden"], generator=g) / 85).to(torch.bfloat16)
    before = torch.tensor([63, 64], dtype=torch.int32)  # one page per row: only slot 63 fits
    say("append past the row")
    kv0 = inp["kv_pages"].clone()
    kv = inp["kv_pages"].cuda()
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, inp["page_table"].cuda(), before.cuda())
    torch.cuda.synchronize()
    got = kv.cpu()
    p0 = int(inp["page_table"][0, 0])
    changed = (got.view(torch.int16) != kv0.view(torch.int16)).any(dim=2)
    assert changed[p0, 63] and int(changed.sum()) == 1


def test_decode_reads_appended_tokens(M):
    # append one token to each of 3 sequences on the GPU, then decode over the longer
    # sequences; the oracle decodes the same cache bytes
    inp, kv, before = _append_and_check(M, "deepseek", [100, 64, 300], 1, 44)
    inp["kv_pages"] = kv.cpu()
    inp["seq_lens"] = before + 1
    check_against_oracle(M, inp, label="decode after append")


def test_unallocated_page_entry_is_not_written(M):
    # a new token whose page-table entry names no pool page (-1: not allocated yet, or past
    # the pool) is skipped: every other slot of the pool stays bit for bit as it was, and the
    # tokens with valid entries are written as usual
    inp, x, Wd, Wr, before = _case("mha2mla", [62, 130, 5], 3, 45)
    pt = inp["page_table"].clone()
    pt[0, 1] = -1                         # page of position 64 (sequence 0's third new token)
    pt[1, 2] = inp["kv_pages"].shape[0]   # past the pool: positions 128.. of sequence 1
    say("append with unallocated page entries")
    kv0 = inp["kv_pages"].clone()
    kv = inp["kv_pages"].cuda()
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, pt.cuda(), before.cuda())
    torch.cuda.synchronize()
    got = kv.cpu()
    rows, where = oracle.cache_append(W.u16(x), W.u16(Wd), W.u16(Wr), pt.numpy(),
                                      before.numpy())
    written = np.zeros(got.shape[:2], dtype=bool)
    skipped = 0
    for b in range(3):
        for i in range(3):
            page, slot = where[b, i]
            if page < 0 or page >= got.shape[0]:
                skipped += 1
                continue
            ref = rows[b, i]
            err = np.abs(got[page, slot].double().numpy() - ref)
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), (b, i, float(err.max()))
            written[page, slot] = True
    assert skipped == 4  # sequence 0: position 64; sequence 1: positions 130, 131, 132
    same = got.view(torch.int16).numpy()[~written] == kv0.view(torch.int16).numpy()[~written]
    assert np.all(same), "a slot outside the valid new tokens changed"


def test_check_mode_refuses_unallocated_page_entry(M):
    import os
    inp, x, Wd, Wr, before = _case("mha2mla", [62, 10], 3, 46)
    pt = inp["page_table"].clone()
    pt[0, 1] = -1
    kv0 = inp["kv_pages"].clone()
    kv = inp["kv_pages"].cuda()
    old = os.environ.get("MLA_CHECK")
    os.environ["MLA_CHECK"] = "1"
    try:
        say("append check mode: -1 entry")
        with pytest.raises(M.MlaError) as e:
            M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, pt.cuda(), before.cuda())
        assert e.value.code == 7  # MLA_ERR_DEVICE_CHECK
        torch.cuda.synchronize()
        assert torch.equal(kv.cpu().view(torch.int16), kv0.view(torch.int16))  # nothing written
        # valid entries pass the check and are appended
        M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, inp["page_table"].cuda(),
                       before.cuda())
        torch.cuda.synchronize()
        assert not torch.equal(kv.cpu().view(torch.int16), kv0.view(torch.int16))
    finally:
        if old is None:
            del os.environ["MLA_CHECK"]
        else:
            os.environ["MLA_CHECK"] = old
