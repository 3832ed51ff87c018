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
