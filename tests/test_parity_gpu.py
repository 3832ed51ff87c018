"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded inputs.

Small cases span several tiles, ragged tails (lengths around the 32- and 64-token tile edges)
and many split plans; the five workloads run at full size in the launch configuration the
benchmark times (num_units = 0), with every (b, h) compared except for the 1M-token
workload, which compares a seeded sample of (b, h) pairs.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import check_against_oracle, need_gpu, say, to_dev, gpu_decode

pytestmark = pytest.mark.gpu

DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)
M2 = dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128)


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _inp(dims, lens, seed, **kw):
    return W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                         dims["d_v"], lens, seed, **kw)


@pytest.mark.parametrize("units", [0, 1, 2, 3, 5, 16, 64])
def test_deepseek_ragged(M, units):
    inp = _inp(DS, [1, 31, 32, 33, 300, 64 * 9 + 5], 11)
    check_against_oracle(M, inp, units=units, label="deepseek ragged")


@pytest.mark.parametrize("units", [0, 1, 2, 3, 7, 40])
def test_mha2mla_ragged(M, units):
    inp = _inp(M2, [1, 63, 64, 65, 1000, 130], 12)
    check_against_oracle(M, inp, units=units, label="mha2mla ragged")


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
@pytest.mark.parametrize("units", [1, 2])
def test_long_sequences_few_units(M, dims, units):
    # a unit walks more than 64 pages of one sequence (its page-table window refills inside
    # the unit) and then crosses into the next sequence
    inp = _inp(dims, [64 * 150 + 7, 64 * 70], 17)
    check_against_oracle(M, inp, units=units, label="long sequences, %d units" % units)


def test_deepseek_many_short_sequences(M):
    lens = [1 + (7 * i) % 90 for i in range(300)]  # more sequences than units
    check_against_oracle(M, _inp(DS, lens, 13), label="deepseek 300 short")


def test_mha2mla_many_short_sequences(M):
    lens = [1 + (11 * i) % 200 for i in range(200)]
    check_against_oracle(M, _inp(M2, lens, 14), label="mha2mla 200 short")


def test_explicit_scale_and_wide_logits(M):
    inp = _inp(DS, [200, 777], 15)
    inp["q_rope"] = (inp["q_rope"].float() * 4).to(torch.bfloat16)  # logits spread ~4x
    check_against_oracle(M, inp, label="deepseek wide logits")


@pytest.mark.parametrize("dims,heads", [(DS, [5, 37, 77, 126]), (M2, [5, 13, 30])],
                         ids=["deepseek", "mha2mla"])
@pytest.mark.parametrize("units", [1, 3])
def test_rescale_on_some_heads(M, dims, heads, units):
    # One late token per sequence whose RoPE logit is several hundred (log2 units) above every
    # other logit, for a few heads only, none of them the first of a block of 16: mid-segment
    # the running reference max of those heads moves far past the rescale threshold while that
    # of the other heads stays, so the rescale must reach exactly those heads' accumulators.
    # (The tokens sit in neither the first tile of a segment nor the first of a sequence.)
    inp = _inp(dims, [700, 1500], 18)
    qr = inp["q_rope"].float()
    for b in range(2):
        for h in heads:
            qr[b, h, :] = 0.0
            qr[b, h, 0] = 64.0
    inp["q_rope"] = qr.to(torch.bfloat16)
    for b, t in ((0, 650), (1, 1400)):
        page = int(inp["page_table"][b, t // 64])
        inp["kv_pages"][page, t % 64, dims["d_c"]] = 64.0
    check_against_oracle(M, inp, units=units, label="rescale on heads %s" % heads)


def test_empty_sequence_gives_zero_and_neg_inf(M):
    inp = _inp(DS, [100, 5, 64], 16)
    d = to_dev(inp)
    d["seq_lens"][1] = 0
    say("empty sequence")
    out, lse = gpu_decode(M, d, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out[1].float() == 0)
    assert torch.all(torch.isneginf(lse[1]))
    assert torch.isfinite(out[0].float()).all() and torch.isfinite(out[2].float()).all()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_full_size(M, cfg):
    inp = W.config_inputs(cfg)
    pairs = None
    if cfg == 4:  # 1M tokens: a seeded sample of (b, h), every sequence, spread over heads
        rng = np.random.default_rng(4)
        pairs = [(b, int(h)) for b in range(inp["B"]) for h in rng.choice(inp["H"], 8, False)]
    check_against_oracle(M, inp, pairs=pairs, label="workload %d %s" % (cfg, W.CONFIGS[cfg]["name"]))
