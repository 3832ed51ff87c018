"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded inputs.

Small cases span several tiles, ragged tails (lengths around the 32- and 64-token tile edges)
and many split plans; the five workloads run at full size in the launch configuration the
benchmark times (num_units = 0), with every (b, h) compared. Each check also reports the worst
(b, h) row's relative error and the worst element error against the largest output.
"""
import numpy as np
import pytest
import torch

import workloads as W
import oracle
from tests.gpu_helpers import check_against_oracle, errors, need_gpu, say, to_dev, gpu_decode

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
    # every (b, h) of each workload, the 1M-token one included (a few seconds of the oracle on
    # the host's cores)
    inp = W.config_inputs(cfg)
    check_against_oracle(M, inp, label="workload %d %s" % (cfg, W.CONFIGS[cfg]["name"]))


# ---- several query tokens per sequence (the T newest tokens, causal among themselves)

def _with_tokens(inp, T, seed):
    g = torch.Generator().manual_seed(seed)
    B, H, d_n, d_R = inp["B"], inp["H"], inp["d_n"], inp["d_R"]
    inp["q_nope"] = torch.randn(B, T, H, d_n, generator=g).to(torch.bfloat16)
    inp["q_rope"] = torch.randn(B, T, H, d_R, generator=g).to(torch.bfloat16)
    return inp


@pytest.mark.parametrize("T", [2, 4])
@pytest.mark.parametrize("units", [0, 1, 5])
def test_deepseek_query_tokens(M, T, units):
    inp = _with_tokens(_inp(DS, [4, 31, 33, 300, 64 * 9 + 5], 31), T, 32)
    check_against_oracle(M, inp, units=units, label="deepseek %d query tokens" % T)


@pytest.mark.parametrize("T", [2, 3])
@pytest.mark.parametrize("units", [0, 3])
def test_mha2mla_query_tokens(M, T, units):
    inp = _with_tokens(_inp(M2, [4, 63, 65, 1000], 33), T, 34)
    check_against_oracle(M, inp, units=units, label="mha2mla %d query tokens" % T)


def test_query_tokens_full_size(M):
    # B = 16 sequences of 4096 tokens with two query tokens each (shuffled pages)
    inp = _with_tokens(W.config_inputs(2), 2, 35)
    check_against_oracle(M, inp, label="deepseek B=16 S=4096, 2 query tokens")


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
def test_one_query_token_as_4d_is_plain_decode(M, dims):
    inp = _inp(dims, [70, 300, 129], 36)
    d = to_dev(inp)
    say("4-d query, one token", dims["d_c"])
    o3 = gpu_decode(M, d)
    d4 = dict(d)
    d4["q_nope"] = d["q_nope"][:, None].contiguous()
    d4["q_rope"] = d["q_rope"][:, None].contiguous()
    o4 = gpu_decode(M, d4)
    torch.cuda.synchronize()
    assert o4.shape == (3, 1, dims["H"], dims["d_v"])
    assert torch.equal(o3.view(torch.int16), o4[:, 0].view(torch.int16))


def test_query_tokens_without_context(M):
    # S_b = 1 with 3 query tokens: tokens 0 and 1 of that sequence have nothing to attend to
    # (out = 0, lse = -inf); token 2 is the sequence's only cached token and sees it alone
    inp = _with_tokens(_inp(DS, [1, 200], 37), 3, 38)
    d = to_dev(inp)
    say("query tokens without context")
    out, lse = gpu_decode(M, d, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out[0, :2].float() == 0) and torch.all(torch.isneginf(lse[0, :2]))
    one = dict(inp)
    one["q_nope"], one["q_rope"] = inp["q_nope"][:, 2], inp["q_rope"][:, 2]
    ref, ref_lse = oracle.decode(*W.oracle_args(one))
    rel, mx = errors(out[:, 2].float().cpu().numpy()[:1], ref[:1])
    assert rel <= 5e-3 and mx <= 2e-2, (rel, mx)
    assert np.max(np.abs(lse[0, 2].cpu().numpy() - ref_lse[0])) <= 1e-2


def test_more_sequences_than_the_plan_keeps_in_lds(M):
    # over 4096 sequences: the plan builder walks the units from each sequence instead of
    # searching offsets held in LDS
    lens = [1 + (13 * i) % 40 for i in range(4200)]
    check_against_oracle(M, _inp(DS, lens, 39), label="deepseek 4200 short")


def test_query_tokens_over_4096_rows(M):
    # 2100 sequences x 2 query tokens = 4200 virtual sequences (the same plan path)
    lens = [2 + (7 * i) % 30 for i in range(2100)]
    inp = _with_tokens(_inp(M2, lens, 40), 2, 41)
    check_against_oracle(M, inp, label="mha2mla 2100 x 2 query tokens")
