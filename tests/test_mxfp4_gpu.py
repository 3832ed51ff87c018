"""GPU parity of the MXFP4 latent cache (MHA2MLA widths): the decode over a cache of E2M1 codes
with an E8M0 scale per token and block of 32 latent elements, through mla_decode_mxfp4, against
the fp64 oracle run on the bf16 cache that the MXFP4 one stands for (oracle.dequant_mxfp4_cache;
every dequantised element is a bf16 value, so both sides see the same numbers and the bf16
bounds apply unchanged). The caches are synthetic: uniformly drawn codes and scale bytes
(workloads.mxfp4_cache), the k_R part and the page geometry of the bf16 inputs."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import LSE_ABS, MAX_ABS, REL_L2, errors, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

M2 = dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128)
DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _inp(lens, seed, dims=M2, **kw):
    return W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                         dims["d_v"], lens, seed, **kw)


def check_mx(M, inp, units=0, pairs=None, poison=False, label="", seed=5):
    kv4, sc = W.mxfp4_cache(inp, seed=seed, poison=poison)
    say(label, "mxfp4 B=%d units=%d T=%d" % (inp["B"], units,
                                              inp["q_nope"].shape[1] if inp["q_nope"].dim() == 4
                                              else 1))
    d = to_dev(inp)
    out, lse = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv4.cuda(),
                        d["page_table"], d["seq_lens"], num_units=units, return_lse=True,
                        kv_scales=sc.cuda())
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    args = list(W.oracle_args(inp))
    args[4] = oracle.dequant_mxfp4_cache(kv4.numpy(), sc.numpy(), inp["d_c"])
    if inp["q_nope"].dim() == 4:
        ref, ref_lse = oracle.decode_tokens(*args)
    else:
        ref, ref_lse = oracle.decode(*args, pairs=pairs)
    if pairs is not None:
        idx = np.asarray(pairs)
        out, lse = out[idx[:, 0], idx[:, 1]], lse[idx[:, 0], idx[:, 1]]
    rel, mx = errors(out, ref)
    lerr = float(np.max(np.abs(lse - ref_lse)))
    say(label, "rel_l2=%.3e max_abs=%.3e lse_err=%.3e" % (rel, mx, lerr))
    assert np.all(np.isfinite(out))
    assert rel <= REL_L2 and mx <= MAX_ABS and lerr <= LSE_ABS, (label, rel, mx, lerr)
    return out


@pytest.mark.parametrize("units", [0, 1, 2, 3, 7, 40])
def test_mxfp4_ragged(M, units):
    # lengths around the 64-token tile (one page) edge; 0xFF bytes and NaN scales (255) in
    # every slot no sequence uses
    inp = _inp([1, 63, 64, 65, 1000, 130], 12, poison=True)
    check_mx(M, inp, units=units, poison=True, label="mxfp4 ragged")


@pytest.mark.parametrize("units", [1, 2])
def test_mxfp4_long_sequences_few_units(M, units):
    # a unit walks more than 64 pages of one sequence and crosses into the next
    check_mx(M, _inp([64 * 150 + 7, 64 * 70], 17), units=units, label="mxfp4 long")


def test_mxfp4_many_short_sequences(M):
    lens = [1 + (11 * i) % 200 for i in range(200)]
    check_mx(M, _inp(lens, 14), label="mxfp4 200 short")


@pytest.mark.parametrize("T", [2, 4])
def test_mxfp4_query_tokens(M, T):
    inp = _inp([70, T, 200, 64 * 3 + 1], 31)
    g = torch.Generator().manual_seed(32)
    B = inp["B"]
    inp["q_nope"] = torch.randn(B, T, 32, 120, generator=g).to(torch.bfloat16)
    inp["q_rope"] = torch.randn(B, T, 32, 8, generator=g).to(torch.bfloat16)
    check_mx(M, inp, label="mxfp4 %d query tokens" % T)


def test_mxfp4_equals_bf16_on_the_same_values(M):
    # with the bf16 cache holding exactly the dequantised values, both paths form the same bf16
    # MFMA operands (the score operand converted in registers with the block's scale, the
    # values from the tile's bf16 copy) in the same order: bit-identical results
    inp = _inp([300, 64, 1000], 41)
    kv4, sc = W.mxfp4_cache(inp, seed=2)
    deq = oracle.dequant_mxfp4_cache(kv4.numpy(), sc.numpy(), inp["d_c"])
    inp["kv_pages"] = torch.from_numpy(deq.view(np.int16)).view(torch.bfloat16)
    d = to_dev(inp)
    for units in (0, 3):
        a, la = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv4.cuda(),
                         d["page_table"], d["seq_lens"], kv_scales=sc.cuda(), num_units=units,
                         return_lse=True)
        b, lb = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                         d["page_table"], d["seq_lens"], num_units=units, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(la, lb), units


def test_mxfp4_empty_sequence_gives_zero_and_neg_inf(M):
    inp = _inp([100, 5, 64], 86)
    kv4, sc = W.mxfp4_cache(inp, seed=1)
    d = to_dev(inp)
    d["seq_lens"][1] = 0
    out, lse = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv4.cuda(),
                        d["page_table"], d["seq_lens"], return_lse=True, kv_scales=sc.cuda())
    torch.cuda.synchronize()
    assert torch.all(out[1].float() == 0)
    assert torch.all(torch.isneginf(lse[1]))


def test_mxfp4_check_mode_flags_nan_scales(M):
    # MLA_CHECK=1 inspects every block scale of every slot a sequence uses: a 255 (E8M0's NaN)
    # there is reported (MLA_ERR_DEVICE_CHECK) and nothing is decoded; past a sequence's end it
    # is ignored
    inp = _inp([300, 64, 129], 51)
    kv4, sc = W.mxfp4_cache(inp, seed=6)
    d = to_dev(inp)
    pt = inp["page_table"].numpy()
    kv4 = kv4.cuda()

    def run(scales):
        o = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv4, d["page_table"],
                     d["seq_lens"], kv_scales=scales.cuda())
        torch.cuda.synchronize()
        return o

    ref = run(sc)
    os.environ["MLA_CHECK"] = "1"
    try:
        assert torch.equal(run(sc), ref)
        for b, tt, blk in ((0, 17, 0), (0, 299, 1), (1, 0, 1), (2, 128, 0)):
            s2 = sc.clone()
            s2[pt[b, tt // 64], tt % 64, blk] = 255
            say("mxfp4 check: NaN scale at sequence %d token %d block %d" % (b, tt, blk))
            with pytest.raises(M.MlaError) as e:
                run(s2)
            assert e.value.code == 7  # MLA_ERR_DEVICE_CHECK
        s2 = sc.clone()  # past the end of sequence 2 (129 tokens)
        s2[pt[2, 129 // 64], 129 % 64, 0] = 255
        assert torch.equal(run(s2), ref)
    finally:
        del os.environ["MLA_CHECK"]


def test_mxfp4_workload_full_size(M):
    # the MHA2MLA workload (B=32, S=32768) over an MXFP4 cache of its geometry, every (b, h)
    inp = W.config_inputs(5)
    check_mx(M, inp, label="mxfp4 workload 5")


def test_mxfp4_not_at_deepseek_widths(M):
    inp = _inp([64, 5], 90, DS)
    kv4, sc = W.mxfp4_cache(inp, seed=1)
    d = to_dev(inp)
    with pytest.raises(M.MlaError) as e:
        M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv4.cuda(), d["page_table"],
                 d["seq_lens"], kv_scales=sc.cuda())
    assert e.value.code == 5  # MLA_ERR_UNSUPPORTED
