"""GPU decode with the merged output projection (mla_decode_out) against the fp64 oracle:
out_hidden[b, n] = sum_{h,c} o_lat[b,h,c] W_UVO[n, h*d_c + c], at both widths, with one and
with two query tokens per sequence, and the lse equal to the plain decode's."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import LSE_ABS, MAX_ABS, REL_L2, errors, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)
M2 = dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128)


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _case(dims, lens, hidden, seed, T=1):
    inp = W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                        dims["d_v"], lens, seed)
    g = torch.Generator().manual_seed(seed + 1)
    K = dims["H"] * dims["d_c"]
    # the scale of W_UV W_O with the workloads' weights: variance 1 / (H d_c)
    W_UVO = (torch.randn(hidden, K, generator=g) / K ** 0.5).to(torch.bfloat16)
    if T > 1:
        B, H = len(lens), dims["H"]
        inp["q_nope"] = torch.randn(B, T, H, dims["d_n"], generator=g).to(torch.bfloat16)
        inp["q_rope"] = torch.randn(B, T, H, dims["d_R"], generator=g).to(torch.bfloat16)
    return inp, W_UVO


def _check(M, inp, W_UVO, label):
    say(label)
    d = to_dev(inp)
    out, lse = M.decode_out(d["q_nope"], d["q_rope"], d["W_UK"], W_UVO.cuda(), d["kv_pages"],
                            d["page_table"], d["seq_lens"], return_lse=True)
    torch.cuda.synchronize()
    a = W.oracle_args(inp)
    ref, ref_lse = oracle.decode_out(a[0], a[1], a[2], W.u16(W_UVO), a[4], a[5], a[6])
    rel, mx = errors(out.float().cpu().numpy(), ref)
    lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    say(label, "rel_l2=%.3e max_abs=%.3e lse_err=%.3e" % (rel, mx, lerr))
    assert rel <= REL_L2 and mx <= MAX_ABS and lerr <= LSE_ABS, (rel, mx, lerr)


@pytest.mark.parametrize("T", [1, 2])
def test_mha2mla_merged_output_projection(M, T):
    inp, W_UVO = _case(M2, [3, 64, 65, 1000, 300], 4096, 51, T)
    _check(M, inp, W_UVO, "mha2mla merged W_UV W_O, hidden 4096, %d query tokens" % T)


def test_deepseek_merged_output_projection(M):
    inp, W_UVO = _case(DS, [40, 300, 129], 256, 52)
    _check(M, inp, W_UVO, "deepseek merged W_UV W_O, hidden 256")


def test_mha2mla_full_size_merged(M):
    # the MHA2MLA workload's sequences (B = 32 of 32768 tokens) with the Llama-2-7B width
    inp = W.config_inputs(5)
    g = torch.Generator().manual_seed(53)
    W_UVO = (torch.randn(4096, 32 * 64, generator=g) / 2048 ** 0.5).to(torch.bfloat16)
    _check(M, inp, W_UVO, "mha2mla B=32 S=32768 merged, hidden 4096")
