"""mla_decode_noalloc: the decode whose scratch is an array built into the library.

It runs mla_decode's kernels on the same inputs, so its outputs must equal mla_decode's bit for
bit. Two calls in a row share the array, the second on a smaller input, so that anything the
first call left there and the second read would show up as a difference. Dims that need more
scratch than the array holds are refused on the host before anything is enqueued."""
import pytest
import torch

import workloads as W
from tests.gpu_helpers import gpu_decode, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)
M2 = dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128)


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _inp(dims, lens, seed):
    return W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                         dims["d_v"], lens, seed)


def _both(M, d, label):
    """(out, lse) of mla_decode and of mla_decode_noalloc on the same device inputs."""
    say("noalloc", label)
    B, H = d["q_nope"].shape[0], d["q_nope"].shape[1]
    d_v = d["W_UV"].shape[2]
    ref = gpu_decode(M, d, return_lse=True)
    out = torch.full((B, H, d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    got = gpu_decode(M, d, out=out, lse=lse, return_lse=True, no_alloc=True)
    torch.cuda.synchronize()
    assert got[0] is out and got[1] is lse
    return ref, got


@pytest.mark.parametrize("dims,big,small", [
    (DS, [4096, 1, 777, 2048, 64, 3000, 129, 4000], [5, 300, 63]),
    (M2, [8192, 4000, 1, 65, 6000, 129] * 4, [2, 1000, 64, 70]),
], ids=["deepseek", "mha2mla"])
def test_noalloc_matches_decode_twice(M, dims, big, small):
    a = to_dev(_inp(dims, big, 71))
    b = to_dev(_inp(dims, small, 72))
    need_a = M.workspace_bytes(M.make_dims(a["q_nope"], a["q_rope"], a["W_UK"], a["W_UV"],
                                           a["kv_pages"], a["page_table"]))
    assert 0 < need_a <= M.NOALLOC_SCRATCH_BYTES
    for d, label in ((a, "first, larger"), (b, "second, smaller")):
        ref, got = _both(M, d, "%s d_c=%d B=%d" % (label, dims["d_c"], len(d["seq_lens"])))
        assert torch.isfinite(got[0].float()).all()
        assert torch.equal(got[0], ref[0]), label
        assert torch.equal(got[1], ref[1]), label

