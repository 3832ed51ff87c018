"""The decode captured in a HIP graph (torch's graph capture, which is hipGraph on ROCm).

On its normal path the call only enqueues kernels on the caller's stream (no allocation, copy,
memset or synchronisation), so a captured call must replay to exactly the bits of the eager
call. The graph's input buffers are refilled with a different input set between replays, as a
serving loop would, with eager decodes and synchronisations in between; every replay is
checked bit for bit against the eager result of the inputs it was given."""
import pytest
import torch

import workloads as W
from tests.gpu_helpers import gpu_decode, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)
M2 = dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128)
INPUTS = ("q_nope", "q_rope", "W_UK", "W_UV", "kv_pages", "page_table", "seq_lens")


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _inp(dims, lens, seed):
    return W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                         dims["d_v"], lens, seed)


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
def test_graph_replays_match_eager(M, dims):
    lens = [1, 33, 100, 190, 700]
    a = to_dev(_inp(dims, lens, 31))
    b = to_dev(_inp(dims, lens, 32))  # same shapes and lengths, other values

    def eager(d):
        o, l = gpu_decode(M, d, return_lse=True)
        torch.cuda.synchronize()
        return o, l

    ref = {"a": eager(a), "b": eager(b)}
    assert not torch.equal(ref["a"][0], ref["b"][0])

    # the graph's own buffers: inputs, outputs and workspace live as long as the graph
    st = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in a.items()}
    B, H, d_v = len(lens), dims["H"], dims["d_v"]
    out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    dm = M.make_dims(st["q_nope"], st["q_rope"], st["W_UK"], st["W_UV"], st["kv_pages"],
                     st["page_table"])
    ws = torch.empty(M.workspace_bytes(dm), dtype=torch.uint8, device="cuda")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one call before capture, off the default stream
        gpu_decode(M, st, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph capture", dims["d_c"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_decode(M, st, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()

    sets = {"a": a, "b": b}
    for rep, name in enumerate(["a", "b", "b", "a", "b"]):
        for k in INPUTS:
            st[k].copy_(sets[name][k])
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("graph replay", rep, name)
        assert torch.equal(out.view(torch.int16), ref[name][0].view(torch.int16)), (rep, name)
        assert torch.equal(lse.view(torch.int32), ref[name][1].view(torch.int32)), (rep, name)
        eager(sets["b" if name == "a" else "a"])  # eager work on the same stream in between
