"""GPU parity of the decompressed branch (T query tokens per sequence at or above the prefill
threshold, 256 unless the dims say otherwise) and of the switch between the two branches.

Both branches compute the same attention (the decompressed one expands K_nope = W_UK c_KV and
V = W_UV^T c_KV per head, the absorbed one folds W_UK into the query and W_UV into the output),
so both are held to the oracle's causal multi-token decode with the same tolerances, on both
sides of the threshold, at both widths, with sequences shorter than T (query rows with no
token to attend to: out = 0, lse = -inf)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import (LSE_ABS, MAX_ABS, REL_L2, HipEvents, errors, need_gpu, say,
                               to_dev)

pytestmark = pytest.mark.gpu

DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)
M2 = dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128)


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _inp(dims, lens, T, seed):
    inp = W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                        dims["d_v"], lens, seed)
    if T > 1:
        g = torch.Generator().manual_seed(seed + 1)
        B = len(lens)
        inp["q_nope"] = torch.randn(B, T, dims["H"], dims["d_n"], generator=g).to(torch.bfloat16)
        inp["q_rope"] = torch.randn(B, T, dims["H"], dims["d_R"], generator=g).to(torch.bfloat16)
    return inp


def _inp_pages(dims, lens, T, seed, max_pages):
    """_inp with the page-table rows (and so the per-sequence workspace rows) max_pages long."""
    inp = W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                        dims["d_v"], lens, seed, max_pages=max_pages)
    g = torch.Generator().manual_seed(seed + 1)
    B = len(lens)
    inp["q_nope"] = torch.randn(B, T, dims["H"], dims["d_n"], generator=g).to(torch.bfloat16)
    inp["q_rope"] = torch.randn(B, T, dims["H"], dims["d_R"], generator=g).to(torch.bfloat16)
    return inp


def _run(M, d, **kw):
    out, lse = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                        d["page_table"], d["seq_lens"], return_lse=True, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _oracle_rows(inp):
    """(out, lse) of the oracle for every (b, i, h): the causal multi-token decode for the
    sequences with at least T tokens; for a shorter one, row i with no token to attend to
    (S_b - T + i < 0) is out = 0, lse = -inf, and row i with context is the single-token
    decode over its first S_b - T + 1 + i tokens."""
    args = W.oracle_args(inp)
    if inp["q_nope"].dim() == 3:
        return oracle.decode(*args)
    qn, qr, wuk, wuv, kv, pt, sl = args
    B, T, H = qn.shape[0], qn.shape[1], qn.shape[2]
    d_v = wuv.shape[2]
    out = np.zeros((B, T, H, d_v))
    lse = np.full((B, T, H), -np.inf)
    full = [b for b in range(B) if sl[b] >= T]
    if full:
        o, l = oracle.decode_tokens(qn[full], qr[full], wuk, wuv, kv, pt[full], sl[full])
        out[full], lse[full] = o, l
    for b in range(B):
        if sl[b] >= T:
            continue
        for i in range(T - int(sl[b]), T):
            S = np.array([int(sl[b]) - T + 1 + i], dtype=np.int32)
            o, l = oracle.decode(qn[b, i][None], qr[b, i][None], wuk, wuv, kv, pt[b:b + 1], S)
            out[b, i], lse[b, i] = o[0], l[0]
    return out, lse


def _check(M, inp, label, **kw):
    d = to_dev(inp)
    out, lse = _run(M, d, **kw)
    ref, ref_lse = _oracle_rows(inp)
    rel, mx = errors(out, ref)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), label  # the rows with no token agree
    lerr = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    say(label, "rel_l2=%.3e max_abs=%.3e lse_err=%.3e" % (rel, mx, lerr))
    assert np.all(np.isfinite(out))
    assert np.all(out[~fin] == 0)
    assert rel <= REL_L2 and mx <= MAX_ABS and lerr <= LSE_ABS, (label, rel, mx, lerr)
    return out


@pytest.mark.parametrize("T", [1, 2, 16, 255, 256, 257, 512])
def test_mha2mla_across_the_threshold(M, T):
    # lengths: longer than T, equal to T, and shorter than T (its first rows attend to nothing);
    # at these widths the decompressed branch runs only with a threshold set (here 256)
    inp = _inp(M2, [T + 700, T, max(1, T // 2), T + 65], T, 10 + T)
    _check(M, inp, "mha2mla T=%d (%s branch)" % (T, "decompressed" if T >= 256 else "absorbed"),
           prefill_threshold=256)
    if T == 512:  # and without it, the absorbed branch serves any T
        _check(M, inp, "mha2mla T=512 absorbed")


@pytest.mark.parametrize("T", [256, 300])
def test_deepseek_decompressed(M, T):
    inp = _inp(DS, [T + 260, T, T - 100], T, 20 + T)
    _check(M, inp, "deepseek T=%d decompressed" % T)


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
def test_threshold_moves_the_branch(M, dims):
    # T = 200 and T = 300 each decoded by both branches: decompressed from a threshold at or
    # below T, absorbed with one above it. All four are held to the oracle, and each pair
    # agrees within the same bound.
    for T, lo, hi in ((200, 128, 1024), (300, 256, 512)):
        inp = _inp(dims, [T + 90, T + 1], T, 30 + T)
        a = _check(M, inp, "T=%d threshold %d" % (T, lo), prefill_threshold=lo)
        b = _check(M, inp, "T=%d threshold %d" % (T, hi), prefill_threshold=hi)
        rel, mx = errors(a, b)
        assert rel <= 2 * REL_L2 and mx <= 2 * MAX_ABS, (T, rel, mx)


def test_single_token_rows_through_the_decompressed_branch(M):
    # threshold 1: even one query token per sequence takes the decompressed branch
    inp = _inp(M2, [1, 63, 64, 65, 700], 1, 41)
    inp["q_nope"] = inp["q_nope"][:, None]
    inp["q_rope"] = inp["q_rope"][:, None]
    _check(M, inp, "T=1 decompressed", prefill_threshold=1)


def test_deepseek_prefill_groups(M):
    # more sequences than one group holds (1 GiB of decompressed keys and values: at
    # max_seq_len 16384 one sequence per group), so the branch loops over groups. Checked on
    # sampled (sequence, row, head) triples: row i of sequence b is the single-token decode
    # over its first S_b - T + 1 + i tokens.
    T = 256
    lens = [16384, 300, 2000]
    inp = _inp(DS, lens, T, 51)
    say("deepseek prefill groups")
    d = to_dev(inp)
    out, lse = _run(M, d)
    qn, qr, wuk, wuv, kv, pt, _ = W.oracle_args(inp)
    rng = np.random.default_rng(52)
    for b in range(3):
        for i in (0, 1, 127, 128, 255):
            heads = [int(h) for h in rng.choice(128, 4, replace=False)]
            S = np.array([lens[b] - T + 1 + i], dtype=np.int32)
            ref, ref_lse = oracle.decode(qn[b, i][None], qr[b, i][None], wuk, wuv, kv,
                                         pt[b:b + 1], S, pairs=[(0, h) for h in heads])
            rel, mx = errors(out[b, i, heads], ref)
            assert rel <= REL_L2 and mx <= MAX_ABS, (b, i, rel, mx)
            assert np.max(np.abs(lse[b, i, heads] - ref_lse)) <= LSE_ABS, (b, i)


def test_timed_entry_point_brackets_the_branch(M):
    inp = _inp(DS, [800, 400], 256, 61)
    d = to_dev(inp)
    hip = HipEvents()
    ev = [hip.create() for _ in range(6)]
    a = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                 d["page_table"], d["seq_lens"])
    b = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                 d["page_table"], d["seq_lens"], kernel_events=ev)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert hip.ms(ev[2], ev[3]) > 0
    assert hip.ms(ev[0], ev[1]) >= 0 and hip.ms(ev[4], ev[5]) >= 0
    for e in ev:
        hip.destroy(e)


def test_decompressed_branch_graph_replays_match_eager(M):
    # the decompressed branch captured in a HIP graph: transpose, then per group of sequences
    # the decompression and the attention (here two groups: at 16384 rows per sequence one
    # sequence fills a group), replayed with the inputs swapped between replays and eager work
    # in between; every replay bit for bit equal to the eager call on its inputs
    T = 256
    lens = [700, 300]
    a = to_dev(_inp_pages(DS, lens, T, 71, 256))
    b = to_dev(_inp_pages(DS, lens, T, 72, 256))

    def call(d, **kw):
        return M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                        d["page_table"], d["seq_lens"], return_lse=True, **kw)

    def eager(d):
        o, l = call(d)
        torch.cuda.synchronize()
        return o, l

    ref = {"a": eager(a), "b": eager(b)}
    assert not torch.equal(ref["a"][0], ref["b"][0])
    st = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in a.items()}
    out = torch.empty_like(ref["a"][0])
    lse = torch.empty_like(ref["a"][1])
    dm = M.make_dims(st["q_nope"], st["q_rope"], st["W_UK"], st["W_UV"], st["kv_pages"],
                     st["page_table"])
    ws = torch.empty(M.workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(st, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("prefill graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(st, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    sets = {"a": a, "b": b}
    for rep, name in enumerate(["b", "a", "b"]):
        for k in ("q_nope", "q_rope", "W_UK", "W_UV", "kv_pages", "page_table", "seq_lens"):
            st[k].copy_(sets[name][k])
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("prefill graph replay", rep, name)
        assert torch.equal(out.view(torch.int16), ref[name][0].view(torch.int16)), (rep, name)
        assert torch.equal(lse.view(torch.int32), ref[name][1].view(torch.int32)), (rep, name)
        eager(sets["a" if name == "b" else "b"])
