"""GPU invariants that hold exactly: bit-exact page gathers, bit-identical outputs under
page-table permutation and under poisoned (NaN) unused cache slots and pages, softmax rows
summing to one, run-to-run determinism, and split-plan invariance within tolerance."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import REL_L2, HipEvents, errors, gpu_decode, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)
M2 = dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128)


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _inp(dims, lens, seed, **kw):
    return W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                         dims["d_v"], lens, seed, **kw)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu()


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
def test_gather_bit_exact(M, dims):
    inp = _inp(dims, [1, 31, 32, 33, 64, 65, 200], 21, poison=True)
    d = to_dev(inp)
    say("gather", dims["d_c"])
    got = M.gather_pages(d["kv_pages"], d["page_table"], d["seq_lens"], dims["d_c"])
    torch.cuda.synchronize()
    S_max = inp["max_pages"] * inp["page_size"]
    ref = oracle.gather_pages(W.u16(inp["kv_pages"]), inp["page_table"].numpy(),
                              inp["seq_lens"].numpy(), S_max, dims["d_c"])
    assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), ref)


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
def test_permutation_bit_identical(M, dims):
    a = _inp(dims, [70, 300, 129], 22, layout="contiguous")
    b = _inp(dims, [70, 300, 129], 22, layout="shuffled")
    assert not torch.equal(a["page_table"], b["page_table"])
    say("permutation", dims["d_c"])
    oa = gpu_decode(M, to_dev(a))
    ob = gpu_decode(M, to_dev(b))
    torch.cuda.synchronize()
    assert torch.equal(_bits(oa), _bits(ob))


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
def test_poisoned_unused_slots_do_not_leak(M, dims):
    inp = _inp(dims, [1, 33, 100, 190], 23, poison=True)
    clean = dict(inp)
    clean["kv_pages"] = torch.nan_to_num(inp["kv_pages"].float(), nan=0.0).to(torch.bfloat16)
    # page-table entries past each sequence point at arbitrary (even invalid) ids
    far = dict(clean)
    far["page_table"] = inp["page_table"].clone()
    for b in range(inp["B"]):
        n = -(-int(inp["seq_lens"][b]) // 64)
        far["page_table"][b, n:] = -7 if b % 2 else 1 << 30
    say("poison", dims["d_c"])
    op = gpu_decode(M, to_dev(inp))
    oc = gpu_decode(M, to_dev(clean))
    of = gpu_decode(M, to_dev(far))
    torch.cuda.synchronize()
    assert torch.isfinite(op.float()).all()
    assert torch.equal(_bits(op), _bits(oc))
    assert torch.equal(_bits(of), _bits(oc))


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
def test_softmax_rows_sum_to_one(M, dims):
    # value channel 0 of every token = 1 and W_UV[h][:, 0] = e_0: out[b,h,0] = sum_t p_t.
    # The same constant adds q_abs[0] to every logit of a head, which softmax ignores.
    inp = _inp(dims, [1, 45, 64, 500, 1030], 24)
    inp["kv_pages"][:, :, 0] = 1.0
    inp["W_UV"][:, :, 0] = 0.0
    inp["W_UV"][:, 0, 0] = 1.0
    say("rows sum to one", dims["d_c"])
    out = gpu_decode(M, to_dev(inp))
    torch.cuda.synchronize()
    col = out[:, :, 0].float().cpu()
    assert torch.all((col - 1.0).abs() <= 2.0 ** -7), col


def test_deterministic_and_split_invariant(M):
    inp = _inp(DS, [3000, 17, 1500, 64], 25)
    d = to_dev(inp)
    say("determinism / split plans")
    base = gpu_decode(M, d)
    again = gpu_decode(M, d)
    torch.cuda.synchronize()
    assert torch.equal(_bits(base), _bits(again))
    ref, _ = oracle.decode(*W.oracle_args(inp))
    for units in (1, 2, 7, 33, 128, 1000):
        o = gpu_decode(M, d, num_units=units).float().cpu().numpy()
        rel, _ = errors(o, ref)
        assert rel <= REL_L2, (units, rel)
        rel_b, _ = errors(o, base.float().cpu().numpy())
        assert rel_b <= REL_L2, (units, rel_b)


def test_sequence_longer_than_table_is_clamped(M):
    inp = _inp(DS, [128, 64], 26)
    d = to_dev(inp)
    over = dict(d)
    over["seq_lens"] = d["seq_lens"].clone()
    over["seq_lens"][0] = 10 ** 6  # clamped to what page_table row 0 addresses (128 tokens)
    say("length clamp")
    a = gpu_decode(M, d)
    b = gpu_decode(M, over)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("dims", [DS, M2], ids=["deepseek", "mha2mla"])
def test_timed_entry_point(M, dims):
    # mla_decode_timed gives the same bits as mla_decode, and its six events bracket the three
    # kernels in stream order: every kernel takes time, none starts before the previous ends
    inp = _inp(dims, [300, 1000, 64], 24)
    d = to_dev(inp)
    say("timed entry point", dims["d_c"])
    ref = gpu_decode(M, d)
    hip = HipEvents()
    ev = [hip.create() for _ in range(6)]
    out = gpu_decode(M, d, kernel_events=ev)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref))
    for k in range(3):
        assert hip.ms(ev[2 * k], ev[2 * k + 1]) > 0
    assert hip.ms(ev[1], ev[2]) >= 0 and hip.ms(ev[3], ev[4]) >= 0
    # events may be left out (NULL): only the attention kernel timed
    out2 = gpu_decode(M, d, kernel_events=[None, None, ev[2], ev[3], None, None])
    torch.cuda.synchronize()
    assert torch.equal(_bits(out2), _bits(ref))
    assert hip.ms(ev[2], ev[3]) > 0
    for e in ev:
        hip.destroy(e)


def test_log_mode_prints_the_plan(M):
    # MLA_LOG=1: the plan the absorb kernel built, copied back and printed on stderr. Lengths
    # 100, 5 and 300 make 4 + 1 + 10 = 15 tiles of 32 tokens; five units take 3 tiles each,
    # unit g starting at tile 3g, across sequence boundaries
    import os
    import re
    import tempfile
    inp = W.make_inputs(3, 128, 128, 512, 64, 128, [100, 5, 300], 61)
    d = to_dev(inp)
    say("MLA_LOG plan print")
    os.environ["MLA_LOG"] = "1"
    with tempfile.TemporaryFile() as f:
        saved = os.dup(2)
        os.dup2(f.fileno(), 2)
        try:
            M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                     d["page_table"], d["seq_lens"], num_units=5)
            torch.cuda.synchronize()
        finally:
            os.dup2(saved, 2)
            os.close(saved)
            del os.environ["MLA_LOG"]
        f.seek(0)
        text = f.read().decode()
    head = re.search(r"mla_decode plan: (\d+) sequences x (\d+) query tokens, (\d+) tiles of "
                     r"(\d+) tokens, (\d+) units of up to (\d+) tiles, bf16 cache", text)
    assert head, text[:500]
    assert [int(x) for x in head.groups()] == [3, 1, 15, 32, 5, 3]
    rows = [tuple(map(int, m)) for m in re.findall(r"row (\d+): tiles (-?\d+)\.\.(-?\d+)", text)]
    assert rows == [(0, 0, 3), (1, 4, 4), (2, 5, 14)]
    units = [tuple(map(int, m)) for m in re.findall(
        r"unit (\d+): row (\d+) tile (\d+) of (\d+) \(length (\d+), page (-?\d+)\), (\d+) tiles",
        text)]
    assert len(units) == 5
    first = {r: a for r, a, _ in rows}
    for g, row, j, nj, S, page, n in units:
        assert first[row] + j == 3 * g and n == 3, units
        assert S == [100, 5, 300][row] and nj == -(-S // 32)
        assert page == int(inp["page_table"][row, j * 32 // 64])
