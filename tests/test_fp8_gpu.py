"""GPU parity of the FP8 latent cache (both widths): the decode over an FP8 e4m3 cache with
per-token power-of-two scales, through mla_decode_fp8, against the fp64 oracle run on the bf16
cache that the FP8 one stands for (oracle.dequant_fp8_cache; with power-of-two scales every
dequantised value is a bf16 value, so both sides see the same numbers and the bf16 bounds
apply unchanged)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import LSE_ABS, MAX_ABS, REL_L2, errors, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

# DeepSeek widths, FP8 against the bf16 path on the same values: the scores differ by the
# block-scaled FP8 MFMA's own accumulation (measured on the device: up to 8.4e-5 of the sum of
# |products| of one 16x16x128 instruction, where fp32 summation would give about 1e-7). On the
# case below that moved the outputs by 7-8e-4 (rel-L2) and the lse by 4.7e-4; the bounds leave
# 2.5x and 4x of that, still below the oracle bounds the two paths each meet
FP8_VS_BF16_REL = 2e-3
FP8_VS_BF16_LSE = 2e-3

M2 = dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128)
DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)


@pytest.fixture(scope="module")
def M():
    return need_gpu()


def _inp(lens, seed, dims=M2, **kw):
    return W.make_inputs(len(lens), dims["H"], dims["d_n"], dims["d_c"], dims["d_R"],
                         dims["d_v"], lens, seed, **kw)


def check_fp8(M, inp, units=0, pairs=None, poison=False, label="", seed=5, exps=(-6, -2)):
    kv8, sc = W.fp8_cache(inp, seed=seed, poison=poison, exps=exps)
    say(label, "fp8 B=%d units=%d T=%d" % (inp["B"], units,
                                            inp["q_nope"].shape[1] if inp["q_nope"].dim() == 4
                                            else 1))
    d = to_dev(inp)
    out, lse = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv8.cuda(),
                        d["page_table"], d["seq_lens"], num_units=units, return_lse=True,
                        kv_scales=sc.cuda())
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    args = list(W.oracle_args(inp))
    args[4] = oracle.dequant_fp8_cache(kv8.numpy(), sc.numpy(), inp["d_c"])
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
def test_fp8_ragged(M, units):
    inp = _inp([1, 63, 64, 65, 1000, 130], 12, poison=True)
    check_fp8(M, inp, units=units, poison=True, label="fp8 ragged")


@pytest.mark.parametrize("units", [1, 2])
def test_fp8_long_sequences_few_units(M, units):
    # a unit walks more than 64 pages of one sequence and crosses into the next
    check_fp8(M, _inp([64 * 150 + 7, 64 * 70], 17), units=units, label="fp8 long")


def test_fp8_many_short_sequences(M):
    lens = [1 + (11 * i) % 200 for i in range(200)]
    check_fp8(M, _inp(lens, 14), label="fp8 200 short")


def test_fp8_wide_scale_range(M):
    # scales from 2^-6 to 2^-2: small |c_KV| lands on FP8 subnormals and zero
    inp = _inp([500, 77, 2048], 21)
    check_fp8(M, inp, label="fp8 scale range")


@pytest.mark.parametrize("T", [2, 4])
def test_fp8_query_tokens(M, T):
    inp = _inp([70, T, 200, 64 * 3 + 1], 31)
    g = torch.Generator().manual_seed(32)
    B = inp["B"]
    inp["q_nope"] = torch.randn(B, T, 32, 120, generator=g).to(torch.bfloat16)
    inp["q_rope"] = torch.randn(B, T, 32, 8, generator=g).to(torch.bfloat16)
    check_fp8(M, inp, label="fp8 %d query tokens" % T)


def test_fp8_equals_bf16_on_the_same_values(M):
    # with the bf16 cache holding exactly the dequantised values, the two paths compute the
    # same numbers from the same bf16 operands: results agree to fp32 summation-order noise
    inp = _inp([300, 64, 1000], 41)
    kv8, sc = W.fp8_cache(inp, seed=2)
    deq = oracle.dequant_fp8_cache(kv8.numpy(), sc.numpy(), inp["d_c"])
    inp["kv_pages"] = torch.from_numpy(deq.view(np.int16)).view(torch.bfloat16)
    d = to_dev(inp)
    a = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv8.cuda(), d["page_table"],
                 d["seq_lens"], kv_scales=sc.cuda())
    b = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                 d["page_table"], d["seq_lens"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_fp8_check_mode_flags_scales_off_contract(M):
    # MLA_CHECK=1 inspects the scale of every slot a sequence uses: a scale that is not a
    # positive normal power of two there is reported (MLA_ERR_DEVICE_CHECK) and nothing is
    # decoded; the same value in a slot past the sequence's end is ignored
    import os
    inp = _inp([300, 64, 129], 51)
    kv8, sc = W.fp8_cache(inp, seed=6)
    d = to_dev(inp)
    pt = inp["page_table"].numpy()
    kv8 = kv8.cuda()

    def run(scales):
        o = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv8, d["page_table"],
                     d["seq_lens"], kv_scales=scales.cuda())
        torch.cuda.synchronize()
        return o

    ref = run(sc)
    os.environ["MLA_CHECK"] = "1"
    try:
        assert torch.equal(run(sc), ref)
        for b, tt, bad in ((0, 17, 0.3), (0, 299, 1.5), (1, 0, 0.0), (2, 128, -0.25)):
            s2 = sc.clone()
            s2[pt[b, tt // 64], tt % 64] = bad
            say("fp8 check: bad scale %r at sequence %d token %d" % (bad, b, tt))
            with pytest.raises(M.MlaError) as e:
                run(s2)
            assert e.value.code == 7  # MLA_ERR_DEVICE_CHECK
        # past the end of sequence 2 (129 tokens): slot 129 of its page table row
        s2 = sc.clone()
        s2[pt[2, 129 // 64], 129 % 64] = 0.3
        assert torch.equal(run(s2), ref)
    finally:
        del os.environ["MLA_CHECK"]


def test_fp8_workload_full_size(M):
    # the MHA2MLA workload (B=32, S=32768) over an FP8 copy of its cache, every (b, h)
    inp = W.config_inputs(5)
    check_fp8(M, inp, label="fp8 workload 5")


# ---- DeepSeek widths (a 640-byte FP8 row plus its scale, against 1152 bytes in bf16)

@pytest.mark.parametrize("units", [0, 1, 3, 7, 40])
def test_fp8_deepseek_ragged(M, units):
    # lengths around the 32-token tile and 64-token page edges, NaN in every unused slot
    inp = _inp([1, 31, 32, 33, 64, 65, 700, 130], 81, DS, poison=True)
    check_fp8(M, inp, units=units, poison=True, label="fp8 deepseek ragged")


@pytest.mark.parametrize("units", [1, 2])
def test_fp8_deepseek_long_sequences_few_units(M, units):
    # a unit walks more than 64 pages (the page window refills) and crosses into the next
    check_fp8(M, _inp([64 * 70 + 7, 64 * 3 + 40], 82, DS), units=units,
              label="fp8 deepseek long")


def test_fp8_deepseek_query_split_scales(M):
    # the absorbed query is split into two FP8 parts with a per-head E8M0 scale chosen from the
    # head's largest element (the split does not depend on the scale elsewhere): an all-zero
    # query (no scale to take), queries scaled by 2^-60 and by 2^-122 (largest |q_abs| below
    # 2^-120, where the hi scale clamps to its smallest code), and one left as drawn
    inp = _inp([300, 200, 129, 64], 87, DS)
    qn = inp["q_nope"].float()
    qn[0] = 0.0
    qn[1] *= 2.0 ** -60
    qn[2] *= 2.0 ** -122
    inp["q_nope"] = qn.to(torch.bfloat16)
    qa = np.einsum("bhd,hdc->bhc", inp["q_nope"].float().numpy(), inp["W_UK"].float().numpy())
    say("fp8 deepseek split scales: largest |q_abs| per sequence %s"
        % ", ".join("%.1e" % float(np.abs(qa[b]).max()) for b in range(4)))
    assert np.abs(qa[2]).max() < 2.0 ** -120  # the clamped case is the one exercised
    check_fp8(M, inp, label="fp8 deepseek split scales")


def test_fp8_deepseek_query_tokens(M):
    inp = _inp([70, 2, 200, 64 * 3 + 1], 83, DS)
    g = torch.Generator().manual_seed(84)
    inp["q_nope"] = torch.randn(4, 2, 128, 128, generator=g).to(torch.bfloat16)
    inp["q_rope"] = torch.randn(4, 2, 128, 64, generator=g).to(torch.bfloat16)
    check_fp8(M, inp, label="fp8 deepseek 2 query tokens")


def test_fp8_deepseek_close_to_bf16_on_the_same_values(M):
    # the scores come from the block-scaled FP8 MFMA (cache bytes as stored, the token's scale as
    # the block scale, the query split exactly into two FP8 parts), the values as in the bf16
    # path: against the bf16 path on the dequantised values only the scores' rounding differs
    inp = _inp([300, 64, 1000, 33], 85, DS)
    kv8, sc = W.fp8_cache(inp, seed=3)
    deq = oracle.dequant_fp8_cache(kv8.numpy(), sc.numpy(), inp["d_c"])
    inp["kv_pages"] = torch.from_numpy(deq.view(np.int16)).view(torch.bfloat16)
    d = to_dev(inp)
    for units in (0, 3):
        a, la = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv8.cuda(),
                         d["page_table"], d["seq_lens"], kv_scales=sc.cuda(), num_units=units,
                         return_lse=True)
        b, lb = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                         d["page_table"], d["seq_lens"], num_units=units, return_lse=True)
        torch.cuda.synchronize()
        rel, mx = errors(a.float().cpu().numpy(), b.float().cpu().numpy())
        lerr = (la - lb).abs().max().item()
        say("fp8 deepseek vs bf16 path, units=%d: rel_l2=%.3e max_abs=%.3e lse=%.3e"
            % (units, rel, mx, lerr))
        assert rel <= FP8_VS_BF16_REL and lerr <= FP8_VS_BF16_LSE, (units, rel, lerr)


def test_fp8_deepseek_empty_sequence_gives_zero_and_neg_inf(M):
    inp = _inp([100, 5, 64], 86, DS)
    kv8, sc = W.fp8_cache(inp, seed=1)
    d = to_dev(inp)
    d["seq_lens"][1] = 0
    out, lse = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv8.cuda(),
                        d["page_table"], d["seq_lens"], return_lse=True, kv_scales=sc.cuda())
    torch.cuda.synchronize()
    assert torch.all(out[1].float() == 0)
    assert torch.all(torch.isneginf(lse[1]))
    assert torch.isfinite(out[0].float()).all() and torch.isfinite(out[2].float()).all()


@pytest.mark.parametrize("cfg", [2, 4])
def test_fp8_deepseek_workload_full_size(M, cfg):
    # B=16 at S=4096 (every (b, h)) and at S=65536 (a seeded sample of (b, h) pairs, every
    # sequence) over an FP8 copy of the workload's cache
    inp = W.config_inputs(cfg)
    pairs = None
    if cfg == 4:
        rng = np.random.default_rng(44)
        pairs = [(b, int(h)) for b in range(inp["B"]) for h in rng.choice(inp["H"], 4, False)]
    check_fp8(M, inp, pairs=pairs, label="fp8 workload %d" % cfg, exps=(-5, -1))


@pytest.mark.parametrize("units", [1, 5, 33])
def test_fp8_query_tokens_split_plans(M, units):
    # three query tokens per sequence over split plans: a unit's tiles cross virtual sequences
    inp = _inp([200, 3, 64 * 5 + 9], 61, poison=True)
    g = torch.Generator().manual_seed(62)
    inp["q_nope"] = torch.randn(3, 3, 32, 120, generator=g).to(torch.bfloat16)
    inp["q_rope"] = torch.randn(3, 3, 32, 8, generator=g).to(torch.bfloat16)
    check_fp8(M, inp, units=units, poison=True, label="fp8 3 tokens, %d units" % units)


def test_fp8_empty_sequence_gives_zero_and_neg_inf(M):
    inp = _inp([100, 5, 64], 63)
    kv8, sc = W.fp8_cache(inp, seed=1)
    d = to_dev(inp)
    d["seq_lens"][1] = 0
    say("fp8 empty sequence")
    out, lse = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv8.cuda(),
                        d["page_table"], d["seq_lens"], return_lse=True, kv_scales=sc.cuda())
    torch.cuda.synchronize()
    assert torch.all(out[1].float() == 0)
    assert torch.all(torch.isneginf(lse[1]))
    assert torch.isfinite(out[0].float()).all() and torch.isfinite(out[2].float()).all()


def test_fp8_check_mode_decodes_as_without(M):
    import os
    inp = _inp([1, 65, 300, 128], 64)
    kv8, sc = W.fp8_cache(inp, seed=2)
    d = to_dev(inp)
    kv8, sc = kv8.cuda(), sc.cuda()

    def run():
        o = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv8, d["page_table"],
                     d["seq_lens"], kv_scales=sc)
        torch.cuda.synchronize()
        return o

    ref = run()
    os.environ["MLA_CHECK"] = "1"
    try:
        got = run()
        good = d["seq_lens"].clone()
        d["seq_lens"][2] = 64 * d["page_table"].shape[1] + 1  # past the page table
        with pytest.raises(M.MlaError) as e:
            run()
        assert e.value.code == 7  # MLA_ERR_DEVICE_CHECK
        d["seq_lens"].copy_(good)
    finally:
        del os.environ["MLA_CHECK"]
    assert torch.equal(got, ref)


def test_fp8_graph_replays_match_eager(M):
    # the FP8 decode captured in a HIP graph: replays with refilled inputs (other values, same
    # shapes), eager decodes in between, each replay bit-identical to the eager call
    lens = [1, 33, 100, 190, 700]
    sets = {}
    for name, seed in (("a", 71), ("b", 72)):
        inp = _inp(lens, seed)
        kv8, sc = W.fp8_cache(inp, seed=seed)
        dd = to_dev(inp)
        dd["kv_pages"], dd["kv_scales"] = kv8.cuda(), sc.cuda()
        sets[name] = dd
    keys = ("q_nope", "q_rope", "W_UK", "W_UV", "kv_pages", "kv_scales", "page_table",
            "seq_lens")

    def call(d, **kw):
        return M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], d["kv_pages"],
                        d["page_table"], d["seq_lens"], kv_scales=d["kv_scales"], **kw)

    def eager(d):
        o, l = call(d, return_lse=True)
        torch.cuda.synchronize()
        return o, l

    ref = {k: eager(v) for k, v in sets.items()}
    assert not torch.equal(ref["a"][0], ref["b"][0])
    st = {k: sets["a"][k].clone() for k in keys}
    B = len(lens)
    out = torch.empty((B, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 32), dtype=torch.float32, device="cuda")
    dm = M.make_dims(st["q_nope"], st["q_rope"], st["W_UK"], st["W_UV"], st["kv_pages"],
                     st["page_table"])
    ws = torch.empty(M.workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(st, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("fp8 graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(st, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for rep, name in enumerate(["a", "b", "b", "a", "b"]):
        for k in keys:
            st[k].copy_(sets[name][k])
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("fp8 graph replay", rep, name)
        assert torch.equal(out.view(torch.int16), ref[name][0].view(torch.int16)), (rep, name)
        assert torch.equal(lse.view(torch.int32), ref[name][1].view(torch.int32)), (rep, name)
        eager(sets["b" if name == "a" else "a"])
