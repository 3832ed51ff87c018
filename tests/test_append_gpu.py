"""GPU cache append (mla_cache_append) against the fp64 oracle: the written [c_KV | k_R] rows
within half a bf16 ulp (plus fp32 summation noise) of the exact values, every other cache byte
unchanged, tokens past the page-table row not written, and the decode reading what was
appended."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import (LSE_ABS, MAX_ABS, REL_L2, errors, need_gpu, say, to_dev,
                               to_bf16_bits)

pytestmark = pytest.mark.gpu

SHAPES = {"deepseek": dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128, hidden=7168),
          "mha2mla": dict(H=32, d_n=120, d_c=64, d_R=8, d_v=128, hidden=4096),
          # the widest row the append takes (d_latent 1024, d_rope 512): two threads per
          # column quad in the finishing kernel, so its slice count is capped at 16
          "wide": dict(H=16, d_n=64, d_c=1024, d_R=512, d_v=64, hidden=5120)}


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
                                          ("mha2mla", [1, 63, 64, 1000], 3),
                                          ("wide", [5, 70, 130], 2),
                                          # 160 and 100 token rows: partial work groups
                                          # of 64 and 32 rows, each with a ragged last block
                                          ("deepseek", [1 + 37 * i for i in range(10)], 16),
                                          ("deepseek", [3 + 41 * i for i in range(50)], 2)])
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


def _decode_vs_oracle(M, inp, kv_gpu, seq_lens, kv_ref, label, kv_scales=None):
    """GPU decode over the cache the GPU append wrote, against the oracle's decode over its own
    cache (the same initial pool with the oracle's append written in)."""
    d = to_dev(inp)
    out, lse = M.decode(d["q_nope"], d["q_rope"], d["W_UK"], d["W_UV"], kv_gpu,
                        d["page_table"], seq_lens.cuda(), return_lse=True, kv_scales=kv_scales)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    args = list(W.oracle_args(inp))
    args[4], args[6] = kv_ref, seq_lens.numpy()
    ref, ref_lse = oracle.decode(*args)
    rel, mx = errors(out, ref)
    lerr = float(np.max(np.abs(lse - ref_lse)))
    say(label, "rel_l2=%.3e max_abs=%.3e lse_err=%.3e" % (rel, mx, lerr))
    assert np.all(np.isfinite(out))
    assert rel <= REL_L2 and mx <= MAX_ABS and lerr <= LSE_ABS, (label, rel, mx, lerr)


def test_decode_reads_appended_tokens(M):
    # append one token to each of 3 sequences on the GPU, then decode over the longer
    # sequences; the oracle decodes its own cache: the initial pool with its fp64 append
    # rounded to bf16 at the new slots (the two caches may differ in a last bit)
    inp, x, Wd, Wr, before = _case("deepseek", [100, 64, 300], 1, 44)
    kv_ref = W.u16(inp["kv_pages"]).copy()
    kv = inp["kv_pages"].cuda()
    say("decode after append")
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, inp["page_table"].cuda(), before.cuda())
    rows, where = oracle.cache_append(W.u16(x), W.u16(Wd), W.u16(Wr), inp["page_table"].numpy(),
                                      before.numpy())
    bits = to_bf16_bits(rows)
    for b in range(rows.shape[0]):
        page, slot = where[b, 0]
        kv_ref[page, slot] = bits[b, 0]
    _decode_vs_oracle(M, inp, kv, before + 1, kv_ref, "decode after append")


def test_unallocated_page_entry_is_not_written(M):
    # a new token whose page-table entry names no pool page (-1: not allocated yet, or past
    # the pool) is skipped: every other slot of the pool stays bit for bit as it was, and the
    # tokens with valid entries are written as usual
    inp, x, Wd, Wr, before = _case("mha2mla", [62, 130, 5], 3, 45)
    pt = inp["page_table"].clone()
    pt[0, 1] = -1                         # page of position 64 (sequence 0's third new token)
    pt[1, 2] = inp["kv_pages"].shape[0]   # past the pool: positions 128.. of sequence 1
    say("append with unallocated page entries")
    kv0 = inp["kv_pages"].clone()
    kv = inp["kv_pages"].cuda()
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, pt.cuda(), before.cuda())
    torch.cuda.synchronize()
    got = kv.cpu()
    rows, where = oracle.cache_append(W.u16(x), W.u16(Wd), W.u16(Wr), pt.numpy(),
                                      before.numpy())
    written = np.zeros(got.shape[:2], dtype=bool)
    skipped = 0
    for b in range(3):
        for i in range(3):
            page, slot = where[b, i]
            if page < 0 or page >= got.shape[0]:
                skipped += 1
                continue
            ref = rows[b, i]
            err = np.abs(got[page, slot].double().numpy() - ref)
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), (b, i, float(err.max()))
            written[page, slot] = True
    assert skipped == 4  # sequence 0: position 64; sequence 1: positions 130, 131, 132
    same = got.view(torch.int16).numpy()[~written] == kv0.view(torch.int16).numpy()[~written]
    assert np.all(same), "a slot outside the valid new tokens changed"


def test_check_mode_refuses_unallocated_page_entry(M):
    import os
    inp, x, Wd, Wr, before = _case("mha2mla", [62, 10], 3, 46)
    pt = inp["page_table"].clone()
    pt[0, 1] = -1
    kv0 = inp["kv_pages"].clone()
    kv = inp["kv_pages"].cuda()
    old = os.environ.get("MLA_CHECK")
    os.environ["MLA_CHECK"] = "1"
    try:
        say("append check mode: -1 entry")
        with pytest.raises(M.MlaError) as e:
            M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, pt.cuda(), before.cuda())
        assert e.value.code == 7  # MLA_ERR_DEVICE_CHECK
        torch.cuda.synchronize()
        assert torch.equal(kv.cpu().view(torch.int16), kv0.view(torch.int16))  # nothing written
        # valid entries pass the check and are appended
        M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv, inp["page_table"].cuda(),
                       before.cuda())
        torch.cuda.synchronize()
        assert not torch.equal(kv.cpu().view(torch.int16), kv0.view(torch.int16))
    finally:
        if old is None:
            del os.environ["MLA_CHECK"]
        else:
            os.environ["MLA_CHECK"] = old


# ---- appending into an FP8 cache (mla_cache_append_fp8)

def _fp8_pool(inp, seed):
    kv8, sc = W.fp8_cache(inp, seed=seed)
    return kv8, sc


@pytest.mark.parametrize("shape,lens,T", [("deepseek", [62, 64, 500], 2),
                                          ("deepseek", [1 + 37 * i for i in range(16)], 1),
                                          ("mha2mla", [1, 63, 64, 1000], 3),
                                          ("wide", [5, 70, 130], 2)])
def test_fp8_append_matches_oracle(M, shape, lens, T):
    # Each new token's scale is the smallest power of two 2^e with max |c_KV| <= 448 * 2^e and
    # its bytes are c_KV / 2^e rounded to the nearest even E4M3 value. The kernel decides
    # from fp32 sums and the oracle from fp64 ones, so a code may differ by one step where the
    # exact value sits within summation noise of a rounding midpoint, and a scale where max
    # |c_KV| sits at a power-of-two edge; everything else must agree exactly, and every other
    # byte of the pool and its scales stays as it was.
    inp, x, Wd, Wr, before = _case(shape, lens, T, 44)
    c = SHAPES[shape]
    d_c, d_R = c["d_c"], c["d_R"]
    kv8_0, sc0 = _fp8_pool(inp, 3)
    kv8, sc = kv8_0.clone().cuda(), sc0.clone().cuda()
    say("fp8 append", shape, "B=%d T=%d" % (len(lens), T))
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv8, inp["page_table"].cuda(), before.cuda(),
                   kv_scales=sc)
    torch.cuda.synchronize()
    got8, gotsc = kv8.cpu().numpy(), sc.cpu().numpy()
    codes, scales, kr, where = oracle.cache_append_fp8(
        W.u16(x), W.u16(Wd), W.u16(Wr), inp["page_table"].numpy(), before.numpy())
    rows, _ = oracle.cache_append(W.u16(x), W.u16(Wd), W.u16(Wr), inp["page_table"].numpy(),
                                  before.numpy())
    written = np.zeros(got8.shape[:2], dtype=bool)
    n_codes = n_diff = 0
    for b in range(len(lens)):
        for i in range(T):
            page, slot = where[b, i]
            written[page, slot] = True
            s_gpu = float(gotsc[page, slot])
            if s_gpu != scales[b, i]:  # only at an edge of the scale rule
                amax = np.max(np.abs(rows[b, i, :d_c]))
                ratio = amax / (448 * min(s_gpu, scales[b, i]))
                assert abs(ratio - 1) < 1e-5, (b, i, s_gpu, scales[b, i])
                continue
            g = got8[page, slot, :d_c].astype(np.int64)
            r = codes[b, i].astype(np.int64)
            diff = g != r
            n_codes += g.size
            n_diff += int(diff.sum())
            # a differing code is the other neighbour of a value at a rounding midpoint
            vg = oracle.fp8_e4m3_value(g[diff]) * s_gpu
            vr = oracle.fp8_e4m3_value(r[diff]) * s_gpu
            exact = rows[b, i, :d_c][diff]
            assert np.all(np.abs(np.abs(vg - exact) - np.abs(vr - exact)) <= 1e-5 * s_gpu + 1e-6 * np.abs(exact)), (b, i)
            # k_R: bf16 within half an ulp of the fp64 rotation
            krg = got8[page, slot, d_c:].view(np.uint16).astype(np.uint32) << 16
            krg = krg.view(np.float32).astype(np.float64)
            assert np.all(np.abs(krg - kr[b, i]) <= 2.0 ** -8 * np.abs(kr[b, i]) + 1e-5), (b, i)
    assert n_diff <= max(2, n_codes // 200), (n_diff, n_codes)
    assert np.array_equal(got8[~written], kv8_0.numpy()[~written])
    assert np.array_equal(gotsc[~written], sc0.numpy()[~written], equal_nan=True)


def test_fp8_append_then_decode(M):
    # tokens appended into an FP8 cache are read back by mla_decode_fp8: the decode agrees with
    # the oracle run on the bf16 cache that the FP8 one stands for (dequant_fp8_cache)
    lens, T = [70, 300, 5], 2
    inp, x, Wd, Wr, before = _case("deepseek", lens, T, 45)
    kv8_0, sc0 = _fp8_pool(inp, 4)
    kv8, sc = kv8_0.clone().cuda(), sc0.clone().cuda()
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv8, inp["page_table"].cuda(), before.cuda(),
                   kv_scales=sc)
    say("fp8 append then decode")
    # the oracle's own FP8 cache: the initial pool with its append (codes, scales, and k_R
    # rounded to bf16) written in, read through the format's dequantisation
    codes, scales, kr, where = oracle.cache_append_fp8(
        W.u16(x), W.u16(Wd), W.u16(Wr), inp["page_table"].numpy(), before.numpy())
    d_c = inp["d_c"]
    kv8_ref, sc_ref = kv8_0.numpy().copy(), sc0.numpy().copy()
    krb = to_bf16_bits(kr)
    for b in range(len(lens)):
        for i in range(T):
            page, slot = where[b, i]
            kv8_ref[page, slot, :d_c] = codes[b, i]
            kv8_ref[page, slot, d_c:] = krb[b, i].view(np.uint8)
            sc_ref[page, slot] = scales[b, i]
    kv_ref = oracle.dequant_fp8_cache(kv8_ref, sc_ref, d_c)
    _decode_vs_oracle(M, inp, kv8, inp["seq_lens"], kv_ref, "fp8 append then decode",
                      kv_scales=sc)


# ---- MXFP4 cache (OCP MX: E2M1 codes, an E8M0 scale per token and block of 32 elements)

@pytest.mark.parametrize("shape,lens,T", [("mha2mla", [1, 63, 64, 1000], 3),
                                          ("deepseek", [62, 64, 500], 2),
                                          ("wide", [5, 70, 130], 2)])
def test_mxfp4_append_matches_oracle(M, shape, lens, T):
    # Per block of 32 latent elements the scale byte is X + 127, X = floor(log2 max|c_KV|) - 2,
    # and each code is c_KV / 2^X rounded to the nearest even E2M1 value (saturating at 6). The
    # kernel decides from fp32 sums and the oracle from fp64 ones, so a scale may differ where a
    # block's maximum sits at a power of two, and a code where a value sits within summation
    # noise of a rounding midpoint; everything else must agree exactly, and every other byte of
    # the pool and its scales stays as it was.
    inp, x, Wd, Wr, before = _case(shape, lens, T, 46)
    c = SHAPES[shape]
    d_c, d_R, nb = c["d_c"], c["d_R"], c["d_c"] // 32
    kv4_0, sc0 = W.mxfp4_cache(inp, seed=7)
    kv4, sc = kv4_0.clone().cuda(), sc0.clone().cuda()
    say("mxfp4 append", shape, "B=%d T=%d" % (len(lens), T))
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv4, inp["page_table"].cuda(), before.cuda(),
                   kv_scales=sc)
    torch.cuda.synchronize()
    got4, gotsc = kv4.cpu().numpy(), sc.cpu().numpy()
    codes, scales, kr, where = oracle.cache_append_mxfp4(
        W.u16(x), W.u16(Wd), W.u16(Wr), inp["page_table"].numpy(), before.numpy())
    rows, _ = oracle.cache_append(W.u16(x), W.u16(Wd), W.u16(Wr), inp["page_table"].numpy(),
                                  before.numpy())
    written = np.zeros(got4.shape[:2], dtype=bool)
    n_codes = n_diff = n_edge = 0
    for b in range(len(lens)):
        for i in range(T):
            page, slot = where[b, i]
            written[page, slot] = True
            g_codes = oracle.unpack_fp4(got4[page, slot, :d_c // 2]).astype(np.int64)
            for k in range(nb):
                blk = rows[b, i, 32 * k:32 * k + 32]
                sg, sr = int(gotsc[page, slot, k]), int(scales[b, i, k])
                if sg != sr:  # only at a power-of-two edge of the block's maximum
                    amax = np.max(np.abs(blk))
                    ratio = amax / 2.0 ** (max(sg, sr) - 127 + 2)
                    assert abs(ratio - 1) < 1e-5, (b, i, k, sg, sr, amax)
                    n_edge += 1
                    continue
                g = g_codes[32 * k:32 * k + 32]
                r = codes[b, i, 32 * k:32 * k + 32].astype(np.int64)
                diff = g != r
                n_codes += g.size
                n_diff += int(diff.sum())
                # a differing code is the other neighbour of a value at a rounding midpoint
                s = 2.0 ** (sg - 127)
                a = np.minimum(np.abs(blk[diff]) / s, 6.0)
                vg = np.abs(oracle.fp4_e2m1_value(g[diff]))
                vr = np.abs(oracle.fp4_e2m1_value(r[diff]))
                assert np.all(np.abs(np.abs(vg - a) - np.abs(vr - a)) <= 1e-5 * (1 + a)), (b, i, k)
            # k_R: bf16 within half an ulp of the fp64 rotation
            krg = got4[page, slot, d_c // 2:].view(np.uint16).astype(np.uint32) << 16
            krg = krg.view(np.float32).astype(np.float64)
            assert np.all(np.abs(krg - kr[b, i]) <= 2.0 ** -8 * np.abs(kr[b, i]) + 1e-5), (b, i)
    say("  codes compared %d, differing %d, scales at an edge %d" % (n_codes, n_diff, n_edge))
    assert n_diff <= max(2, n_codes // 200), (n_diff, n_codes)
    assert np.array_equal(got4[~written], kv4_0.numpy()[~written])
    assert np.array_equal(gotsc[~written], sc0.numpy()[~written])


def test_mxfp4_append_then_decode(M):
    # tokens appended into an MXFP4 cache are read back by mla_decode_mxfp4 (MHA2MLA widths);
    # the oracle decodes its own MXFP4 cache (the initial pool with its append written in)
    lens, T = [70, 300, 5], 2
    inp, x, Wd, Wr, before = _case("mha2mla", lens, T, 47)
    kv4_0, sc0 = W.mxfp4_cache(inp, seed=8)
    kv4, sc = kv4_0.clone().cuda(), sc0.clone().cuda()
    M.cache_append(x.cuda(), Wd.cuda(), Wr.cuda(), kv4, inp["page_table"].cuda(), before.cuda(),
                   kv_scales=sc)
    say("mxfp4 append then decode")
    codes, scales, kr, where = oracle.cache_append_mxfp4(
        W.u16(x), W.u16(Wd), W.u16(Wr), inp["page_table"].numpy(), before.numpy())
    d_c = inp["d_c"]
    kv4_ref, sc_ref = kv4_0.numpy().copy(), sc0.numpy().copy()
    krb = to_bf16_bits(kr)
    for b in range(len(lens)):
        for i in range(T):
            page, slot = where[b, i]
            kv4_ref[page, slot, :d_c // 2] = oracle.pack_fp4(codes[b, i])
            kv4_ref[page, slot, d_c // 2:] = krb[b, i].view(np.uint8)
            sc_ref[page, slot] = scales[b, i]
    kv_ref = oracle.dequant_mxfp4_cache(kv4_ref, sc_ref, d_c)
    _decode_vs_oracle(M, inp, kv4, inp["seq_lens"], kv_ref, "mxfp4 append then decode",
                      kv_scales=sc)
