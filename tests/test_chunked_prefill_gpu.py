"""Chunked prefill through the HIP path: a prompt appended to the paged cache and attended to in
chunks, each chunk's new tokens written by the cache append (lpnh.cn/news/2494972 S2.1,
c_kv = x W_dkv with the decoupled RoPE key) and then decoded as `q_len` query tokens, causal
among themselves over everything cached before them (bhfrc.com/news/60867 S1 and S6: the
prefill side of the split at the 256-row threshold, S3 `kPrefillThresh`).

A chunk at or above the threshold runs the decompressed branch, a shorter one the absorbed
branch; a prompt of 600 tokens in chunks of 256 takes both (256, 256, then 88). Every chunk's
outputs and log-sum-exps are held to the oracle's causal multi-token decode over the oracle's
own cache, which it builds with its fp64 append rounded to bf16 (the two caches may differ in
the last bit of a few values; nothing of the HIP path feeds the oracle)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import LSE_ABS, MAX_ABS, REL_L2, errors, need_gpu, say, to_bf16_bits

pytestmark = pytest.mark.gpu

DS = dict(H=128, d_n=128, d_c=512, d_R=64, d_v=128)
HIDDEN = 1024


@pytest.fixture(scope="module")
def M():
    return need_gpu()


@pytest.mark.parametrize("chunk", [256, 512])
def test_chunked_prefill_matches_oracle(M, chunk):
    prior, prompt = [37, 300], 600
    B = len(prior)
    d = DS
    # pages for the final lengths; the cache rows past the prior context are overwritten by
    # the appends (their initial contents never reach an output)
    inp = W.make_inputs(B, d["H"], d["d_n"], d["d_c"], d["d_R"], d["d_v"],
                        [p + prompt for p in prior], 90 + chunk)
    g = torch.Generator().manual_seed(91 + chunk)
    Wd = (torch.randn(d["d_c"], HIDDEN, generator=g) / HIDDEN ** 0.5).to(torch.bfloat16)
    Wr = (torch.randn(d["d_R"], HIDDEN, generator=g) / HIDDEN ** 0.5).to(torch.bfloat16)
    pt = inp["page_table"]
    dev = torch.device("cuda")
    kv_gpu = inp["kv_pages"].to(dev)
    kv_ref = W.u16(inp["kv_pages"]).copy()
    wuk, wuv = W.u16(inp["W_UK"]), W.u16(inp["W_UV"])
    W_UK, W_UV, pt_d = inp["W_UK"].to(dev), inp["W_UV"].to(dev), pt.to(dev)
    Wd_d, Wr_d = Wd.to(dev), Wr.to(dev)
    lens = np.array(prior, dtype=np.int32)
    pos = 0
    while pos < prompt:
        C = min(chunk, prompt - pos)
        branch = "decompressed" if C >= 256 else "absorbed"
        say("chunked prefill: chunk %d..%d (T=%d, %s branch)" % (pos, pos + C, C, branch))
        x = torch.randn(B, C, HIDDEN, generator=g).to(torch.bfloat16)
        qn = torch.randn(B, C, d["H"], d["d_n"], generator=g).to(torch.bfloat16)
        qr = torch.randn(B, C, d["H"], d["d_R"], generator=g).to(torch.bfloat16)
        # the HIP path: append the chunk at the current lengths, then decode its C tokens
        before = torch.from_numpy(lens.copy())
        M.cache_append(x.to(dev), Wd_d, Wr_d, kv_gpu, pt_d, before.to(dev))
        after = torch.from_numpy(lens + C)
        out, lse = M.decode(qn.to(dev), qr.to(dev), W_UK, W_UV, kv_gpu, pt_d, after.to(dev),
                            return_lse=True)
        torch.cuda.synchronize()
        out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
        # the oracle: its own append into its own cache, then the causal multi-token decode
        rows, where = oracle.cache_append(W.u16(x), W.u16(Wd), W.u16(Wr), pt.numpy(), lens)
        bits = to_bf16_bits(rows)
        for b in range(B):
            for i in range(C):
                page, slot = where[b, i]
                kv_ref[page, slot] = bits[b, i]
        lens = lens + C
        ref, ref_lse = oracle.decode_tokens(W.u16(qn), W.u16(qr), wuk, wuv, kv_ref, pt.numpy(),
                                            lens)
        rel, mx = errors(out, ref)
        lerr = float(np.max(np.abs(lse - ref_lse)))
        say("  rel_l2=%.3e max_abs=%.3e lse_err=%.3e" % (rel, mx, lerr))
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
        assert rel <= REL_L2 and mx <= MAX_ABS and lerr <= LSE_ABS, (pos, C, rel, mx, lerr)
        pos += C
    assert list(lens) == [p + prompt for p in prior]
