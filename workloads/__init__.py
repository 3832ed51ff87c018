"""Seeded synthetic inputs for MLA decode (shared by the tests, the benchmark and the smoke check).

This module draws random numbers and lays them out; it holds none of the method's arithmetic.
Both the GPU path and the CPU oracle consume the exact bytes it produces.

Draw order for one seed (torch CPU generator, fp32 normal draws rounded to bf16 by RNE):
  q_nope [B,H,d_n], q_rope [B,H,d_R]            ~ N(0, 1)
  W_UK [H,d_n,d_c], W_UV [H,d_c,d_v]            ~ N(0, w_std^2), w_std = 1/sqrt(d_c) by default
  seq_lens [B] (only for ragged batches)         uniform integers in [lo, hi]
  per sequence b: c_KV [S_b, d_c] then k_R [S_b, d_R]   ~ N(0, 1)
  physical page permutation (shuffled layout)    torch.randperm(pool_pages)

Cache layout: pool [pool_pages, page_size, d_c + d_R] bf16, a token is [c_KV | k_R]; logical
page j of sequence b is pool page perm[off_b + j] with off_b = sum of earlier sequences' page
counts. page_table [B, max_pages] int32; its entries past ceil(S_b / page_size) point at a valid
page that is not part of the sequence. With poison=True the slots past S_b in a last page and
all extra pool pages hold NaN, so any read of them that reaches the output shows up.

The workloads stand in for the pages' shapes: DeepSeek-V2/V3 decode dimensions with 64-token
pages (bhfrc.com/news/60867 S1, S3) and the MHA2MLA Llama-2-7B attention config
(lpnh.cn/news/2494972 S3.2).
"""
import math

import numpy as np
import torch

PAGE = 64
BF16_NAN = 0x7FC0

# The five workloads (name -> shape recipe). seq = ("fixed", S) or ("uniform", lo, hi).
CONFIGS = {
    1: dict(name="deepseek_b1_s512_contiguous", B=1, H=128, d_n=128, d_c=512, d_R=64, d_v=128,
            seq=("fixed", 512), layout="contiguous", seed=0),
    2: dict(name="deepseek_b16_s4096", B=16, H=128, d_n=128, d_c=512, d_R=64, d_v=128,
            seq=("fixed", 4096), layout="shuffled", seed=1),
    3: dict(name="deepseek_b64_ragged_1k_8k", B=64, H=128, d_n=128, d_c=512, d_R=64, d_v=128,
            seq=("uniform", 1024, 8192), layout="shuffled", seed=2),
    4: dict(name="deepseek_b16_s65536", B=16, H=128, d_n=128, d_c=512, d_R=64, d_v=128,
            seq=("fixed", 65536), layout="shuffled", seed=3),
    5: dict(name="mha2mla_llama2_7b_b32_s32768", B=32, H=32, d_n=120, d_c=64, d_R=8, d_v=128,
            seq=("fixed", 32768), layout="shuffled", seed=4),
}


def _bf16(x):
    return x.to(torch.bfloat16)


def make_inputs(B, H, d_n, d_c, d_R, d_v, seq, seed, layout="shuffled", w_std=None,
                poison=False, extra_pages=None, max_pages=None, page_size=PAGE):
    """Draw one input set. ``seq`` is a list of lengths, ("fixed", S) or ("uniform", lo, hi).

    Returns a dict of CPU tensors (bf16 / int32) plus layout metadata.
    """
    g = torch.Generator().manual_seed(int(seed))
    if w_std is None:
        w_std = 1.0 / math.sqrt(d_c)
    q_nope = _bf16(torch.randn(B, H, d_n, generator=g))
    q_rope = _bf16(torch.randn(B, H, d_R, generator=g))
    W_UK = _bf16(torch.randn(H, d_n, d_c, generator=g) * w_std)
    W_UV = _bf16(torch.randn(H, d_c, d_v, generator=g) * w_std)
    if isinstance(seq, tuple) and seq[0] == "fixed":
        lens = [int(seq[1])] * B
    elif isinstance(seq, tuple) and seq[0] == "uniform":
        lens = torch.randint(int(seq[1]), int(seq[2]) + 1, (B,), generator=g).tolist()
    else:
        lens = [int(s) for s in seq]
        if len(lens) != B:
            raise ValueError("need one length per sequence")
    npg = [max(1, -(-s // page_size)) for s in lens]  # pages per sequence (>= 1)
    used = sum(npg)
    if extra_pages is None:
        extra_pages = -(-used // 20) if poison else 0  # pool + 5 % in poison mode
    pool_pages = used + int(extra_pages)
    if max_pages is None:
        max_pages = max(npg)
    if max_pages < max(npg):
        raise ValueError("max_pages too small")
    w = d_c + d_R
    fill = float("nan") if poison else 0.0
    pool = torch.full((pool_pages, page_size, w), fill, dtype=torch.bfloat16)
    # draw the logical cache sequence by sequence, then place it
    logical = []
    for b in range(B):
        S = lens[b]
        c = torch.randn(S, d_c, generator=g)
        r = torch.randn(S, d_R, generator=g)
        buf = torch.full((npg[b] * page_size, w), fill, dtype=torch.bfloat16)
        buf[:S, :d_c] = _bf16(c)
        buf[:S, d_c:] = _bf16(r)
        logical.append(buf.view(npg[b], page_size, w))
    if layout == "shuffled":
        perm = torch.randperm(pool_pages, generator=g)
    elif layout == "contiguous":
        perm = torch.arange(pool_pages)
    else:
        raise ValueError(layout)
    spare = int(perm[used]) if extra_pages > 0 else 0
    page_table = torch.full((B, max_pages), spare, dtype=torch.int32)
    off = 0
    for b in range(B):
        ids = perm[off:off + npg[b]]
        pool[ids] = logical[b]
        page_table[b, :npg[b]] = ids.to(torch.int32)
        off += npg[b]
    return dict(q_nope=q_nope, q_rope=q_rope, W_UK=W_UK, W_UV=W_UV, kv_pages=pool,
                page_table=page_table, seq_lens=torch.tensor(lens, dtype=torch.int32),
                B=B, H=H, d_n=d_n, d_c=d_c, d_R=d_R, d_v=d_v, page_size=page_size,
                max_pages=max_pages, pool_pages=pool_pages, used_pages=used,
                scale=1.0 / math.sqrt(d_n + d_R))


def config_inputs(i, seed=None, poison=False):
    """Inputs of workload ``i`` (1..5) with its own seed unless one is given."""
    c = CONFIGS[i]
    return make_inputs(c["B"], c["H"], c["d_n"], c["d_c"], c["d_R"], c["d_v"], c["seq"],
                       c["seed"] if seed is None else seed, layout=c["layout"], poison=poison)


def u16(t):
    """uint16 bit-pattern view (numpy) of a bf16 CPU tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_args(inp):
    """The eight inputs as the numpy arrays the oracle takes."""
    return (u16(inp["q_nope"]), u16(inp["q_rope"]), u16(inp["W_UK"]), u16(inp["W_UV"]),
            u16(inp["kv_pages"]), inp["page_table"].numpy(), inp["seq_lens"].numpy())


FP8_NAN = 0x7F  # an e4m3 NaN byte


def _used_slots(inp, P, ps):
    used = torch.zeros(P, ps, dtype=torch.bool)
    for b in range(inp["B"]):
        S = int(inp["seq_lens"][b])
        for t in range(S):
            used[int(inp["page_table"][b, t // ps]), t % ps] = True
    return used


def mxfp4_cache(inp, seed=0, scale_codes=(124, 126), poison=False):
    """A synthetic MXFP4 cache with the page geometry and k_R of ``inp``: every c_KV element a
    uniformly drawn 4-bit E2M1 code, every block of 32 elements a scale byte (E8M0, 2^(code-127))
    drawn uniformly from [scale_codes[0], scale_codes[1]] (seeded). The default scales, 2^-3 to
    2^-1, give c_KV elements of rms about 0.97 (at most 3), the size of the bf16 inputs' N(0, 1)
    latent. Returns (kv4 uint8
    [P, 64, d_c/2 + 2*d_R] with rows [c_KV codes, two per byte, element 2k in the low nibble |
    k_R bf16 bytes], scales uint8 [P, 64, d_c/32]). With poison=True every slot that is not
    part of a sequence holds 0xFF bytes and NaN scales (255)."""
    kv = inp["kv_pages"]
    P, ps, w = kv.shape
    d_c = inp["d_c"]
    g = torch.Generator().manual_seed(int(seed))
    nib = torch.randint(0, 16, (P, ps, d_c), generator=g, dtype=torch.int32)
    packed = (nib[:, :, 0::2] | (nib[:, :, 1::2] << 4)).to(torch.uint8)
    scales = torch.randint(int(scale_codes[0]), int(scale_codes[1]) + 1, (P, ps, d_c // 32),
                           generator=g, dtype=torch.int32).to(torch.uint8)
    kr = kv[:, :, d_c:].contiguous().view(torch.uint8).reshape(P, ps, 2 * (w - d_c))
    kv4 = torch.cat([packed, kr], dim=2).contiguous()
    if poison:
        used = _used_slots(inp, P, ps)
        kv4[~used] = 0xFF
        scales[~used] = 255
    return kv4, scales


def fp8_cache(inp, seed=0, exps=(-6, -2), poison=False):
    """An FP8 copy of the cache of ``inp``: each token's c_KV is divided by a power of two
    2^k, k drawn uniformly from [exps[0], exps[1]] per token slot (seeded), and cast to FP8
    e4m3 by torch (RNE); k_R stays bf16. Returns (kv8 uint8 [P, 64, d_c + 2*d_R] with rows
    [c_KV bytes | k_R bf16 bytes], scales fp32 [P, 64] = 2^k). With poison=True every slot that
    is not part of a sequence holds NaN bytes and a NaN scale."""
    kv = inp["kv_pages"]
    P, ps, w = kv.shape
    d_c = inp["d_c"]
    g = torch.Generator().manual_seed(int(seed))
    k = torch.randint(int(exps[0]), int(exps[1]) + 1, (P, ps), generator=g)
    scales = torch.pow(2.0, k.to(torch.float64)).to(torch.float32)
    c = kv[:, :, :d_c].float() / scales[:, :, None]
    codes = c.to(torch.float8_e4m3fn).view(torch.uint8)
    kr = kv[:, :, d_c:].contiguous().view(torch.uint8).reshape(P, ps, 2 * (w - d_c))
    kv8 = torch.cat([codes, kr], dim=2).contiguous()
    if bool((((codes & 0x7F) == 0x7F) & ~torch.isnan(c)).any()):  # NaN past 464
        raise ValueError("c_KV out of the FP8 range for these scales")
    if poison:
        used = _used_slots(inp, P, ps)
        kv8[~used] = FP8_NAN
        scales[~used] = float("nan")
    return kv8, scales
