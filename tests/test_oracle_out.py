"""Pin of the oracle's merged output projection (oracle.decode_out): with W_UVO formed from
W_UV and an output matrix W_O in fp64, the merged form equals projecting the decode's output
with W_O afterwards (lpnh.cn/news/2494972 S2.2: merging W_uv and W_o changes nothing but the
number of products), for one and for two query tokens."""
import numpy as np
import torch

import oracle
import workloads as W
from tests.pins import _tiny, _rel, _f64


def _merged(inp, W_O):
    H, d_c, d_v = inp["H"], inp["d_c"], inp["d_v"]
    Wv = _f64(W.u16(inp["W_UV"]))                                     # [H, d_c, d_v]
    Wo = W_O.reshape(H, d_v, -1)                                      # [H, d_v, N]
    return np.einsum("hce,hen->nhc", Wv, Wo).reshape(W_O.shape[1], H * d_c)


def test_merged_projection_equals_projecting_the_output():
    rng = np.random.default_rng(7)
    for seed, (seq, kw) in enumerate([([5, 64, 77], {}), ([33, 2, 100], dict(H=3, d_c=16))]):
        inp = _tiny(seq, 1300 + seed, **kw)
        N = 24
        W_O = rng.standard_normal((inp["H"] * inp["d_v"], N))
        args = list(W.oracle_args(inp))
        out, lse = oracle.decode_out(args[0], args[1], args[2], _merged(inp, W_O), *args[4:])
        o3, l3 = oracle.decode(*args)                                 # [B, H, d_v]
        ref = o3.reshape(inp["B"], -1) @ W_O
        assert _rel(out, ref) <= 1e-12 and np.array_equal(lse, l3)
        # two query tokens per sequence
        g = torch.Generator().manual_seed(1400 + seed)
        qn = torch.randn(inp["B"], 2, inp["H"], inp["d_n"], generator=g).to(torch.bfloat16)
        qr = torch.randn(inp["B"], 2, inp["H"], inp["d_R"], generator=g).to(torch.bfloat16)
        out2, _ = oracle.decode_out(W.u16(qn), W.u16(qr), args[2], _merged(inp, W_O), *args[4:])
        o4, _ = oracle.decode_tokens(W.u16(qn), W.u16(qr), *args[2:])  # [B, 2, H, d_v]
        assert _rel(out2, o4.reshape(inp["B"], 2, -1) @ W_O) <= 1e-12
