"""Pins of the CPU oracle: checks against what the pages and the mathematics fix.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle disagrees.
``test_oracle_pins.py`` runs them on the real oracle (all must pass);
``test_oracle_mutants.py`` runs them on builds with a planted mistake (one must fail).

Pins, and the passage or fact each one rests on:
  naive_equals_absorbed  the naive (K and V decompressed per head) and absorbed forms give the
                         same attention (bhfrc.com/news/60867 S4 compares exactly these two
                         paths; lpnh.cn/news/2494972 S2.1 derives the absorption).
  sdpa_library           torch's scaled_dot_product_attention in float64, on K = [W_UK c | k_R]
                         and V = W_UV^T c, with its default scale 1/sqrt(d_n + d_R)
                         (bhfrc.com/news/60867 S4 scale; lpnh.cn/news/2494972 S2.1 equations).
  rows_sum_to_one        softmax weights are non-negative and sum to 1.
  single_token           S = 1: the output is the up-projected latent of that token.
  zero_query             zero queries: uniform weights, the output is the up-projected mean.
  identical_tokens       all tokens equal: output = up-projected token, lse = s + ln S.
  dominant_rope          one token's RoPE logit dominates: output = that token's value.
  permutation            the output depends on the logical cache only, not on where its pages
                         sit in the pool (bhfrc.com/news/60867 S3 paged layout).
  split_combine          cutting the tokens into ranges and merging by log-sum-exp gives the
                         single-pass result.
  gather_numpy           the logical copy of the paged cache equals an independent numpy
                         gather (page_table[b, t // page_size], slot t % page_size, zero past
                         S_b) byte for byte, on a shuffled pool with NaN-poisoned unused slots
                         and pages (bhfrc.com/news/60867 S3 paged layout).
  tokens_causal_sdpa     several query tokens per sequence (the sequence's newest tokens):
                         torch's scaled_dot_product_attention in float64 with an explicit
                         causal mask (query token i of T sees tokens 0 .. S - T + i) on the
                         same decompressed K and V; one query token gives exactly the plain
                         decode.
"""
import math

import numpy as np
import torch

import workloads as W

TINY = dict(B=3, H=2, d_n=4, d_c=8, d_R=2, d_v=6)


def _f64(u16):
    """Exact fp64 value of bf16 bit patterns."""
    return (np.asarray(u16, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _tiny(seq, seed, layout="shuffled", page_size=4, **kw):
    d = dict(TINY)
    d.update(kw)
    return W.make_inputs(d["B"], d["H"], d["d_n"], d["d_c"], d["d_R"], d["d_v"], seq, seed,
                         layout=layout, page_size=page_size)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _logical(inp):
    """Logical cache per sequence as fp64 [S_b, d_c + d_R] (plain page-table indexing)."""
    kv = _f64(W.u16(inp["kv_pages"]))
    P = inp["page_size"]
    out = []
    for b in range(inp["B"]):
        S = int(inp["seq_lens"][b])
        t = np.arange(S)
        pages = inp["page_table"][b].numpy()[t // P]
        out.append(kv[pages, t % P])
    return out


def naive_equals_absorbed(O):
    for seed, seq in enumerate([[1, 5, 63], [64, 65, 130], [7, 9, 4]]):
        inp = _tiny(seq, 100 + seed)
        a, la = O.decode(*W.oracle_args(inp))
        n, ln = O.decode_naive(*W.oracle_args(inp))
        assert _rel(a, n) <= 1e-12, ("out", _rel(a, n))
        assert np.max(np.abs(la - ln)) <= 1e-12, "lse"
    # the pages' own check runs at DeepSeek widths (d_n 128, d_c 512, d_R 64, S 2048)
    inp = W.make_inputs(1, 4, 128, 512, 64, 128, [2048], 42)
    a, la = O.decode(*W.oracle_args(inp))
    n, ln = O.decode_naive(*W.oracle_args(inp))
    assert _rel(a, n) <= 1e-12, ("deepseek widths", _rel(a, n))
    assert np.max(np.abs(la - ln)) <= 1e-11


def sdpa_library(O):
    for seed, (seq, kw) in enumerate([([5, 64, 77], {}),
                                      ([33, 1, 100], dict(H=3, d_n=5, d_c=16, d_R=3, d_v=4)),
                                      ([130, 2, 65], dict(d_n=8, d_c=12, d_R=4))]):
        inp = _tiny(seq, 200 + seed, **kw)
        out, lse = O.decode(*W.oracle_args(inp))
        qn = torch.from_numpy(_f64(W.u16(inp["q_nope"])))
        qr = torch.from_numpy(_f64(W.u16(inp["q_rope"])))
        Wk = torch.from_numpy(_f64(W.u16(inp["W_UK"])))  # [H, d_n, d_c]
        Wv = torch.from_numpy(_f64(W.u16(inp["W_UV"])))  # [H, d_c, d_v]
        d_c = inp["d_c"]
        for b, tok in enumerate(_logical(inp)):
            tok = torch.from_numpy(tok)
            c, r = tok[:, :d_c], tok[:, d_c:]
            H = inp["H"]
            K = torch.cat([torch.matmul(Wk, c.T).transpose(1, 2),              # [H, S, d_n]
                           r.unsqueeze(0).expand(H, -1, -1)], dim=2)           # [H, S, d_n+d_R]
            V = torch.matmul(c.unsqueeze(0), Wv)                               # [H, S, d_v]
            Q = torch.cat([qn[b], qr[b]], dim=1).unsqueeze(1)                  # [H, 1, d_n+d_R]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[:, 0]
            assert _rel(out[b], ref.numpy()) <= 1e-12, ("sdpa", b, _rel(out[b], ref.numpy()))
            scale = 1.0 / math.sqrt(K.shape[2])
            ref_lse = torch.logsumexp(scale * torch.matmul(K, Q.transpose(1, 2))[:, :, 0], dim=1)
            assert np.max(np.abs(lse[b] - ref_lse.numpy())) <= 1e-12, "lse"


def rows_sum_to_one(O):
    inp = _tiny([70, 1, 129], 300)
    args = W.oracle_args(inp)
    for b in range(inp["B"]):
        for h in range(inp["H"]):
            p = O.probs(*args, b=b, h=h)
            assert p.shape == (int(inp["seq_lens"][b]),)
            assert np.all(p >= 0.0)
            assert abs(p.sum() - 1.0) <= 1e-12


def _up(inp, h, lat):
    return lat @ _f64(W.u16(inp["W_UV"]))[h]


def single_token(O):
    inp = _tiny([1, 1, 1], 400)
    out, lse = O.decode(*W.oracle_args(inp))
    d_c = inp["d_c"]
    for b, tok in enumerate(_logical(inp)):
        for h in range(inp["H"]):
            assert _rel(out[b, h], _up(inp, h, tok[0, :d_c])) <= 1e-14


def zero_query(O):
    inp = _tiny([9, 64, 3], 500)
    inp["q_nope"].zero_()
    inp["q_rope"].zero_()
    out, lse = O.decode(*W.oracle_args(inp))
    d_c = inp["d_c"]
    for b, tok in enumerate(_logical(inp)):
        S = tok.shape[0]
        for h in range(inp["H"]):
            assert _rel(out[b, h], _up(inp, h, tok[:, :d_c].mean(axis=0))) <= 1e-13
            assert abs(lse[b, h] - math.log(S)) <= 1e-13


def identical_tokens(O):
    inp = _tiny([10, 1, 67], 600)
    kv = inp["kv_pages"]
    kv[:] = kv[inp["page_table"][0, 0], 0].clone()  # every slot holds the same token
    out, lse = O.decode(*W.oracle_args(inp))
    tok = _f64(W.u16(kv[0, 0]))
    d_c = inp["d_c"]
    qn = _f64(W.u16(inp["q_nope"]))
    qr = _f64(W.u16(inp["q_rope"]))
    Wk = _f64(W.u16(inp["W_UK"]))
    scale = 1.0 / math.sqrt(inp["d_n"] + inp["d_R"])
    for b in range(inp["B"]):
        S = int(inp["seq_lens"][b])
        for h in range(inp["H"]):
            assert _rel(out[b, h], _up(inp, h, tok[:d_c])) <= 1e-13
            s = scale * (qn[b, h] @ (Wk[h] @ tok[:d_c]) + qr[b, h] @ tok[d_c:])
            assert abs(lse[b, h] - (s + math.log(S))) <= 1e-12


def dominant_rope(O):
    inp = _tiny([40, 70, 5], 700)
    inp["q_rope"].zero_()
    inp["q_rope"][:, :, 0] = 64.0
    d_c = inp["d_c"]
    P = inp["page_size"]
    for b in range(inp["B"]):
        S = int(inp["seq_lens"][b])
        star = (7 * b + 3) % S
        for t in range(S):
            pg = inp["page_table"][b, t // P]
            inp["kv_pages"][pg, t % P, d_c] = 64.0 if t == star else 0.0
    out, _ = O.decode(*W.oracle_args(inp))
    for b, tok in enumerate(_logical(inp)):
        star = (7 * b + 3) % tok.shape[0]
        for h in range(inp["H"]):
            # the winning logit leads the others by about 4096/sqrt(6) > 1600: e^-1600 is 0
            assert _rel(out[b, h], _up(inp, h, tok[star, :d_c])) <= 1e-12


def permutation(O):
    a = _tiny([37, 64, 100], 800, layout="contiguous")
    b = _tiny([37, 64, 100], 800, layout="shuffled")
    assert not np.array_equal(a["page_table"].numpy(), b["page_table"].numpy())
    oa, la = O.decode(*W.oracle_args(a))
    ob, lb = O.decode(*W.oracle_args(b))
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def split_combine(O):
    inp = _tiny([150, 1, 77], 900)
    o1, l1 = O.decode(*W.oracle_args(inp))
    for ns in (2, 3, 7, 16, 200):
        o, l = O.decode(*W.oracle_args(inp), n_split=ns)
        assert _rel(o, o1) <= 1e-13, ("split", ns)
        assert np.max(np.abs(l - l1)) <= 1e-13


def _queries(B, T, H, d_n, d_R, seed):
    g = torch.Generator().manual_seed(seed)
    qn = torch.randn(B, T, H, d_n, generator=g).to(torch.bfloat16)
    qr = torch.randn(B, T, H, d_R, generator=g).to(torch.bfloat16)
    return qn, qr


def tokens_causal_sdpa(O):
    for seed, (seq, T, kw) in enumerate([([5, 64, 77], 3, {}),
                                         ([33, 4, 100], 4, dict(H=3, d_n=5, d_c=16, d_R=3)),
                                         ([130, 2, 65], 2, dict(d_n=8, d_c=12, d_R=4))]):
        inp = _tiny(seq, 1000 + seed, **kw)
        B, H, d_c = inp["B"], inp["H"], inp["d_c"]
        qn_t, qr_t = _queries(B, T, H, inp["d_n"], inp["d_R"], 1100 + seed)
        args = list(W.oracle_args(inp))
        args[0], args[1] = W.u16(qn_t), W.u16(qr_t)
        out, lse = O.decode_tokens(*args)
        assert out.shape == (B, T, H, inp["d_v"]) and lse.shape == (B, T, H)
        qn, qr = torch.from_numpy(_f64(W.u16(qn_t))), torch.from_numpy(_f64(W.u16(qr_t)))
        Wk = torch.from_numpy(_f64(W.u16(inp["W_UK"])))
        Wv = torch.from_numpy(_f64(W.u16(inp["W_UV"])))
        for b, tok in enumerate(_logical(inp)):
            tok = torch.from_numpy(tok)
            S = tok.shape[0]
            c, r = tok[:, :d_c], tok[:, d_c:]
            K = torch.cat([torch.matmul(Wk, c.T).transpose(1, 2),
                           r.unsqueeze(0).expand(H, -1, -1)], dim=2)           # [H, S, d_n+d_R]
            V = torch.matmul(c.unsqueeze(0), Wv)                               # [H, S, d_v]
            Q = torch.cat([qn[b], qr[b]], dim=2).transpose(0, 1)               # [H, T, d_n+d_R]
            mask = torch.arange(S)[None, :] <= (S - T + torch.arange(T))[:, None]  # [T, S]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
            got = torch.from_numpy(out[b]).transpose(0, 1)                     # [H, T, d_v]
            assert _rel(got.numpy(), ref.numpy()) <= 1e-12, ("tokens", b)
            logits = torch.matmul(Q, K.transpose(1, 2)) / math.sqrt(K.shape[2])
            ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=2)  # [H, T]
            assert np.max(np.abs(lse[b].T - ref_lse.numpy())) <= 1e-12, ("tokens lse", b)
    # one query token: exactly the plain decode
    inp = _tiny([9, 70, 3], 1200)
    args = list(W.oracle_args(inp))
    o1, l1 = O.decode(*args)
    args[0], args[1] = args[0][:, None], args[1][:, None]
    o2, l2 = O.decode_tokens(*args)
    assert np.array_equal(o1, o2[:, 0]) and np.array_equal(l1, l2[:, 0])


def gather_numpy(O):
    for seed, (seq, kw) in enumerate([([37, 64, 100], {}), ([1, 4, 9, 130], dict(d_c=16, d_R=4)),
                                      ([63, 65, 0, 128], {})]):
        B = len(seq)
        d = dict(TINY)
        d.update(kw)
        inp = W.make_inputs(B, d["H"], d["d_n"], d["d_c"], d["d_R"], d["d_v"], seq, 1300 + seed,
                            layout="shuffled", poison=True, page_size=4)
        kv = W.u16(inp["kv_pages"])
        pt = inp["page_table"].numpy().astype(np.int64)
        sl = inp["seq_lens"].numpy().astype(np.int64)
        P = inp["page_size"]
        S_max = pt.shape[1] * P
        # independent gather: numpy advanced indexing over every (b, t), then a zero mask
        t = np.arange(S_max)
        pages = pt[:, t // P]                                    # [B, S_max]
        ref = kv[pages, (t % P)[None, :]]                        # [B, S_max, d_c + d_R]
        ref = np.where((t[None, :] < sl[:, None])[:, :, None], ref, np.uint16(0))
        got = O.gather_pages(kv, inp["page_table"].numpy(), inp["seq_lens"].numpy(), S_max,
                             d["d_c"])
        assert got.dtype == np.uint16 and got.shape == ref.shape
        assert np.array_equal(got, ref), ("gather", seed)


ALL = [naive_equals_absorbed, sdpa_library, rows_sum_to_one, single_token, zero_query,
       identical_tokens, dominant_rope, permutation, split_combine, gather_numpy,
       tokens_causal_sdpa]
