"""Pins of the oracle's cache append (oracle.cache_append, oracle.rope_rotate): closed forms and
invariants of the rotary encoding, and brute force for the projections and the slot placement.
None of them retypes the oracle's formula."""
import math

import numpy as np
import torch

import oracle
import workloads as W


def test_rope_first_pair_turns_by_the_position():
    # the first pair's frequency is base^0 = 1: e_0 turns into (cos p) e_0 + (sin p) e_{d/2}
    for d in (8, 64):
        for p in (0.0, 1.0, 3.0, 1000.0):
            e = np.zeros(d)
            e[0] = 1.0
            r = oracle.rope_rotate(e, p)
            want = np.zeros(d)
            want[0], want[d // 2] = math.cos(p), math.sin(p)
            assert np.allclose(r, want, rtol=0, atol=1e-15)


def test_rope_frequencies_at_base_1e4_and_width_8():
    # d = 8, base 10^4: the four pair frequencies are 1, 0.1, 0.01, 0.001
    for j, f in enumerate((1.0, 0.1, 0.01, 0.001)):
        e = np.zeros(8)
        e[j] = 1.0
        p = 1.0 / f  # turns pair j by exactly one radian
        r = oracle.rope_rotate(e, p)
        assert abs(r[j] - math.cos(1.0)) <= 1e-12 and abs(r[j + 4] - math.sin(1.0)) <= 1e-12


def test_rope_is_a_rotation_by_relative_position():
    rng = np.random.default_rng(1)
    for d in (8, 64):
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        for m, n, s in ((5, 2, 7), (1000, 17, 4096), (0, 0, 1)):
            r = oracle.rope_rotate(k, n)
            assert abs(np.linalg.norm(r) - np.linalg.norm(k)) <= 1e-12  # length kept
            a = oracle.rope_rotate(q, m) @ oracle.rope_rotate(k, n)
            b = oracle.rope_rotate(q, m + s) @ oracle.rope_rotate(k, n + s)
            assert abs(a - b) <= 1e-9 * max(1.0, abs(a))  # depends on m - n only
        # turning by a then by b is turning by a + b; position 0 changes nothing
        assert np.allclose(oracle.rope_rotate(oracle.rope_rotate(k, 30), 12),
                           oracle.rope_rotate(k, 42), rtol=0, atol=1e-12)
        assert np.array_equal(oracle.rope_rotate(k, 0), k)


def test_append_projections_and_slots_by_brute_force():
    g = torch.Generator().manual_seed(3)
    B, T, hidden, d_c, d_R = 2, 3, 16, 4, 8
    x = torch.randn(B, T, hidden, generator=g).to(torch.bfloat16)
    Wd = (torch.randn(d_c, hidden, generator=g) / 4).to(torch.bfloat16)
    Wr = (torch.randn(d_R, hidden, generator=g) / 4).to(torch.bfloat16)
    pt = np.array([[5, 2, 7], [1, 0, 3]], dtype=np.int32)
    sl = np.array([62, 64], dtype=np.int32)
    rows, where = oracle.cache_append(W.u16(x), W.u16(Wd), W.u16(Wr), pt, sl)
    xf, wd, wr = x.double().numpy(), Wd.double().numpy(), Wr.double().numpy()
    for b in range(B):
        for i in range(T):
            p = int(sl[b]) + i
            assert tuple(where[b, i]) == (pt[b][p // 64], p % 64)
            for c in range(d_c):
                s = 0.0
                for k in range(hidden):
                    s += xf[b, i, k] * wd[c, k]
                assert abs(rows[b, i, c] - s) <= 1e-12
            kr = np.array([sum(xf[b, i, k] * wr[j, k] for k in range(hidden)) for j in range(d_R)])
            assert np.allclose(rows[b, i, d_c:], oracle.rope_rotate(kr, p), rtol=0, atol=1e-12)
