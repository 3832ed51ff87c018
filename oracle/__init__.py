"""CPU fp64 oracle for absorbed MLA decode (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The GPU library never calls it and shares no code with it.

All arrays are numpy. bf16 tensors are passed as their uint16 bit patterns; the C code
widens them exactly to fp64 and does every step in fp64 (see ``mla_oracle.c`` for the
steps and the passages of the pages each one follows).

Pins (what each function is checked against) live in ``tests/test_oracle_*.py``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIBS = {}

_U16P = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_I32P = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_F64P = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


def _lib(mutant=0, path=None):
    key = (mutant, path)
    if key in _LIBS:
        return _LIBS[key]
    if path is None:
        path = _build.LIB if mutant == 0 else os.path.join(
            _build.HERE, "libmla_oracle_mutant%d.so" % mutant)
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build(out=path, mutant=mutant)
    L = ctypes.CDLL(path)
    i = ctypes.c_int
    vp = ctypes.c_void_p
    L.oracle_decode_absorbed.restype = i
    L.oracle_decode_absorbed.argtypes = [i] * 8 + [_U16P] * 5 + [_I32P, _I32P, ctypes.c_double,
                                                                 vp, i, i, _F64P, vp, i]
    L.oracle_decode_naive.restype = i
    L.oracle_decode_naive.argtypes = [i] * 8 + [_U16P] * 5 + [_I32P, _I32P, ctypes.c_double,
                                                              _F64P, vp, i]
    L.oracle_probs.restype = i
    L.oracle_probs.argtypes = [i] * 8 + [_U16P] * 4 + [_I32P, _I32P, ctypes.c_double, i, i,
                                                       _F64P]
    L.oracle_gather_pages.restype = i
    L.oracle_gather_pages.argtypes = [i] * 5 + [_U16P, _I32P, _I32P, i, _U16P]
    L.oracle_mutant.restype = i
    _LIBS[key] = L
    return L


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns, got %s" % a.dtype)
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _dims(q_nope, q_rope, W_UK, W_UV, kv_pages, page_table):
    B, H, d_n = q_nope.shape
    d_R = q_rope.shape[2]
    d_c = W_UK.shape[2]
    d_v = W_UV.shape[2]
    page_size = kv_pages.shape[1]
    if q_rope.shape[:2] != (B, H) or W_UK.shape != (H, d_n, d_c) or W_UV.shape != (H, d_c, d_v) \
            or kv_pages.shape[2] != d_c + d_R or page_table.shape[0] != B:
        raise ValueError("inconsistent shapes")
    return B, H, d_n, d_c, d_R, d_v, page_size, page_table.shape[1]


class Oracle:
    """Handle on one build of the oracle (mutant=0 is the real one)."""

    def __init__(self, mutant=0, path=None):
        self.L = _lib(mutant, path)
        self.mutant = self.L.oracle_mutant()

    def decode(self, q_nope, q_rope, W_UK, W_UV, kv_pages, page_table, seq_lens, scale=0.0,
               pairs=None, n_split=1, threads=0):
        """Absorbed decode. Returns (out, lse): out [B,H,d_v] fp64 and lse [B,H] fp64, or
        for an explicit ``pairs`` list of (b,h): out [n,d_v] and lse [n]."""
        args = [_u16(q_nope), _u16(q_rope), _u16(W_UK), _u16(W_UV), _u16(kv_pages)]
        dims = _dims(*args, page_table)
        B, H, d_v = dims[0], dims[1], dims[5]
        pt, sl = _i32(page_table), _i32(seq_lens)
        if pairs is None:
            n, pp = B * H, None
            out = np.zeros((B, H, d_v))
            lse = np.zeros((B, H))
        else:
            pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
            n, pp = pairs.shape[0], pairs.ctypes.data
            out = np.zeros((n, d_v))
            lse = np.zeros((n,))
        rc = self.L.oracle_decode_absorbed(*dims, *args, pt, sl, float(scale), pp, n,
                                           int(n_split), out, lse.ctypes.data, int(threads))
        if rc != 0:
            raise ValueError("oracle_decode_absorbed failed (%d)" % rc)
        return out, lse

    def decode_tokens(self, q_nope, q_rope, W_UK, W_UV, kv_pages, page_table, seq_lens,
                      scale=0.0, threads=0):
        """Several query tokens per sequence: q_nope [B,T,H,d_n], q_rope [B,T,H,d_R]. Query
        token i of sequence b is the token at position S_b - T + i (the T newest tokens are in
        the cache); it attends to the cached tokens 0 .. S_b - T + i, itself included, i.e.
        the decode above over the first S_b - T + 1 + i tokens of sequence b. Returns
        out [B,T,H,d_v] and lse [B,T,H]."""
        q_nope, q_rope = _u16(q_nope), _u16(q_rope)
        B, T, H = q_nope.shape[:3]
        sl = _i32(seq_lens)
        lens = np.repeat(sl, T) - (T - 1 - np.tile(np.arange(T, dtype=np.int32), B))
        if np.any(lens <= 0):
            raise ValueError("every query token needs at least one token to attend to")
        rows = np.repeat(np.arange(B), T)
        out, lse = self.decode(q_nope.reshape(B * T, H, -1), q_rope.reshape(B * T, H, -1),
                               W_UK, W_UV, kv_pages, _i32(page_table)[rows], lens, scale=scale,
                               threads=threads)
        return out.reshape(B, T, H, -1), lse.reshape(B, T, H)

    def decode_naive(self, q_nope, q_rope, W_UK, W_UV, kv_pages, page_table, seq_lens,
                     scale=0.0, threads=0):
        """Naive decompressed decode (K and V materialised per head). Returns (out, lse)."""
        args = [_u16(q_nope), _u16(q_rope), _u16(W_UK), _u16(W_UV), _u16(kv_pages)]
        dims = _dims(*args, page_table)
        B, H, d_v = dims[0], dims[1], dims[5]
        out = np.zeros((B, H, d_v))
        lse = np.zeros((B, H))
        rc = self.L.oracle_decode_naive(*dims, *args, _i32(page_table), _i32(seq_lens),
                                        float(scale), out, lse.ctypes.data, int(threads))
        if rc != 0:
            raise ValueError("oracle_decode_naive failed (%d)" % rc)
        return out, lse

    def probs(self, q_nope, q_rope, W_UK, W_UV, kv_pages, page_table, seq_lens, b, h,
              scale=0.0):
        """Softmax weights p_t, t < S_b, of one (b,h)."""
        args = [_u16(q_nope), _u16(q_rope), _u16(W_UK), _u16(W_UV), _u16(kv_pages)]
        dims = _dims(*args, page_table)
        sl = _i32(seq_lens)
        p = np.zeros((int(sl[b]),))
        rc = self.L.oracle_probs(*dims, args[0], args[1], args[2], args[4], _i32(page_table), sl,
                                 float(scale), int(b), int(h), p)
        if rc != 0:
            raise ValueError("oracle_probs failed (%d)" % rc)
        return p

    def gather_pages(self, kv_pages, page_table, seq_lens, S_max, d_c):
        """Logical copy of the paged cache: [B, S_max, d_c+d_R] uint16, zero past S_b."""
        kv = _u16(kv_pages)
        pt, sl = _i32(page_table), _i32(seq_lens)
        B = pt.shape[0]
        w = kv.shape[2]
        dst = np.zeros((B, int(S_max), w), dtype=np.uint16)
        rc = self.L.oracle_gather_pages(B, int(d_c), w - int(d_c), kv.shape[1], pt.shape[1], kv,
                                        pt, sl, int(S_max), dst)
        if rc != 0:
            raise ValueError("oracle_gather_pages failed (%d)" % rc)
        return dst


def decode_out(q_nope, q_rope, W_UK, W_UVO, kv_pages, page_table, seq_lens, scale=0.0,
               threads=0):
    """The decode followed by the merged output projection (lpnh.cn/news/2494972 S2.2: W_uv
    and W_o merged offline): out[b, n] = sum_{h,c} o_lat[b,h,c] W_UVO[n, h*d_c + c], with
    o_lat the latent attention output (the decode's result before W_UV). W_UVO is uint16 bf16
    bits [hidden, H*d_c] or an fp64 array. Queries [B,H,.] or [B,T,H,.]. Returns
    (out [.., hidden], lse [.., H])."""
    q_nope = _u16(q_nope)
    H, d_c = W_UK.shape[0], W_UK.shape[2]
    # o_lat: the decode with W_UV = identity per head (exact in fp64)
    eye = np.zeros((H, d_c, d_c), dtype=np.uint16)
    eye[:, np.arange(d_c), np.arange(d_c)] = 0x3F80  # bf16 1.0
    if q_nope.ndim == 4:
        o_lat, lse = default().decode_tokens(q_nope, q_rope, W_UK, eye, kv_pages, page_table,
                                             seq_lens, scale=scale, threads=threads)
    else:
        o_lat, lse = default().decode(q_nope, q_rope, W_UK, eye, kv_pages, page_table, seq_lens,
                                      scale=scale, threads=threads)
    W = np.asarray(W_UVO)
    W = _f64(W) if W.dtype == np.uint16 else W.astype(np.float64)
    out = o_lat.reshape(o_lat.shape[:-2] + (H * d_c,)) @ W.T
    return out, lse


def rope_rotate(k, pos, base=10000.0):
    """Rotary position encoding of one vector k [d] (d even) at position pos, in fp64: the
    pairs (k[j], k[j + d/2]) turn by the angle pos * base^(-2j/d) (lpnh.cn/news/2494972 S2.1
    RoPE on the decoupled key; pairing of the two halves is this library's reading)."""
    k = np.asarray(k, dtype=np.float64)
    d = k.shape[-1]
    h = d // 2
    out = np.empty_like(k)
    for j in range(h):
        a = pos * base ** (-2.0 * j / d)
        c, s = np.cos(a), np.sin(a)
        out[..., j] = k[..., j] * c - k[..., j + h] * s
        out[..., j + h] = k[..., j] * s + k[..., j + h] * c
    return out


def cache_append(x, W_DKV, W_KR, page_table, seq_lens, base=10000.0):
    """Cache append in fp64 (lpnh.cn/news/2494972 S2.1: c_kv = x W_dkv, and the decoupled
    RoPE key; bhfrc.com/news/60867 S1 [c_KV | k_R] format): for token i of sequence b, at
    position p = seq_lens[b] + i, the row [x W_DKV^T | rope(x W_KR^T, p)]. x is uint16 bf16
    bits [B, T, hidden]; W_DKV [d_c, hidden], W_KR [d_R, hidden]. Returns rows [B, T, d_c+d_R]
    (fp64, not rounded) and, per (b, i), its (page, slot) from the page table."""
    x = _f64(_u16(x))
    Wd, Wr = _f64(_u16(W_DKV)), _f64(_u16(W_KR))
    B, T = x.shape[:2]
    pt, sl = _i32(page_table), _i32(seq_lens)
    P = 64
    rows = np.zeros((B, T, Wd.shape[0] + Wr.shape[0]))
    where = np.zeros((B, T, 2), dtype=np.int64)
    for b in range(B):
        for i in range(T):
            p = int(sl[b]) + i
            rows[b, i, :Wd.shape[0]] = Wd @ x[b, i]
            rows[b, i, Wd.shape[0]:] = rope_rotate(Wr @ x[b, i], p, base)
            where[b, i] = (pt[b, p // P], p % P)
    return rows, where


def cache_append_fp8(x, W_DKV, W_KR, page_table, seq_lens, base=10000.0):
    """Cache append into an FP8 cache: cache_append's rows with the latent part quantised per
    token (quantise_fp8_row) and the RoPE key left in fp64 (stored as bf16). Returns
    (codes uint8 [B, T, d_c], scales [B, T], k_R fp64 [B, T, d_R], where [B, T, 2])."""
    rows, where = cache_append(x, W_DKV, W_KR, page_table, seq_lens, base)
    d_c = _u16(W_DKV).shape[0]
    B, T = rows.shape[:2]
    codes = np.zeros((B, T, d_c), dtype=np.uint8)
    scales = np.zeros((B, T))
    for b in range(B):
        for i in range(T):
            codes[b, i], scales[b, i] = quantise_fp8_row(rows[b, i, :d_c])
    return codes, scales, rows[:, :, d_c:], where


def fp8_e4m3_value(code):
    """Exact value of FP8 E4M3 bytes (the OCP 8-bit float format with 4 exponent bits, bias 7,
    and 3 mantissa bits; no infinities, S.1111.111 is NaN), as fp64. This is the element format
    of the quantised latent cache (the pages' quantised gather of the latent cache,
    bhfrc.com/news/60867 S1 and S5, read as an 8-bit float cache with per-token scales)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, v)


def fp8_e4m3_encode(v):
    """The E4M3 byte nearest to each value v (fp64, |v| <= 448, no NaN): among the 127 finite
    non-negative E4M3 values, the nearest to |v|, a tie going to the even code (last mantissa
    bit 0), with the sign bit of v (0 gets code 0x00). This is round-to-nearest-even into the
    format fp8_e4m3_value reads, written out as a search over the format's values."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)) or np.any(np.abs(v) > 448.0):
        raise ValueError("E4M3 encodes finite values of magnitude at most 448")
    codes = np.arange(127)
    vals = fp8_e4m3_value(codes)                 # increasing in the code
    a = np.abs(v)
    hi = np.clip(np.searchsorted(vals, a), 0, 126)  # first value >= |v|
    lo = np.clip(hi - 1, 0, 126)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == vals[hi], hi, pick)
    return (pick | np.where((v < 0) & (pick != 0), 0x80, 0)).astype(np.uint8)


def fp8_scale_exponent(amax):
    """The exponent e of an FP8 row's scale 2^e: the smallest integer with
    amax <= 448 * 2^e (448 = 0.875 * 2^9, the largest E4M3 value), kept within -126 .. 127;
    0 for amax = 0. With amax = m * 2^k, 0.5 <= m < 1, that is k - 9 when m <= 0.875, else
    k - 8 (exact)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    m, k = np.frexp(amax)
    e = int(k) - 9 if m <= 0.875 else int(k) - 8
    return min(127, max(-126, e))


def quantise_fp8_row(c):
    """A latent row c (fp64) as an FP8 cache row: (E4M3 codes of c / 2^e, 2^e) with e from
    fp8_scale_exponent(max |c|) (the writer of the quantised latent cache, bhfrc.com/news/60867
    S1 and S5, read as a per-token power-of-two scaled E4M3 cache)."""
    c = np.asarray(c, dtype=np.float64)
    e = fp8_scale_exponent(np.max(np.abs(c)) if c.size else 0.0)
    return fp8_e4m3_encode(c * 2.0 ** -e), 2.0 ** e


def check_scales(scales):
    """The per-token scales of an FP8 cache as fp64, after checking the format's contract:
    every scale is a positive normal power of two (exponent-only, as in the microscaling
    formats), i.e. 2^e with -126 <= e <= 127. NaN is accepted (a slot no sequence uses may
    hold anything); any other value raises ValueError."""
    s = np.asarray(scales, dtype=np.float64)
    ok = np.isnan(s)
    with np.errstate(invalid="ignore"):
        m, e = np.frexp(np.where(ok, 1.0, s))
    pow2 = (m == 0.5) & (e - 1 >= -126) & (e - 1 <= 127) & (s > 0)
    if not np.all(ok | pow2):
        bad = s[~(ok | pow2)]
        raise ValueError("FP8 cache scales must be positive normal powers of two; got %r"
                         % (bad[:4].tolist(),))
    return s


def dequant_fp8_cache(kv8, scales, d_c):
    """The bf16 cache that an FP8 cache stands for: token row [c_KV bytes (d_c) | k_R bf16
    (2*d_R bytes)] with a positive normal fp32 power-of-two scale per token slot
    (check_scales);
    c_KV[c] = value(byte c) * scale, k_R copied. Returns uint16 bf16 bits [P, 64, d_c + d_R].
    Every product is a bf16 value (an E4M3 value times a power of two, in range); the function
    checks that rather than assume it."""
    kv8 = np.ascontiguousarray(kv8, dtype=np.uint8)
    P, ps, w8 = kv8.shape
    d_R = (w8 - d_c) // 2
    v = fp8_e4m3_value(kv8[:, :, :d_c]) * check_scales(scales)[:, :, None]
    f = v.astype(np.float32)
    ok = np.isnan(v) | (f.astype(np.float64) == v)
    bits = f.view(np.uint32)
    if not np.all(ok) or np.any((bits[~np.isnan(v)] & 0xFFFF) != 0):
        raise ValueError("dequantised c_KV is not exactly a bf16 value")
    out = np.empty((P, ps, d_c + d_R), dtype=np.uint16)
    out[:, :, :d_c] = np.where(np.isnan(v), 0x7FC0, bits >> 16).astype(np.uint16)
    out[:, :, d_c:] = kv8[:, :, d_c:].copy().view(np.uint16).reshape(P, ps, d_R)
    return out


# ---- MXFP4 latent cache (the pages' 4-bit quantised gather of the latent cache,
# bhfrc.com/news/60867 S1 and S5, in the OCP Microscaling (MX) v1.0 format: blocks of 32
# elements, each an FP4 E2M1 value, sharing one E8M0 power-of-two scale)

MX_BLOCK = 32
FP4_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # E2M1 codes 0..7, see below


def fp4_e2m1_value(code):
    """Exact value of FP4 E2M1 codes (4 bits: sign, 2 exponent bits with bias 1, 1 mantissa
    bit; exponent 0 is subnormal: 0 or 0.5; no infinities or NaN), as fp64. Only the low four
    bits of each code are read."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e.astype(np.float64) - 1.0))
    return np.where(c & 0x8, -mag, mag)


def fp4_e2m1_encode(v):
    """The E2M1 code nearest to each value v (fp64, finite): among the 8 non-negative E2M1
    values, the nearest to min(|v|, 6) (magnitudes above the largest, 6, saturate to it, as the
    MX conversion does), a tie going to the even code (mantissa bit 0), with the sign of v in
    bit 3 unless the magnitude code is 0 (zero is stored as +0)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E2M1 encodes finite values")
    vals = fp4_e2m1_value(np.arange(8))          # increasing in the code
    a = np.minimum(np.abs(v), vals[7])
    hi = np.clip(np.searchsorted(vals, a), 0, 7)  # first value >= |v|
    lo = np.clip(hi - 1, 0, 7)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == vals[hi], hi, pick)
    return (pick | np.where((v < 0) & (pick != 0), 0x8, 0)).astype(np.uint8)


def e8m0_value(code):
    """Exact value of E8M0 scale bytes: 2^(code - 127), code 255 is NaN."""
    c = np.asarray(code, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def mx_scale_exponent(amax):
    """The shared exponent X of an MXFP4 block (its scale 2^X): floor(log2(amax)) minus 2, the
    exponent of E2M1's largest value (6 = 1.5 * 2^2), kept within E8M0's -127 .. 127; 0 for an
    all-zero block. With amax = m * 2^k, 0.5 <= m < 1, floor(log2(amax)) = k - 1 (exact)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    _, k = np.frexp(amax)
    return min(127, max(-127, int(k) - 1 - 2))


def quantise_mxfp4_row(c):
    """A latent row c (fp64, length a multiple of 32) as MXFP4: per block of 32 elements the
    shared exponent X = mx_scale_exponent(max |c_block|) and the E2M1 codes of c_block / 2^X.
    Returns (codes uint8 [len(c)], one code per element, and scale bytes uint8 [len(c)/32],
    X + 127)."""
    c = np.asarray(c, dtype=np.float64)
    if c.size % MX_BLOCK:
        raise ValueError("an MXFP4 row holds whole blocks of 32 elements")
    blocks = c.reshape(-1, MX_BLOCK)
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    scales = np.zeros(blocks.shape[0], dtype=np.uint8)
    for k, blk in enumerate(blocks):
        X = mx_scale_exponent(np.max(np.abs(blk)))
        codes[k] = fp4_e2m1_encode(blk * 2.0 ** -X)
        scales[k] = X + 127
    return codes.reshape(-1), scales


def pack_fp4(codes):
    """E2M1 codes [..., n] (n even) as bytes [..., n/2]: element 2k in the low nibble of byte
    k, element 2k + 1 in its high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_fp4(packed):
    """The inverse of pack_fp4: bytes [..., m] -> codes [..., 2m]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_mxfp4_cache(kv4, scales, d_c):
    """The bf16 cache that an MXFP4 cache stands for: token row [c_KV as packed E2M1
    (d_c/2 bytes) | k_R bf16 (2*d_R bytes)] and per token d_c/32 E8M0 scale bytes;
    c_KV[c] = value(code c) * 2^(scale[c/32] - 127), k_R copied. Returns uint16 bf16 bits
    [P, 64, d_c + d_R]; a NaN scale (255) gives NaN values. Every finite product is a bf16
    value (at most 2 significant bits, exponent in range); the function checks that rather
    than assume it."""
    kv4 = np.ascontiguousarray(kv4, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    P, ps, w4 = kv4.shape
    d_R = (w4 - d_c // 2) // 2
    nb = d_c // MX_BLOCK
    if sc.shape != (P, ps, nb):
        raise ValueError("scales must be [P, 64, d_c/32]")
    v = fp4_e2m1_value(unpack_fp4(kv4[:, :, :d_c // 2])) * \
        np.repeat(e8m0_value(sc), MX_BLOCK, axis=2)
    f = v.astype(np.float32)
    nan = np.isnan(v)
    with np.errstate(invalid="ignore"):
        ok = nan | (f.astype(np.float64) == v)
    bits = f.view(np.uint32)
    if not np.all(ok) or np.any((bits[~nan] & 0xFFFF) != 0):
        raise ValueError("dequantised c_KV is not exactly a bf16 value")
    out = np.empty((P, ps, d_c + d_R), dtype=np.uint16)
    out[:, :, :d_c] = np.where(nan, 0x7FC0, bits >> 16).astype(np.uint16)
    out[:, :, d_c:] = kv4[:, :, d_c // 2:].copy().view(np.uint16).reshape(P, ps, d_R)
    return out


def cache_append_mxfp4(x, W_DKV, W_KR, page_table, seq_lens, base=10000.0):
    """Cache append into an MXFP4 cache: cache_append's rows with the latent part quantised per
    token and block (quantise_mxfp4_row) and the RoPE key left in fp64 (stored as bf16).
    Returns (codes uint8 [B, T, d_c] one per element, scale bytes uint8 [B, T, d_c/32],
    k_R fp64 [B, T, d_R], where [B, T, 2])."""
    rows, where = cache_append(x, W_DKV, W_KR, page_table, seq_lens, base)
    d_c = _u16(W_DKV).shape[0]
    B, T = rows.shape[:2]
    codes = np.zeros((B, T, d_c), dtype=np.uint8)
    scales = np.zeros((B, T, d_c // MX_BLOCK), dtype=np.uint8)
    for b in range(B):
        for i in range(T):
            codes[b, i], scales[b, i] = quantise_mxfp4_row(rows[b, i, :d_c])
    return codes, scales, rows[:, :, d_c:], where


def _f64(u16):
    """Exact fp64 value of bf16 bit patterns."""
    return (np.asarray(u16, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


_DEFAULT = None


def default():
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def decode(*a, **k):
    return default().decode(*a, **k)


def decode_naive(*a, **k):
    return default().decode_naive(*a, **k)


def decode_tokens(*a, **k):
    return default().decode_tokens(*a, **k)


def probs(*a, **k):
    return default().probs(*a, **k)


def gather_pages(*a, **k):
    return default().gather_pages(*a, **k)
