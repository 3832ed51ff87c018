"""The C-ABI library loads, exports what include/mla_decode.h declares, and rejects bad
arguments before it enqueues anything. No call here passes validation, so nothing touches a GPU
(the pointers are placeholders, never dereferenced)."""
import ctypes

import pytest

import mla_latent_kv_14_amd as M
from mla_latent_kv_14_amd.binding import STATUS_CODE

EXPECTED = ["mla_cache_append", "mla_cache_append_fp8", "mla_cache_append_mxfp4",
            "mla_cache_append_workspace_bytes",
            "mla_decode", "mla_decode_fp8", "mla_decode_mxfp4", "mla_decode_noalloc",
            "mla_decode_out", "mla_decode_timed",
            "mla_decode_workspace_bytes", "mla_gather_pages", "mla_last_hip_error",
            "mla_status_str"]


def test_header_declares_the_boundary():
    assert M.header_symbols() == EXPECTED


def test_library_exports_every_declared_symbol():
    L = M.lib()
    for name in M.header_symbols():
        assert getattr(L, name) is not None


def ds_dims(B=16, max_pages=64, num_pages=1024, max_seq_len=4096, units=0):
    d = M.Dims()
    d.batch, d.num_heads, d.d_nope, d.d_latent, d.d_rope, d.d_v = B, 128, 128, 512, 64, 128
    d.page_size, d.max_pages_per_seq, d.num_pages = 64, max_pages, num_pages
    d.max_seq_len, d.softmax_scale, d.num_units = max_seq_len, 0.0, units
    return d


def m2_dims(B=32, max_pages=512, num_pages=16384, max_seq_len=32768, units=0):
    d = ds_dims(B, max_pages, num_pages, max_seq_len, units)
    d.num_heads, d.d_nope, d.d_latent, d.d_rope, d.d_v = 32, 120, 64, 8, 128
    return d


def _al(n=1):
    return ctypes.c_void_p(0x100000 * n)  # 256-aligned placeholder, never dereferenced


def call(d, ptrs=None, ws=None, ws_bytes=None, lse=None):
    p = ptrs or [_al(i + 1) for i in range(8)]
    if ws is None:
        ws = _al(9)
    if ws_bytes is None:
        ws_bytes = M.workspace_bytes(d) if M.workspace_bytes(d) else 1 << 40
    return M.lib().mla_decode(ctypes.byref(d), *p, lse or ctypes.c_void_p(0), ws, ws_bytes,
                              ctypes.c_void_p(0))


def test_workspace_bytes_closed_form():
    # plan (header + offsets, then one 32-byte start record per unit at a 32-byte boundary),
    # q_abs, per-slot lse, per-slot bf16 partials (slots = units + B)
    def plan(B, G):
        return (16 + 4 * B + 31) // 32 * 32 + 32 * G
    def al(x):
        return (x + 255) // 256 * 256
    d = ds_dims()
    slots = 128 + 16
    assert M.workspace_bytes(d) == (al(plan(16, 128)) + al(16 * 128 * 512 * 2) + al(slots * 128 * 4)
                                    + al(slots * 128 * 512 * 2))
    # MHA2MLA widths: sized for the FP8 cache's plan, 2048 units (two work groups per CU),
    # which also covers the bf16 cache's 1024
    d = m2_dims()
    slots = 2048 + 32
    assert M.workspace_bytes(d) == (al(plan(32, 2048)) + al(32 * 32 * 64 * 2) + al(slots * 32 * 4)
                                    + al(slots * 32 * 64 * 2))
    # units are capped by the tiles that can exist: B=1, S=512 -> 16 tiles of 32 tokens
    d = ds_dims(B=1, max_pages=8, num_pages=8, max_seq_len=512)
    assert M.workspace_bytes(d) == al(plan(1, 16)) + al(128 * 512 * 2) + al(17 * 128 * 4) + \
        al(17 * 128 * 512 * 2)


@pytest.mark.parametrize("field,value,status", [
    ("num_heads", 64, "MLA_ERR_UNSUPPORTED"), ("d_latent", 256, "MLA_ERR_UNSUPPORTED"),
    ("page_size", 16, "MLA_ERR_UNSUPPORTED"), ("batch", 0, "MLA_ERR_BAD_DIMS"),
    ("max_pages_per_seq", 0, "MLA_ERR_BAD_DIMS"), ("num_pages", 0, "MLA_ERR_BAD_DIMS"),
    ("max_seq_len", 64 * 64 + 1, "MLA_ERR_BAD_DIMS"), ("num_units", -1, "MLA_ERR_BAD_DIMS"),
    ("num_units", 65537, "MLA_ERR_BAD_DIMS"), ("q_len", -1, "MLA_ERR_BAD_DIMS"),
    ("q_len", 65537, "MLA_ERR_BAD_DIMS"), ("prefill_threshold", -1, "MLA_ERR_BAD_DIMS")])
def test_bad_dims(field, value, status):
    d = ds_dims(max_seq_len=0)  # 0: bounded by the page table alone
    setattr(d, field, value)
    assert M.workspace_bytes(d) == 0
    assert call(d) == STATUS_CODE[status]


def test_prefill_workspace_and_limits():
    al = lambda x: (x + 255) // 256 * 256
    # q_len at the threshold (256 by default): the decompressed branch's workspace, a flag
    # word, W_UV transposed, and the keys and values of one group of sequences (as many as fit
    # in 1 GiB of them, at least one)
    d = ds_dims(B=4, max_pages=16, num_pages=64, max_seq_len=1024)
    d.q_len = 256
    per_seq = 1024 * 128 * (128 + 128) * 2  # 64 MiB
    g = 4
    assert M.workspace_bytes(d) == 256 + al(128 * 128 * 512 * 2) + al(g * 1024 * 128 * 128 * 2) \
        + al(g * 1024 * 128 * 128 * 2)
    d.max_seq_len = 8192
    d.max_pages_per_seq = 128
    g = 2  # 512 MiB per sequence
    assert M.workspace_bytes(d) == 256 + al(128 * 128 * 512 * 2) + 2 * al(g * 8192 * 128 * 128 * 2)
    prefill_bytes = M.workspace_bytes(d)
    # one token below the threshold: the absorbed branch's workspace (1020 virtual rows)
    d.q_len = 255
    slots = 128 + 4 * 255
    plan = (16 + 4 * 1020 + 31) // 32 * 32 + 32 * 128
    assert M.workspace_bytes(d) == al(plan) + al(1020 * 128 * 512 * 2) + al(slots * 128 * 4) \
        + al(slots * 128 * 512 * 2)
    # the threshold moves: q_len 255 from threshold 128 on is decompressed
    d.prefill_threshold = 128
    assert M.workspace_bytes(d) == prefill_bytes
    # MHA2MLA widths: absorbed at any T unless a threshold is set
    d = m2_dims(B=2, max_pages=16, num_pages=64, max_seq_len=1024)
    d.q_len = 300
    absorbed = M.workspace_bytes(d)
    d.prefill_threshold = 256
    assert M.workspace_bytes(d) == 256 + al(32 * 128 * 64 * 2) + al(2 * 1024 * 32 * 120 * 2) \
        + al(2 * 1024 * 32 * 128 * 2) != absorbed
    # the decompressed branch reads a bf16 cache and writes per-head outputs
    d = ds_dims(B=2, max_pages=16, num_pages=64, max_seq_len=1024)
    d.q_len = 300
    p = [_al(k + 1) for k in range(5)] + [_al(6)] + [_al(k + 7) for k in range(3)]
    assert M.lib().mla_decode_fp8(ctypes.byref(d), *p, ctypes.c_void_p(0), _al(10),
                                  M.workspace_bytes(d), ctypes.c_void_p(0), None) == \
        STATUS_CODE["MLA_ERR_UNSUPPORTED"]
    q = [_al(k + 1) for k in range(9)]
    assert M.lib().mla_decode_out(ctypes.byref(d), 1024, *q[:8], ctypes.c_void_p(0), _al(10),
                                  M.workspace_bytes(d), ctypes.c_void_p(0)) == \
        STATUS_CODE["MLA_ERR_UNSUPPORTED"]


def test_null_dims_and_pointers():
    assert M.lib().mla_decode(None, *([_al()] * 10), 1 << 30, None) == STATUS_CODE["MLA_ERR_NULL_ARG"]
    for i in range(8):
        p = [_al(k + 1) for k in range(8)]
        p[i] = ctypes.c_void_p(0)
        assert call(ds_dims(), ptrs=p) == STATUS_CODE["MLA_ERR_NULL_ARG"], i


def test_misaligned():
    for i in range(8):
        p = [_al(k + 1) for k in range(8)]
        p[i] = ctypes.c_void_p(0x100008)
        assert call(ds_dims(), ptrs=p) == STATUS_CODE["MLA_ERR_MISALIGNED"], i
    assert call(ds_dims(), lse=ctypes.c_void_p(0x100004)) == STATUS_CODE["MLA_ERR_MISALIGNED"]
    assert call(ds_dims(), ws=ctypes.c_void_p(0x100010)) == STATUS_CODE["MLA_ERR_MISALIGNED"]


def test_workspace_too_small_or_missing():
    d = ds_dims()
    need = M.workspace_bytes(d)
    assert call(d, ws_bytes=need - 1) == STATUS_CODE["MLA_ERR_WORKSPACE"]
    assert call(d, ws=ctypes.c_void_p(0)) == STATUS_CODE["MLA_ERR_WORKSPACE"]
    # MHA2MLA widths: the bf16 cache needs its own plan's bytes (1024 units), the FP8 cache
    # the full mla_decode_workspace_bytes (2048 units)
    d = m2_dims()
    al = lambda x: (x + 255) // 256 * 256
    bf16_need = (al((16 + 4 * 32 + 31) // 32 * 32 + 32 * 1024) + al(32 * 32 * 64 * 2)
                 + al(1056 * 32 * 4) + al(1056 * 32 * 64 * 2))
    assert call(d, ws_bytes=bf16_need - 256) == STATUS_CODE["MLA_ERR_WORKSPACE"]
    p = [_al(k + 1) for k in range(5)] + [_al(6)] + [_al(k + 7) for k in range(3)]
    assert M.lib().mla_decode_fp8(ctypes.byref(d), *p, ctypes.c_void_p(0), _al(10),
                                  M.workspace_bytes(d) - 256, ctypes.c_void_p(0), None) == \
        STATUS_CODE["MLA_ERR_WORKSPACE"]


def test_noalloc_scratch_size_matches_header():
    import re
    text = open(M.binding.HEADER).read()
    m = re.search(r"#define MLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == M.NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_before_enqueueing():
    # dims checks and the scratch limit come before any device call
    def noalloc(d):
        p = [_al(k + 1) for k in range(9)]
        return M.lib().mla_decode_noalloc(ctypes.byref(d) if d is not None else None, *p,
                                          ctypes.c_void_p(0))
    assert noalloc(None) == STATUS_CODE["MLA_ERR_NULL_ARG"]
    d = ds_dims()
    d.page_size = 32
    assert noalloc(d) == STATUS_CODE["MLA_ERR_BAD_DIMS"]
    # the five benchmark workloads fit; 4096 DeepSeek sequences do not
    assert M.workspace_bytes(ds_dims(B=64, max_pages=128)) <= M.NOALLOC_SCRATCH_BYTES
    d = ds_dims(B=4096, max_pages=512, num_pages=1 << 20, max_seq_len=32768)
    assert M.workspace_bytes(d) > M.NOALLOC_SCRATCH_BYTES
    assert noalloc(d) == STATUS_CODE["MLA_ERR_WORKSPACE"]
    d = m2_dims(B=8192, max_pages=512, num_pages=1 << 22)
    assert M.workspace_bytes(d) > M.NOALLOC_SCRATCH_BYTES
    assert noalloc(d) == STATUS_CODE["MLA_ERR_WORKSPACE"]


def test_gather_rejects_bad_args():
    L = M.lib()
    d = ds_dims()
    args = [_al(1), _al(2), _al(3), _al(4), ctypes.c_void_p(0)]
    assert L.mla_gather_pages(None, *args) == STATUS_CODE["MLA_ERR_NULL_ARG"]
    d.d_latent = 128
    assert L.mla_gather_pages(ctypes.byref(d), *args) == STATUS_CODE["MLA_ERR_UNSUPPORTED"]
    d = ds_dims()
    assert L.mla_gather_pages(ctypes.byref(d), _al(1), _al(2), ctypes.c_void_p(0), _al(4),
                              ctypes.c_void_p(0)) == STATUS_CODE["MLA_ERR_NULL_ARG"]
    assert L.mla_gather_pages(ctypes.byref(d), ctypes.c_void_p(0x100002), _al(2), _al(3), _al(4),
                              ctypes.c_void_p(0)) == STATUS_CODE["MLA_ERR_MISALIGNED"]


def test_workspace_grows_with_query_tokens():
    # T query tokens per sequence: B*T rows of queries and partial slots, units capped by the
    # tiles of B*T rows
    def plan(B, G):
        return (16 + 4 * B + 31) // 32 * 32 + 32 * G
    def al(x):
        return (x + 255) // 256 * 256
    d = ds_dims(B=4, max_pages=8, num_pages=32, max_seq_len=512)
    d.q_len = 3
    rows, units = 12, min(128, 12 * 16)
    slots = units + rows
    assert M.workspace_bytes(d) == (al(plan(rows, units)) + al(rows * 128 * 512 * 2)
                                    + al(slots * 128 * 4) + al(slots * 128 * 512 * 2))


def test_decode_out_rejects_bad_hidden():
    L = M.lib()
    d = ds_dims()
    p = [_al(k + 1) for k in range(8)]
    for hidden, status in ((0, "MLA_ERR_BAD_DIMS"), (-4, "MLA_ERR_BAD_DIMS"),
                           (100, "MLA_ERR_UNSUPPORTED")):
        assert L.mla_decode_out(ctypes.byref(d), hidden, *p, ctypes.c_void_p(0), _al(9),
                                M.workspace_bytes(d), ctypes.c_void_p(0)) == STATUS_CODE[status]


def _append_dims(B=16, T=1, hidden=7168, d_c=512, d_R=64):
    d = M.AppendDims()
    d.batch, d.q_len, d.hidden, d.d_latent, d.d_rope = B, T, hidden, d_c, d_R
    d.page_size, d.max_pages_per_seq, d.num_pages, d.rope_base = 64, 64, 1024, 10000.0
    return d


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, "MLA_ERR_BAD_DIMS"), ("q_len", -1, "MLA_ERR_BAD_DIMS"),
    ("hidden", 1000, "MLA_ERR_UNSUPPORTED"), ("hidden", 1536, "MLA_ERR_UNSUPPORTED"), ("d_latent", 510, "MLA_ERR_UNSUPPORTED"),
    ("d_rope", 10, "MLA_ERR_UNSUPPORTED"), ("page_size", 16, "MLA_ERR_UNSUPPORTED"),
    ("num_pages", 0, "MLA_ERR_BAD_DIMS")])
def test_append_rejects_bad_dims(field, value, status):
    d = _append_dims()
    setattr(d, field, value)
    p = [_al(k + 1) for k in range(6)]
    assert M.lib().mla_cache_append(ctypes.byref(d), *p, _al(7), 1 << 30,
                                    ctypes.c_void_p(0)) == STATUS_CODE[status]
    assert M.lib().mla_cache_append_workspace_bytes(ctypes.byref(d)) == 0


def test_append_rejects_null_and_misaligned():
    L = M.lib()
    assert L.mla_cache_append(None, *[_al(k + 1) for k in range(6)], _al(7), 1 << 30, None) == \
        STATUS_CODE["MLA_ERR_NULL_ARG"]
    for i in range(6):
        p = [_al(k + 1) for k in range(6)]
        p[i] = ctypes.c_void_p(0)
        assert L.mla_cache_append(ctypes.byref(_append_dims()), *p, _al(7), 1 << 30, None) == \
            STATUS_CODE["MLA_ERR_NULL_ARG"], i
        p[i] = ctypes.c_void_p(0x100008)
        assert L.mla_cache_append(ctypes.byref(_append_dims()), *p, _al(7), 1 << 30, None) == \
            STATUS_CODE["MLA_ERR_MISALIGNED"], i
    p = [_al(k + 1) for k in range(6)]
    assert L.mla_cache_append_fp8(ctypes.byref(_append_dims()), *p, None, _al(7), 1 << 30,
                                  None) == STATUS_CODE["MLA_ERR_NULL_ARG"]
    assert L.mla_cache_append_fp8(ctypes.byref(_append_dims()), *p, ctypes.c_void_p(0x100004),
                                  _al(7), 1 << 30, None) == STATUS_CODE["MLA_ERR_MISALIGNED"]


def test_append_workspace():
    # fp32 partial rows, one set per slice of the model width: as many slices (a divisor of
    # hidden / 256) as keep the partial grid within 1024 work groups and within what the
    # finishing work group sums (min(8, 1024 / (N / 4)) threads per column quad, 8 slices each)
    L = M.lib()
    d = _append_dims(B=16)  # 18 column blocks x 1 token block: 28 slices of 256
    need = L.mla_cache_append_workspace_bytes(ctypes.byref(d))
    assert need == 28 * 16 * 576 * 4
    d = _append_dims(B=64, T=16)  # 18 x 16 blocks of 64 token rows: 2 slices
    assert L.mla_cache_append_workspace_bytes(ctypes.byref(d)) == 2 * 1024 * 576 * 4
    d = _append_dims(B=96)  # 18 x 3 blocks of 32 token rows: 14 slices
    assert L.mla_cache_append_workspace_bytes(ctypes.byref(d)) == 14 * 96 * 576 * 4
    d = _append_dims(B=32, hidden=4096, d_c=64, d_R=8)  # 3 x 2 blocks: all 16 slices
    assert L.mla_cache_append_workspace_bytes(ctypes.byref(d)) == 16 * 32 * 72 * 4
    # N = 1536: 2 threads per quad, so at most 16 slices (the grid would allow 20 of 5120 / 256)
    d = _append_dims(B=16, hidden=5120, d_c=1024, d_R=512)
    assert L.mla_cache_append_workspace_bytes(ctypes.byref(d)) == 10 * 16 * 1536 * 4
    d = _append_dims(B=16)
    p = [_al(k + 1) for k in range(6)]
    assert L.mla_cache_append(ctypes.byref(d), *p, _al(7), need - 4, None) == \
        STATUS_CODE["MLA_ERR_WORKSPACE"]
    assert L.mla_cache_append(ctypes.byref(d), *p, ctypes.c_void_p(0), need, None) == \
        STATUS_CODE["MLA_ERR_WORKSPACE"]
    assert L.mla_cache_append(ctypes.byref(d), *p, ctypes.c_void_p(0x100010), need, None) == \
        STATUS_CODE["MLA_ERR_MISALIGNED"]


def test_status_strings():
    for code in range(8):
        assert M.lib().mla_status_str(code)
    assert M.lib().mla_last_hip_error() is not None


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 128, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        M.decode(x, x, x, x, x, torch.zeros(1, 1, dtype=torch.int32),
                 torch.ones(1, dtype=torch.int32))


def test_decode_fp8_rejects_before_enqueueing():
    L = M.lib()
    ptrs = [_al(k + 1) for k in range(5)]           # q_nope, q_rope, W_UK, W_UV, kv_pages
    rest = [_al(7), _al(8), _al(9), ctypes.c_void_p(0)]  # page_table, seq_lens, out, lse
    def call(d, scales):
        return L.mla_decode_fp8(ctypes.byref(d), *ptrs, scales, *rest, _al(10),
                                M.workspace_bytes(d), ctypes.c_void_p(0), None)
    for dims in (m2_dims, ds_dims):  # the FP8 cache at both widths
        assert call(dims(), ctypes.c_void_p(0)) == STATUS_CODE["MLA_ERR_NULL_ARG"]
        assert call(dims(), ctypes.c_void_p(_al(6).value + 4)) == \
            STATUS_CODE["MLA_ERR_MISALIGNED"]
    bad = m2_dims()
    bad.batch = 0
    assert call(bad, _al(6)) == STATUS_CODE["MLA_ERR_BAD_DIMS"]


def test_decode_mxfp4_rejects_before_enqueueing():
    L = M.lib()
    ptrs = [_al(k + 1) for k in range(5)]           # q_nope, q_rope, W_UK, W_UV, kv_pages
    rest = [_al(7), _al(8), _al(9), ctypes.c_void_p(0)]  # page_table, seq_lens, out, lse
    def call(d, scales):
        return L.mla_decode_mxfp4(ctypes.byref(d), *ptrs, scales, *rest, _al(10),
                                  M.workspace_bytes(d), ctypes.c_void_p(0), None)
    assert call(m2_dims(), ctypes.c_void_p(0)) == STATUS_CODE["MLA_ERR_NULL_ARG"]
    assert call(m2_dims(), ctypes.c_void_p(_al(6).value + 4)) == STATUS_CODE["MLA_ERR_MISALIGNED"]
    # the MXFP4 cache is read at the MHA2MLA widths only
    assert call(ds_dims(), _al(6)) == STATUS_CODE["MLA_ERR_UNSUPPORTED"]
    # the decompressed branch reads a bf16 cache
    d = m2_dims(B=2, max_pages=16, num_pages=64, max_seq_len=1024)
    d.q_len, d.prefill_threshold = 300, 256
    assert call(d, _al(6)) == STATUS_CODE["MLA_ERR_UNSUPPORTED"]
    bad = m2_dims()
    bad.batch = 0
    assert call(bad, _al(6)) == STATUS_CODE["MLA_ERR_BAD_DIMS"]
    # the workspace is the one mla_decode_workspace_bytes gives (as for FP8)
    d = m2_dims()
    assert L.mla_decode_mxfp4(ctypes.byref(d), *ptrs, _al(6), *rest, _al(10),
                              M.workspace_bytes(d) - 1, ctypes.c_void_p(0), None) == \
        STATUS_CODE["MLA_ERR_WORKSPACE"]


def test_append_mxfp4_rejects_before_enqueueing():
    L = M.lib()
    p = [_al(k + 1) for k in range(6)]
    assert L.mla_cache_append_mxfp4(ctypes.byref(_append_dims()), *p, None, _al(7), 1 << 30,
                                    None) == STATUS_CODE["MLA_ERR_NULL_ARG"]
    assert L.mla_cache_append_mxfp4(ctypes.byref(_append_dims()), *p, ctypes.c_void_p(0x100004),
                                    _al(7), 1 << 30, None) == STATUS_CODE["MLA_ERR_MISALIGNED"]
    # whole blocks of 32 latent elements only
    assert L.mla_cache_append_mxfp4(ctypes.byref(_append_dims(d_c=500)), *p, _al(8), _al(7),
                                    1 << 30, None) == STATUS_CODE["MLA_ERR_UNSUPPORTED"]


def _small_decode_args(B=2, T=None, H=32, d_n=120, d_c=64, d_R=8, d_v=128, P=4, mp=2):
    import torch
    bf = torch.bfloat16
    lead = (B,) if T is None else (B, T)
    return dict(q_nope=torch.zeros(lead + (H, d_n), dtype=bf),
                q_rope=torch.zeros(lead + (H, d_R), dtype=bf),
                W_UK=torch.zeros(H, d_n, d_c, dtype=bf), W_UV=torch.zeros(H, d_c, d_v, dtype=bf),
                kv_pages=torch.zeros(P, 64, d_c + d_R, dtype=bf),
                page_table=torch.zeros(B, mp, dtype=torch.int32),
                seq_lens=torch.ones(B, dtype=torch.int32))


@pytest.mark.parametrize("name,bad", [
    ("W_UK", (16, 120, 64)), ("W_UK", (32, 128, 64)), ("W_UV", (32, 32, 128)),
    ("kv_pages", (4, 64, 64)), ("page_table", (1, 2)), ("seq_lens", (3,)),
    ("q_rope", (2, 16, 8)), ("out", (2, 32, 64)), ("lse", (1, 32))])
def test_binding_rejects_inconsistent_sizes(name, bad):
    # the C ABI sees only pointers, so the binding is the one place where sizes are checked
    # against each other: every mismatch raises before anything reaches the library (the
    # tensors live on the CPU, so a call that got past the checks would fail differently)
    import torch
    a = _small_decode_args()
    kw = {}
    if name in ("out", "lse"):
        kw[name] = torch.zeros(bad, dtype=torch.bfloat16 if name == "out" else torch.float32)
    else:
        a[name] = torch.zeros(bad, dtype=a[name].dtype)
    with pytest.raises(ValueError, match="shape"):
        M.decode(*a.values(), **kw)


def test_binding_rejects_inconsistent_sizes_other_calls():
    import torch
    bf = torch.bfloat16
    a = _small_decode_args()
    W_UVO = torch.zeros(256, 32 * 64, dtype=bf)
    args = [a["q_nope"], a["q_rope"], a["W_UK"], W_UVO, a["kv_pages"], a["page_table"]]
    with pytest.raises(ValueError, match="shape"):   # out of the wrong width
        M.decode_out(*args, a["seq_lens"], out=torch.zeros(2, 128, dtype=bf))
    with pytest.raises(ValueError, match="shape"):   # one length too few
        M.decode_out(*args, a["seq_lens"][:1])
    with pytest.raises(ValueError):                  # W_UVO not [hidden, H*d_c]
        M.decode_out(a["q_nope"], a["q_rope"], a["W_UK"], torch.zeros(256, 100, dtype=bf),
                     a["kv_pages"], a["page_table"], a["seq_lens"])
    x = torch.zeros(2, 1, 1024, dtype=bf)
    Wd, Wr = torch.zeros(64, 1024, dtype=bf), torch.zeros(8, 1024, dtype=bf)
    with pytest.raises(ValueError, match="shape"):   # seq_lens of another batch
        M.cache_append(x, Wd, Wr, a["kv_pages"], a["page_table"], a["seq_lens"][:1])
    with pytest.raises(ValueError, match="shape"):   # W_KR of another hidden width
        M.cache_append(x, Wd, torch.zeros(8, 512, dtype=bf), a["kv_pages"], a["page_table"],
                       a["seq_lens"])
    with pytest.raises(ValueError, match="shape"):
        M.gather_pages(a["kv_pages"], a["page_table"], a["seq_lens"][:1], 64)
