"""ctypes binding of libmla_decode.so (argument marshalling only).

Every step of the decode runs in the library's HIP kernels; this module checks tensor
dtypes/shapes/devices, allocates outputs and workspace with torch, and passes raw device
pointers plus the current HIP stream. If the library is missing the calls raise.
"""
import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mla_decode.h")

STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL_ARG", 2: "MLA_ERR_BAD_DIMS", 3: "MLA_ERR_MISALIGNED",
          4: "MLA_ERR_WORKSPACE", 5: "MLA_ERR_UNSUPPORTED", 6: "MLA_ERR_HIP",
          7: "MLA_ERR_DEVICE_CHECK"}
STATUS_CODE = {v: k for k, v in STATUS.items()}
# size of the scratch array built into the library for mla_decode_noalloc (the header's
# MLA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 48 << 20


class Dims(ctypes.Structure):
    """Mirror of mla_dims_t."""
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("num_units", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("prefill_threshold", ctypes.c_int32)]


class AppendDims(ctypes.Structure):
    """Mirror of mla_append_dims_t."""
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("rope_base", ctypes.c_float)]


class MlaError(RuntimeError):
    def __init__(self, code, text):
        super().__init__("%s: %s" % (STATUS.get(code, code), text))
        self.code = code


_LIB = None


def lib():
    """The loaded library (loads it on first use; raises if it was not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmla_decode.so is not built (run __graft_entry__.build() or "
                              "python -m mla_latent_kv_14_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, c_int, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        dp = ctypes.POINTER(Dims)
        L.mla_decode_workspace_bytes.restype = sz
        L.mla_decode_workspace_bytes.argtypes = [dp]
        L.mla_decode.restype = c_int
        L.mla_decode.argtypes = [dp] + [vp] * 10 + [sz, vp]
        L.mla_decode_noalloc.restype = c_int
        L.mla_decode_noalloc.argtypes = [dp] + [vp] * 9 + [vp]
        L.mla_decode_timed.restype = c_int
        L.mla_decode_timed.argtypes = [dp] + [vp] * 10 + [sz, vp, ctypes.POINTER(vp)]
        L.mla_decode_fp8.restype = c_int
        L.mla_decode_fp8.argtypes = [dp] + [vp] * 11 + [sz, vp, ctypes.POINTER(vp)]
        L.mla_decode_mxfp4.restype = c_int
        L.mla_decode_mxfp4.argtypes = [dp] + [vp] * 11 + [sz, vp, ctypes.POINTER(vp)]
        L.mla_decode_out.restype = c_int
        L.mla_decode_out.argtypes = [dp, ctypes.c_int32] + [vp] * 10 + [sz, vp]
        L.mla_cache_append.restype = c_int
        L.mla_cache_append.argtypes = [ctypes.POINTER(AppendDims)] + [vp] * 7 + [sz, vp]
        L.mla_cache_append_fp8.restype = c_int
        L.mla_cache_append_fp8.argtypes = [ctypes.POINTER(AppendDims)] + [vp] * 8 + [sz, vp]
        L.mla_cache_append_mxfp4.restype = c_int
        L.mla_cache_append_mxfp4.argtypes = [ctypes.POINTER(AppendDims)] + [vp] * 8 + [sz, vp]
        L.mla_cache_append_workspace_bytes.restype = sz
        L.mla_cache_append_workspace_bytes.argtypes = [ctypes.POINTER(AppendDims)]
        L.mla_gather_pages.restype = c_int
        L.mla_gather_pages.argtypes = [dp, vp, vp, vp, vp, vp]
        L.mla_status_str.restype = ctypes.c_char_p
        L.mla_status_str.argtypes = [c_int]
        L.mla_last_hip_error.restype = ctypes.c_char_p
        L.mla_last_hip_error.argtypes = []
        _LIB = L
    return _LIB


def header_symbols():
    """Names of the functions include/mla_decode.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def _check(code):
    if code != 0:
        L = lib()
        text = L.mla_status_str(code).decode()
        if code == STATUS_CODE["MLA_ERR_HIP"]:
            text += " (" + L.mla_last_hip_error().decode() + ")"
        raise MlaError(code, text)


def make_dims(q_nope, q_rope, W_UK, W_UV, kv_pages, page_table, max_seq_len=None,
              softmax_scale=None, num_units=0, prefill_threshold=0):
    """Dims of a call; q_nope [B, H, d_n] (one query token per sequence) or [B, T, H, d_n]
    (T query tokens per sequence; from prefill_threshold on, 0 = 256, the decompressed
    branch)."""
    if q_nope.dim() == 4:
        B, T, H, d_n = q_nope.shape
    else:
        (B, H, d_n), T = q_nope.shape, 1
    d = Dims()
    d.batch, d.num_heads, d.d_nope = B, H, d_n
    d.q_len = T
    d.d_latent = W_UK.shape[2]
    d.d_rope = q_rope.shape[-1]
    d.d_v = W_UV.shape[2]
    d.page_size = kv_pages.shape[1]
    d.max_pages_per_seq = page_table.shape[1]
    d.num_pages = kv_pages.shape[0]
    d.max_seq_len = int(max_seq_len) if max_seq_len else 0
    d.softmax_scale = float(softmax_scale) if softmax_scale else 0.0
    d.num_units = int(num_units)
    d.prefill_threshold = int(prefill_threshold)
    return d


def workspace_bytes(dims):
    return int(lib().mla_decode_workspace_bytes(ctypes.byref(dims)))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _shape(t, name, want):
    """Raise ValueError unless tensor t has exactly the shape `want` (a tuple of ints)."""
    if tuple(t.shape) != tuple(want):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(want)))


def _want(t, name, dtype, ndim, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def decode(q_nope, q_rope, W_UK, W_UV, kv_pages, page_table, seq_lens, out=None, lse=None,
           max_seq_len=None, softmax_scale=None, num_units=0, workspace=None, stream=None,
           return_lse=False, kernel_events=None, kv_scales=None, no_alloc=False,
           prefill_threshold=0):
    """Absorbed MLA decode through mla_decode(). Tensors live on one HIP device.

    q_nope bf16 [B,H,d_n], q_rope bf16 [B,H,d_R], W_UK bf16 [H,d_n,d_c], W_UV bf16 [H,d_c,d_v],
    kv_pages bf16 [P,64,d_c+d_R], page_table int32 [B,max_pages], seq_lens int32 [B].
    Returns out bf16 [B,H,d_v] (and lse fp32 [B,H] when return_lse).
    Several query tokens per sequence: q_nope [B,T,H,d_n] and q_rope [B,T,H,d_R] give out
    [B,T,H,d_v] and lse [B,T,H]; query token i of sequence b attends to its first
    seq_lens[b] - T + 1 + i cached tokens.
    kernel_events: optional six raw hipEvent_t handles (int or None), passed to
    mla_decode_timed, which binds them to the start and end of the absorb, attention and
    combine kernels.
    kv_scales: a quantised cache. fp32 [P,64]: an FP8 cache (mla_decode_fp8), kv_pages uint8
    [P,64,d_c+2*d_R], token = [c_KV as FP8 e4m3 bytes | k_R bf16], one scale per token.
    uint8 [P,64,d_c/32]: an MXFP4 cache (mla_decode_mxfp4, MHA2MLA widths), kv_pages uint8
    [P,64,d_c/2+2*d_R], token = [c_KV as E2M1 codes, two per byte | k_R bf16], an E8M0 scale
    byte per block of 32 latent elements.
    no_alloc: run mla_decode_noalloc, whose scratch is built into the library (no workspace;
    pass out, and lse when return_lse, so that nothing is allocated here either).
    prefill_threshold: query tokens per sequence from which the decompressed branch serves
    the call (0 = 256).
    """
    bf, i32 = torch.bfloat16, torch.int32
    nq = q_nope.dim() if isinstance(q_nope, torch.Tensor) else 3
    if nq not in (3, 4):
        raise ValueError("q_nope must be [B,H,d_n] or [B,T,H,d_n]")
    if no_alloc and (workspace is not None or kernel_events is not None or
                     kv_scales is not None):
        raise ValueError("no_alloc takes no workspace, kernel_events or kv_scales")
    dev = q_nope.device
    # dtype, rank and layout of every tensor, then the sizes they must agree on (the library
    # only sees pointers: a short tensor here would be read or written past its end on the
    # device), then the device
    for t, n, dt, nd in ((q_nope, "q_nope", bf, nq), (q_rope, "q_rope", bf, nq),
                         (W_UK, "W_UK", bf, 3), (W_UV, "W_UV", bf, 3),
                         (kv_pages, "kv_pages", bf if kv_scales is None else torch.uint8, 3),
                         (page_table, "page_table", i32, 2),
                         (seq_lens, "seq_lens", i32, 1)):
        _want(t, n, dt, nd, t.device)
    dims = make_dims(q_nope, q_rope, W_UK, W_UV, kv_pages, page_table, max_seq_len,
                     softmax_scale, num_units, prefill_threshold)
    mx = kv_scales is not None and kv_scales.dtype == torch.uint8
    B, H, d_v = dims.batch, dims.num_heads, dims.d_v
    d_n, d_c, d_R = dims.d_nope, dims.d_latent, dims.d_rope
    lead = (B,) if nq == 3 else (B, dims.q_len)
    _shape(q_rope, "q_rope", lead + (H, d_R))
    _shape(W_UK, "W_UK", (H, d_n, d_c))
    _shape(W_UV, "W_UV", (H, d_c, d_v))
    row = d_c + d_R if kv_scales is None else (d_c // 2 + 2 * d_R if mx else d_c + 2 * d_R)
    _shape(kv_pages, "kv_pages", (kv_pages.shape[0], kv_pages.shape[1], row))
    _shape(page_table, "page_table", (B, page_table.shape[1]))
    _shape(seq_lens, "seq_lens", (B,))
    if out is not None:
        _want(out, "out", bf, nq, out.device)
        _shape(out, "out", lead + (H, d_v))
    if lse is not None:
        _want(lse, "lse", torch.float32, nq - 1, lse.device)
        _shape(lse, "lse", lead + (H,))
    if mx:
        _want(kv_scales, "kv_scales", torch.uint8, 3, kv_scales.device)
        _shape(kv_scales, "kv_scales", tuple(kv_pages.shape[:2]) + (d_c // 32,))
    elif kv_scales is not None:
        _want(kv_scales, "kv_scales", torch.float32, 2, kv_scales.device)
        _shape(kv_scales, "kv_scales", tuple(kv_pages.shape[:2]))
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or
                                  not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor")
    if dev.type != "cuda":
        raise ValueError("mla decode runs on a HIP device; got %s" % dev)
    for t, n in ((q_rope, "q_rope"), (W_UK, "W_UK"), (W_UV, "W_UV"), (kv_pages, "kv_pages"),
                 (page_table, "page_table"), (seq_lens, "seq_lens"), (out, "out"), (lse, "lse"),
                 (kv_scales, "kv_scales"), (workspace, "workspace")):
        if t is not None and t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (n, t.device, dev))
    if out is None:
        out = torch.empty(lead + (H, d_v), dtype=bf, device=dev)
    if return_lse and lse is None:
        lse = torch.empty(lead + (H,), dtype=torch.float32, device=dev)
    if no_alloc:
        _check(lib().mla_decode_noalloc(
            ctypes.byref(dims), _ptr(q_nope), _ptr(q_rope), _ptr(W_UK), _ptr(W_UV),
            _ptr(kv_pages), _ptr(page_table), _ptr(seq_lens), _ptr(out), _ptr(lse),
            _stream(stream, dev)))
        return (out, lse) if return_lse else out
    nbytes = workspace_bytes(dims)
    if nbytes == 0:
        _check(lib().mla_decode(ctypes.byref(dims), *([ctypes.c_void_p(0)] * 10), 0,
                                ctypes.c_void_p(0)))
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    args = (ctypes.byref(dims), _ptr(q_nope), _ptr(q_rope), _ptr(W_UK), _ptr(W_UV),
            _ptr(kv_pages), _ptr(page_table), _ptr(seq_lens), _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, dev))
    ev = None
    if kernel_events is not None:
        if len(kernel_events) != 6:
            raise ValueError("kernel_events needs six entries (start, end of three kernels)")
        ev = (ctypes.c_void_p * 6)(*[e or None for e in kernel_events])
    if mx:
        code = lib().mla_decode_mxfp4(*args[:6], _ptr(kv_scales), *args[6:], ev)
    elif kv_scales is not None:
        code = lib().mla_decode_fp8(*args[:6], _ptr(kv_scales), *args[6:], ev)
    elif ev is None:
        code = lib().mla_decode(*args)
    else:
        code = lib().mla_decode_timed(*args, ev)
    _check(code)
    return (out, lse) if return_lse else out


def decode_out(q_nope, q_rope, W_UK, W_UVO, kv_pages, page_table, seq_lens, out=None,
               lse=None, max_seq_len=None, softmax_scale=None, num_units=0, workspace=None,
               stream=None, return_lse=False):
    """The decode with the merged output projection (mla_decode_out): W_UVO bf16
    [hidden, H*d_c] replaces W_UV; returns out bf16 [B, hidden] ([B, T, hidden] for 4-d
    queries), and lse fp32 [B, H] ([B, T, H]) when return_lse."""
    bf, i32 = torch.bfloat16, torch.int32
    nq = q_nope.dim() if isinstance(q_nope, torch.Tensor) else 3
    if nq not in (3, 4):
        raise ValueError("q_nope must be [B,H,d_n] or [B,T,H,d_n]")
    dev = q_nope.device
    for t, n, dt, nd in ((q_nope, "q_nope", bf, nq), (q_rope, "q_rope", bf, nq),
                         (W_UK, "W_UK", bf, 3), (W_UVO, "W_UVO", bf, 2),
                         (kv_pages, "kv_pages", bf, 3), (page_table, "page_table", i32, 2),
                         (seq_lens, "seq_lens", i32, 1)):
        _want(t, n, dt, nd, t.device)
    H, d_n, d_c = W_UK.shape
    hidden = W_UVO.shape[0]
    if W_UVO.shape[1] != H * d_c:
        raise ValueError("W_UVO must be [hidden, H*d_c] = [*, %d]" % (H * d_c))
    # d_v does not enter this call; the dims carry the width of the supported shapes
    dims = make_dims(q_nope, q_rope, W_UK, torch.empty((H, d_c, 128), dtype=bf, device="meta"),
                     kv_pages, page_table, max_seq_len, softmax_scale, num_units)
    B, d_R = dims.batch, dims.d_rope
    lead = (B,) if nq == 3 else (B, dims.q_len)
    _shape(q_nope, "q_nope", lead + (H, d_n))
    _shape(q_rope, "q_rope", lead + (H, d_R))
    _shape(kv_pages, "kv_pages", (kv_pages.shape[0], kv_pages.shape[1], d_c + d_R))
    _shape(page_table, "page_table", (B, page_table.shape[1]))
    _shape(seq_lens, "seq_lens", (B,))
    if out is not None:
        _want(out, "out", bf, nq - 1, out.device)
        _shape(out, "out", lead + (hidden,))
    if lse is not None:
        _want(lse, "lse", torch.float32, nq - 1, lse.device)
        _shape(lse, "lse", lead + (H,))
    if dev.type != "cuda":
        raise ValueError("mla decode runs on a HIP device; got %s" % dev)
    for t, n in ((q_rope, "q_rope"), (W_UK, "W_UK"), (W_UVO, "W_UVO"), (kv_pages, "kv_pages"),
                 (page_table, "page_table"), (seq_lens, "seq_lens"), (out, "out"), (lse, "lse"),
                 (workspace, "workspace")):
        if t is not None and t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (n, t.device, dev))
    if out is None:
        out = torch.empty(lead + (hidden,), dtype=bf, device=dev)
    if return_lse and lse is None:
        lse = torch.empty(lead + (H,), dtype=torch.float32, device=dev)
    nbytes = workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().mla_decode_out(ctypes.byref(dims), hidden, _ptr(q_nope), _ptr(q_rope),
                                _ptr(W_UK), _ptr(W_UVO), _ptr(kv_pages), _ptr(page_table),
                                _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(),
                                _stream(stream, dev)))
    return (out, lse) if return_lse else out


def append_workspace_bytes(d):
    return int(lib().mla_cache_append_workspace_bytes(ctypes.byref(d)))


def cache_append(x, W_DKV, W_KR, kv_pages, page_table, seq_lens, rope_base=10000.0,
                 stream=None, kv_scales=None, workspace=None):
    """Writes [c_KV | RoPE(k_R)] of the new tokens into kv_pages in place (mla_cache_append).

    x bf16 [B,T,hidden] (or [B,hidden] for one token), W_DKV bf16 [d_c,hidden], W_KR bf16
    [d_R,hidden], kv_pages bf16 [P,64,d_c+d_R], page_table int32 [B,max_pages], seq_lens int32
    [B] (tokens already cached; token i of sequence b goes to position seq_lens[b] + i).
    kv_scales: a quantised cache, written at the new tokens' slots with kv_pages. fp32 [P,64]:
    an FP8 cache (mla_cache_append_fp8), kv_pages uint8 [P,64,d_c+2*d_R]. uint8
    [P,64,d_c/32]: an MXFP4 cache (mla_cache_append_mxfp4), kv_pages uint8 [P,64,d_c/2+2*d_R].
    workspace: a uint8 tensor of at least mla_cache_append_workspace_bytes (allocated here
    when None).
    """
    bf = torch.bfloat16
    dev = kv_pages.device
    _want(x, "x", bf, x.dim() if x.dim() in (2, 3) else 3, x.device)
    _want(W_DKV, "W_DKV", bf, 2, W_DKV.device)
    _want(W_KR, "W_KR", bf, 2, W_KR.device)
    _want(kv_pages, "kv_pages", bf if kv_scales is None else torch.uint8, 3, dev)
    _want(page_table, "page_table", torch.int32, 2, page_table.device)
    _want(seq_lens, "seq_lens", torch.int32, 1, seq_lens.device)
    d = AppendDims()
    d.batch = x.shape[0]
    d.q_len = x.shape[1] if x.dim() == 3 else 1
    d.hidden = x.shape[-1]
    d.d_latent, d.d_rope = W_DKV.shape[0], W_KR.shape[0]
    _shape(W_DKV, "W_DKV", (d.d_latent, d.hidden))
    _shape(W_KR, "W_KR", (d.d_rope, d.hidden))
    mx = kv_scales is not None and kv_scales.dtype == torch.uint8
    row = (d.d_latent + d.d_rope if kv_scales is None else
           d.d_latent // 2 + 2 * d.d_rope if mx else d.d_latent + 2 * d.d_rope)
    _shape(kv_pages, "kv_pages", (kv_pages.shape[0], kv_pages.shape[1], row))
    _shape(page_table, "page_table", (d.batch, page_table.shape[1]))
    _shape(seq_lens, "seq_lens", (d.batch,))
    if mx:
        _want(kv_scales, "kv_scales", torch.uint8, 3, kv_scales.device)
        _shape(kv_scales, "kv_scales", tuple(kv_pages.shape[:2]) + (d.d_latent // 32,))
    elif kv_scales is not None:
        _want(kv_scales, "kv_scales", torch.float32, 2, kv_scales.device)
        _shape(kv_scales, "kv_scales", tuple(kv_pages.shape[:2]))
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or
                                  not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor")
    if dev.type != "cuda":
        raise ValueError("the cache append runs on a HIP device; got %s" % dev)
    for t, n in ((x, "x"), (W_DKV, "W_DKV"), (W_KR, "W_KR"), (page_table, "page_table"),
                 (seq_lens, "seq_lens"), (kv_scales, "kv_scales"), (workspace, "workspace")):
        if t is not None and t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (n, t.device, dev))
    d.page_size = kv_pages.shape[1]
    d.max_pages_per_seq = page_table.shape[1]
    d.num_pages = kv_pages.shape[0]
    d.rope_base = float(rope_base)
    if workspace is None:
        workspace = torch.empty(max(append_workspace_bytes(d), 1), dtype=torch.uint8, device=dev)
    args = (ctypes.byref(d), _ptr(x), _ptr(W_DKV), _ptr(W_KR), _ptr(page_table),
            _ptr(seq_lens), _ptr(kv_pages))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, dev))
    if kv_scales is None:
        _check(lib().mla_cache_append(*args, *tail))
    elif mx:
        _check(lib().mla_cache_append_mxfp4(*args, _ptr(kv_scales), *tail))
    else:
        _check(lib().mla_cache_append_fp8(*args, _ptr(kv_scales), *tail))
    return kv_pages


def gather_pages(kv_pages, page_table, seq_lens, d_latent, max_seq_len=None, stream=None):
    """Logical copy of the paged cache through the attention kernels' loader (mla_gather_pages).
    Returns bf16 [B, S_max, d_latent + d_rope], zero past each S_b."""
    dev = kv_pages.device
    _want(kv_pages, "kv_pages", torch.bfloat16, 3, dev)
    _want(page_table, "page_table", torch.int32, 2, dev)
    _want(seq_lens, "seq_lens", torch.int32, 1, dev)
    _shape(seq_lens, "seq_lens", (page_table.shape[0],))
    if not 0 < int(d_latent) < kv_pages.shape[2]:
        raise ValueError("d_latent must lie inside the token row (%d)" % kv_pages.shape[2])
    d = Dims()
    d.batch = page_table.shape[0]
    d.d_latent = int(d_latent)
    d.d_rope = kv_pages.shape[2] - int(d_latent)
    d.page_size = kv_pages.shape[1]
    d.max_pages_per_seq = page_table.shape[1]
    d.num_pages = kv_pages.shape[0]
    d.max_seq_len = int(max_seq_len) if max_seq_len else 0
    S_max = d.max_seq_len or d.max_pages_per_seq * d.page_size
    dst = torch.empty((d.batch, S_max, kv_pages.shape[2]), dtype=torch.bfloat16, device=dev)
    _check(lib().mla_gather_pages(ctypes.byref(d), _ptr(kv_pages), _ptr(page_table),
                                  _ptr(seq_lens), _ptr(dst), _stream(stream, dev)))
    return dst
