#!/usr/bin/env python3
"""Benchmark: absorbed MLA decode over a paged latent cache on one MI355X.

A step is one full mla_decode call (absorb -> paged split-KV attention -> combine + W_UV) over
one batch of synthetic inputs already resident in HBM. The default workload is DeepSeek widths
(128 heads, 512-d latent + 64-d RoPE, d_nope 128, d_v 128), B = 16 sequences of 4096 tokens in
64-token pages under a shuffled page table. Distinct input sets (each a full set of queries,
weights and cache) are rotated so that the working set of consecutive steps exceeds the
256 MiB Infinity Cache: the timed steps read from HBM ("cold"). A single-set run is reported
as "warm" next to it.

Timing starts after W untimed calls (default 2000, about 0.1 s of back-to-back calls): the GPU
needs that long to reach its steady clocks, and after a 20-call warm-up the same workload timed
about 13 % slower.

Prints one JSON line (the contract): metric/value (KV tokens per second, from K plain calls),
TFLOP/s, GB/s, the roofline object of the dominant kernel (paged attention; its duration comes
from HIP events bound to that kernel's own start and end in a second pass of K calls)
and the fp64 CPU oracle's throughput on the host cores (a reported baseline).

Algorithmic work of one call (what the method must move or compute; partials and the
decompression it avoids excluded):
  F = 2 B H d_n d_c + 2 H (d_c + d_R) sumS + 2 H d_c sumS + 2 B H d_c d_v
  Bytes = sumS (d_c + d_R) 2 + 2 H d_c (d_n + d_v) + 2 B H (d_n + d_R) + 2 B H d_v
          + 4 (B max_pages + B)
Attention kernel alone (the roofline object): the cache bytes, sumS (d_c + d_R) 2 (1152 B per
token; 644 B over the FP8 cache; at the MHA2MLA widths 144, 84 over FP8 and 50 over MXFP4), the
per-token figure times the tokens. The absorbed queries
it reads (an intermediate the method makes, not an input) are not counted. With several query
tokens the attention kernel's FLOPs per cache byte pass the MFMA ridge (about 315 FLOP/B, from
T = 2 on at the DeepSeek widths), and it is priced on MFMA. On the decompressed branch (from
the prefill threshold on) the object covers that branch's span, priced on its own arithmetic,
2 S H (d_n + d_v) d_c for the decompression plus 2 H (d_n + d_R + d_v) per (query, token) pair;
the top-level TFLOP/s keeps counting the absorbed form's work. The committed counter records
(traffic, MFMA busy share) were taken on the one-token decode and attach to it only.
"""
import argparse
import ctypes
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode KV-tokens/s + TFLOP/s at B=16 S=4096; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # about 315
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic.json")
ATTN_SOURCES = ["attn.hip", "paged_tile.h", "device.h"]


def algorithmic(inp, T=1, row_bytes=None):
    """Algorithmic work of one call with T query tokens per sequence (query token i of
    sequence b attends to S_b - T + 1 + i tokens; the cache is read once). row_bytes: cache
    bytes per token (default the bf16 row, (d_c + d_R) * 2)."""
    B, H = inp["B"], inp["H"]
    d_n, d_c, d_R, d_v = inp["d_n"], inp["d_c"], inp["d_R"], inp["d_v"]
    lens = [int(x) for x in inp["seq_lens"]]
    S = sum(lens)                                                    # cached tokens
    A = sum(max(0, s - T + 1 + i) for s in lens for i in range(T))  # (query, token) pairs
    Q = B * T                                                        # query tokens
    mp = inp["max_pages"]
    rb = (d_c + d_R) * 2 if row_bytes is None else row_bytes
    flops = 2 * Q * H * d_n * d_c + 2 * H * (d_c + d_R) * A + 2 * H * d_c * A + 2 * Q * H * d_c * d_v
    nbytes = (S * rb + 2 * H * d_c * (d_n + d_v) + 2 * Q * H * (d_n + d_R)
              + 2 * Q * H * d_v + 4 * (B * mp + B))
    attn_bytes = S * rb
    attn_flops = 2 * H * (d_c + d_R) * A + 2 * H * d_c * A
    # the decompressed branch's own arithmetic: K_nope and V of every cached token and head,
    # then attention at the head widths (scores over d_n + d_R, values over d_v)
    decomp_flops = 2 * S * H * (d_n + d_v) * d_c + 2 * H * (d_n + d_R + d_v) * A
    return dict(sumS=A, flops=flops, bytes=nbytes, attn_bytes=attn_bytes, attn_flops=attn_flops,
                decomp_flops=decomp_flops)


class Hip:
    """HIP runtime events via ctypes (timing on the stream the library launches on)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.L.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def ms(self, a, b):
        t = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def stage_us(stage_ms, decompressed):
    """Per-kernel durations (µs) from the stage events. The decompressed branch runs no absorb
    or combine kernel (its first and last event pairs mark single points), so it reports the
    branch as one stage."""
    if decompressed:
        return {"decompressed_branch": round(stage_ms[1] * 1e3, 2)}
    return {"absorb": round(stage_ms[0] * 1e3, 2), "attention": round(stage_ms[1] * 1e3, 2),
            "combine": round(stage_ms[2] * 1e3, 2)}


def source_digest():
    """Digest of the attention kernel's sources with comments and blank space removed, so that
    only a change to the code itself retires a stored traffic measurement."""
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "mla_latent_kv_14_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_mfma_util(workload_name):
    """Share of the attention kernel's time its matrix cores were busy (rocprofv3 SQ counters,
    from the same committed record), or None as for the traffic."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload_name)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("mfma_busy_share")


def measured_traffic(workload_name):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, or None
    if there is none for this workload or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload_name)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def run(args):
    import torch
    import mla_latent_kv_14_amd as M
    import workloads as W

    lib = M.lib()
    cfg = W.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = args.q_len

    def with_tokens(inp, seed):  # T query tokens per sequence, seeded like the rest
        if T > 1:
            g = torch.Generator().manual_seed(seed)
            B, H = inp["B"], inp["H"]
            inp["q_nope"] = torch.randn(B, T, H, inp["d_n"], generator=g).to(torch.bfloat16)
            inp["q_rope"] = torch.randn(B, T, H, inp["d_R"], generator=g).to(torch.bfloat16)
        return inp

    def with_fp8(inp, seed):  # a quantised cache: the FP8 copy, or a synthetic MXFP4 one
        if args.kv_fp8:
            kv8, sc = W.fp8_cache(inp, seed=seed)
            inp["kv_pages"], inp["kv_scales"] = kv8, sc
        elif args.kv_mxfp4:
            kv4, sc = W.mxfp4_cache(inp, seed=seed)
            inp["kv_pages"], inp["kv_scales"] = kv4, sc
        return inp

    fp8_row = cfg["d_c"] + 2 * cfg["d_R"] + 4  # FP8 c_KV + bf16 k_R + fp32 scale
    mx_row = cfg["d_c"] // 2 + 2 * cfg["d_R"] + cfg["d_c"] // 32  # E2M1 + bf16 k_R + E8M0
    if args.kv_mxfp4 and cfg["H"] == 128:
        raise SystemExit("--kv-mxfp4: the MXFP4 cache is read at the MHA2MLA widths "
                         "(--workload 5)")
    base = with_fp8(with_tokens(W.config_inputs(args.workload), cfg["seed"] + 500),
                    cfg["seed"] + 700)
    alg = algorithmic(base, T, fp8_row if args.kv_fp8 else (mx_row if args.kv_mxfp4 else None))
    n_sets = args.sets or max(1, math.ceil(2 * MALL_BYTES / alg["bytes"]))
    sets = []
    for i in range(n_sets):
        inp = base if i == 0 else with_fp8(with_tokens(
            W.config_inputs(args.workload, seed=cfg["seed"] + 1000 * i),
            cfg["seed"] + 1000 * i + 500), cfg["seed"] + 1000 * i + 700)
        sets.append({k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()})
    d0 = sets[0]
    dims = M.make_dims(d0["q_nope"], d0["q_rope"], d0["W_UK"], d0["W_UV"], d0["kv_pages"],
                       d0["page_table"], prefill_threshold=args.prefill_threshold)
    ws_bytes = M.workspace_bytes(dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = [torch.empty(((d["B"],) if T == 1 else (d["B"], T)) + (d["H"], d["d_v"]),
                        dtype=torch.bfloat16, device=dev) for d in sets]
    stream = torch.cuda.current_stream(dev)
    vp = ctypes.c_void_p

    names = ("q_nope", "q_rope", "W_UK", "W_UV", "kv_pages") + \
        (("kv_scales",) if args.kv_fp8 or args.kv_mxfp4 else ()) + ("page_table", "seq_lens")

    def argv(i):
        d = sets[i]
        return [vp(d[k].data_ptr()) for k in names] + \
            [vp(outs[i].data_ptr()), vp(0), vp(ws.data_ptr()), ctypes.c_size_t(ws_bytes),
             vp(stream.cuda_stream)]
    call_args = [argv(i) for i in range(n_sets)]
    dref = ctypes.byref(dims)
    hip = Hip()
    K, Wu = args.steps, args.warmup
    ev = [[hip.event() for _ in range(6)] for _ in range(K)]  # start, end of each kernel
    ev_arr = [(vp * 6)(*e) for e in ev]
    nullev = ctypes.POINTER(vp)()

    entry = (lib.mla_decode_fp8 if args.kv_fp8 else
             lib.mla_decode_mxfp4 if args.kv_mxfp4 else lib.mla_decode_timed)

    def step(i, events=nullev):
        rc = entry(dref, *call_args[i % n_sets], events)
        if rc != 0:
            raise RuntimeError("mla_decode failed: %s" % lib.mla_status_str(rc).decode())

    def timed(rotate):
        """Step time from K plain calls (no events in the timed loop), then the per-kernel
        durations from K more calls whose kernels carry HIP events bound to their own start
        and end (the launch gap before a kernel is not counted)."""
        for i in range(Wu):
            step(i if rotate else 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(i if rotate else 0)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(K):
            step(i if rotate else 0, ev_arr[i])
        torch.cuda.synchronize()
        stages = [[hip.ms(e[2 * k], e[2 * k + 1]) for e in ev] for k in range(3)]
        return (t1 - t0) / K, [sum(s) / K for s in stages]

    sec, stage_ms = timed(rotate=True)
    warm_sec, warm_stage_ms = timed(rotate=False) if not args.cold_only else (None, None)

    attn_s = stage_ms[1] * 1e-3
    decompressed = T >= (args.prefill_threshold or (256 if cfg["H"] == 128 else 1 << 30))
    # the counter records were taken on the one-token decode's attention kernel
    record = cfg["name"] + ("_fp8" if args.kv_fp8 else "_mxfp4" if args.kv_mxfp4 else "") \
        if T == 1 else None
    traffic = measured_traffic(record) if record else None
    if decompressed:
        # the middle stage brackets the whole branch: W_UV transpose, then per group of
        # sequences the decompression and the causal attention, all MFMA work
        achieved = alg["decomp_flops"] / attn_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "decompressed branch (transpose_wuv_kernel, decompress_kernel, "
                              + ("prefill_attn_ds_kernel)" if cfg["H"] == 128
                                 else "prefill_attn_kernel)"),
                    "avg_us": round(stage_ms[1] * 1e3, 2)}
    elif alg["attn_flops"] / alg["attn_bytes"] > RIDGE_FLOP_PER_BYTE:
        # several query tokens: each cache byte feeds T rows, past the MFMA ridge point
        achieved = alg["attn_flops"] / attn_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                    "kernel": "attn_deepseek_kernel" if cfg["H"] == 128
                    else "attn_mha2mla_kernel", "avg_us": round(stage_ms[1] * 1e3, 2)}
    else:
        achieved = alg["attn_bytes"] / attn_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "kernel": "attn_deepseek_kernel" if cfg["H"] == 128
                    else "attn_mha2mla_kernel", "avg_us": round(stage_ms[1] * 1e3, 2)}
    call_frac = max(alg["bytes"] / (HBM_PEAK_GBS * 1e9), alg["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)) / sec
    res = {
        "metric": METRIC, "value": round(alg["sumS"] / sec, 1), "unit": "KV-tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wu, "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": cfg["B"], "seq_len": base["seq_lens"].tolist()[0]
                   if cfg["seq"][0] == "fixed" else "ragged", "kv_tokens": alg["sumS"],
                   "heads": cfg["H"], "d_nope": cfg["d_n"], "d_latent": cfg["d_c"],
                   "d_rope": cfg["d_R"], "d_v": cfg["d_v"], "page_size": 64,
                   "page_table": cfg["layout"], "input_sets_rotated": n_sets,
                   "query_tokens_per_seq": T,
                   "branch": "decompressed" if decompressed else "absorbed",
                   "kv_cache": ("fp8_e4m3 c_KV + bf16 k_R + fp32 scale per token, %d B"
                                % fp8_row) if args.kv_fp8 else
                               ("mxfp4 (E2M1) c_KV + bf16 k_R + E8M0 scale per 32 elements, "
                                "%d B per token, synthetic codes" % mx_row)
                               if args.kv_mxfp4 else "bf16"},
        "tflops": round(alg["flops"] / sec / 1e12, 2),
        "gbps": round(alg["bytes"] / sec / 1e9, 1),
        "roofline_frac_call": round(call_frac, 4),
        "kernels_us": stage_us(stage_ms, decompressed),
        "roofline": roofline,
    }
    if warm_sec is not None:
        res["warm"] = {"ms_per_step": round(warm_sec * 1e3, 5),
                       "value": round(alg["sumS"] / warm_sec, 1),
                       "kernels_us": stage_us(warm_stage_ms, decompressed)}
    for e in ev:
        for x in e:
            hip.destroy(x)
    util = measured_mfma_util(record) if record else None
    if util is not None:
        res["roofline"]["mfma_util"] = util
    if not args.no_cpu and T == 1 and not args.kv_fp8 and not args.kv_mxfp4:
        res["cpu_baseline"] = cpu_baseline(base, alg, gpu_out=outs[0].float().cpu().numpy())
    else:
        res["cpu_baseline"] = None
    return res


def run_out(args):
    """Times mla_decode_out (the decode with the merged output projection W_UVO
    [hidden, H*d_c]) on the workload, cold (input sets rotated as in the decode bench), with
    HIP events around K plain calls."""
    import torch
    import mla_latent_kv_14_amd as M
    import workloads as W

    cfg = W.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hidden = args.out_proj
    base = W.config_inputs(args.workload)
    alg = algorithmic(base)
    K = base["H"] * base["d_c"]
    wbytes = 2 * hidden * K
    n_sets = args.sets or max(1, math.ceil(2 * MALL_BYTES / (alg["bytes"] + wbytes)))
    sets = []
    for i in range(n_sets):
        inp = base if i == 0 else W.config_inputs(args.workload, seed=cfg["seed"] + 1000 * i)
        g = torch.Generator().manual_seed(cfg["seed"] + 1000 * i + 9)
        inp = dict(inp)
        inp["W_UVO"] = (torch.randn(hidden, K, generator=g) / K ** 0.5).to(torch.bfloat16)
        sets.append({k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()})
    d0 = sets[0]
    dims = M.make_dims(d0["q_nope"], d0["q_rope"], d0["W_UK"], d0["W_UV"], d0["kv_pages"],
                       d0["page_table"])
    if args.kv_fp8 or args.kv_mxfp4:
        raise SystemExit("--kv-fp8 and --kv-mxfp4 do not apply to --out-proj (its decode reads "
                         "a bf16 cache)")
    ws_bytes = M.workspace_bytes(dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = [torch.empty((d["B"], hidden), dtype=torch.bfloat16, device=dev) for d in sets]
    stream = torch.cuda.current_stream(dev)
    vp = ctypes.c_void_p
    lib = M.lib()
    calls = [[ctypes.byref(dims), ctypes.c_int32(hidden)] +
             [vp(d[k].data_ptr()) for k in ("q_nope", "q_rope", "W_UK", "W_UVO", "kv_pages",
                                            "page_table", "seq_lens")] +
             [vp(o.data_ptr()), vp(0), vp(ws.data_ptr()), ctypes.c_size_t(ws_bytes),
              vp(stream.cuda_stream)] for d, o in zip(sets, outs)]
    for i in range(args.warmup):
        lib.mla_decode_out(*calls[i % n_sets])
    hip = Hip()
    e0, e1 = hip.event(), hip.event()
    hip.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    hip.L.hipEventRecord(e0, vp(stream.cuda_stream))
    for i in range(args.steps):
        if lib.mla_decode_out(*calls[i % n_sets]) != 0:
            raise RuntimeError("mla_decode_out failed")
    hip.L.hipEventRecord(e1, vp(stream.cuda_stream))
    torch.cuda.synchronize()
    sec = hip.ms(e0, e1) * 1e-3 / args.steps
    nbytes = alg["bytes"] - 2 * base["H"] * base["d_c"] * base["d_v"] + wbytes \
        - 2 * base["B"] * base["H"] * base["d_v"] + 2 * base["B"] * hidden
    return {"metric": "MLA decode with merged output projection, KV-tokens/s",
            "value": round(alg["sumS"] / sec, 1), "unit": "KV-tokens/s",
            "ms_per_step": round(sec * 1e3, 5), "steps": args.steps, "warmup": args.warmup,
            "config": {"workload": cfg["name"], "hidden": hidden, "input_sets_rotated": n_sets},
            "gbps": round(nbytes / sec / 1e9, 1)}


def run_append(args):
    """Times mla_cache_append (one new token per sequence of the workload, T = --q-len) with
    HIP events on the library's stream; algorithmic bytes = both weights + x + the written
    rows (it is bound by streaming the weights)."""
    import torch
    import mla_latent_kv_14_amd as M
    import workloads as W

    cfg = W.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hidden = 7168 if cfg["H"] == 128 else 4096  # DeepSeek-V3 and Llama-2-7B model widths
    inp = W.config_inputs(args.workload)
    B, T, d_c, d_R = inp["B"], args.q_len, inp["d_c"], inp["d_R"]
    g = torch.Generator().manual_seed(cfg["seed"] + 7)
    x = torch.randn(B, T, hidden, generator=g).to(torch.bfloat16).to(dev)
    Wd = (torch.randn(d_c, hidden, generator=g) / hidden ** 0.5).to(torch.bfloat16).to(dev)
    Wr = (torch.randn(d_R, hidden, generator=g) / hidden ** 0.5).to(torch.bfloat16).to(dev)
    sc = None
    if args.kv_fp8:  # append into an FP8 copy of the cache
        kv8, sc8 = W.fp8_cache(inp, seed=cfg["seed"] + 8)
        kv, sc = kv8.to(dev), sc8.to(dev)
    elif args.kv_mxfp4:  # append into an MXFP4 cache of the workload's geometry
        kv4, sc4 = W.mxfp4_cache(inp, seed=cfg["seed"] + 8)
        kv, sc = kv4.to(dev), sc4.to(dev)
    else:
        kv = inp["kv_pages"].to(dev)
    pt = inp["page_table"].to(dev)
    # room for the new tokens: append before each sequence's last T tokens
    before = (inp["seq_lens"] - T).clamp(min=0).to(torch.int32).to(dev)
    M.cache_append(x, Wd, Wr, kv, pt, before, kv_scales=sc)  # checks the arguments once
    # then the C entry point directly, with prebuilt arguments (per-call Python checks would
    # make the loop host-bound)
    lib = M.lib()
    d = M.AppendDims()
    d.batch, d.q_len, d.hidden, d.d_latent, d.d_rope = B, T, hidden, d_c, d_R
    d.page_size, d.max_pages_per_seq, d.num_pages = 64, pt.shape[1], kv.shape[0]
    d.rope_base = 10000.0
    stream = torch.cuda.current_stream(dev)
    vp = ctypes.c_void_p
    wsb = M.binding.append_workspace_bytes(d)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    call = [ctypes.byref(d)] + [vp(t.data_ptr()) for t in (x, Wd, Wr, pt, before, kv)] + \
        ([vp(sc.data_ptr())] if sc is not None else []) + \
        [vp(ws.data_ptr()), ctypes.c_size_t(wsb), vp(stream.cuda_stream)]
    entry = (lib.mla_cache_append_fp8 if args.kv_fp8 else
             lib.mla_cache_append_mxfp4 if args.kv_mxfp4 else lib.mla_cache_append)
    for _ in range(args.warmup):
        entry(*call)
    hip = Hip()
    e0, e1 = hip.event(), hip.event()
    hip.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    hip.L.hipEventRecord(e0, ctypes.c_void_p(stream.cuda_stream))
    for _ in range(args.steps):
        if entry(*call) != 0:
            raise RuntimeError("mla_cache_append failed")
    hip.L.hipEventRecord(e1, ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    us = hip.ms(e0, e1) * 1e3 / args.steps
    row = ((d_c + 2 * d_R + 4) if args.kv_fp8 else
           (d_c // 2 + 2 * d_R + d_c // 32) if args.kv_mxfp4 else 2 * (d_c + d_R))
    nbytes = 2 * (d_c + d_R) * hidden + 2 * B * T * hidden + B * T * row
    return {"metric": "MLA cache append (c_KV = x W_DKV, RoPE(x W_KR)) per call",
            "value": round(us, 3), "unit": "us", "higher_is_better": False,
            "steps": args.steps, "warmup": args.warmup,
            "config": {"workload": cfg["name"], "batch": B, "new_tokens_per_seq": T,
                       "hidden": hidden, "d_latent": d_c, "d_rope": d_R,
                       "kv_cache": "fp8" if args.kv_fp8 else "mxfp4" if args.kv_mxfp4
                       else "bf16"},
            "gbps": round(nbytes / us / 1e3, 1),
            "roofline": {"bound": "hbm", "achieved": round(nbytes / us / 1e3, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}}


def cpu_baseline(inp, alg, runs=3, gpu_out=None):
    """The fp64 oracle, as it stands, on the host cores: every (b, h) of one input set, the
    median of `runs` runs (each run well under a minute at every workload but the longest).
    With gpu_out (the timed GPU output of that same input set) the leg also reports how far it
    is from the oracle's output: rel-L2 over the whole tensor and the largest absolute error."""
    import numpy as np
    import oracle
    import workloads as W
    cores = len(os.sched_getaffinity(0))
    args = W.oracle_args(inp)
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        ref, _ = oracle.decode(*args, threads=cores)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    res = {"value": round(alg["sumS"] / dt, 1), "unit": "KV-tokens/s", "cores": cores,
           "kind": "oracle",
           "sample": "all %d (b,h) pairs of one input set of this workload (%d KV tokens), "
                     "fp64, OpenMP over (b,h); median of %d runs, %.2f s wall each"
                     % (inp["B"] * inp["H"], alg["sumS"], runs, dt)}
    if gpu_out is not None:
        g = np.asarray(gpu_out, dtype=np.float64)
        r = np.asarray(ref, dtype=np.float64)
        res["parity"] = {"rel_l2": float("%.3e" % (np.linalg.norm(g - r) / np.linalg.norm(r))),
                         "max_abs": float("%.3e" % np.max(np.abs(g - r))),
                         "of": "the GPU output of that input set, every (b, h)"}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed calls first (the default, about 0.1 s of back-to-back calls, "
                         "brings the GPU to its steady clocks: after 20 calls the same "
                         "workload timed about 13%% slower)")
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="which workload (2 = B=16, S=4096, the headline)")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0 = enough to "
                    "exceed twice the Infinity Cache)")
    ap.add_argument("--q-len", type=int, default=1, help="query tokens per sequence (the "
                    "sequence's newest tokens, causal among themselves); with more than one, "
                    "value counts (query token, cached token) pairs per second")
    ap.add_argument("--prefill-threshold", type=int, default=0, help="query tokens per "
                    "sequence from which the decompressed branch serves the call (0 = 256)")
    ap.add_argument("--out-proj", type=int, default=0, metavar="HIDDEN",
                    help="time mla_decode_out (merged W_UV W_O to width HIDDEN) instead")
    ap.add_argument("--append", action="store_true", help="time the cache append "
                    "(mla_cache_append) of --q-len new tokens per sequence of the workload "
                    "instead of the decode")
    ap.add_argument("--kv-fp8", action="store_true", help="decode over an FP8 copy of the "
                    "cache with per-token scales")
    ap.add_argument("--kv-mxfp4", action="store_true", help="decode over a synthetic MXFP4 "
                    "cache (E2M1 codes, an E8M0 scale per 32 elements) of the workload's "
                    "geometry; MHA2MLA widths (--workload 5)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--all-workloads", action="store_true", help="one JSON line for each of "
                    "the five workloads instead of one for --workload")
    ap.add_argument("--cold-only", action="store_true", help="skip the single-set warm run")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the decode, run 5 device copies of MIB MiB (a plain copy "
                         "kernel of known size, used to scale the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode runs on a single MI355X and has "
              "no multi-GPU path (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.append:
        res = run_append(args)
    elif args.out_proj:
        res = run_out(args)
    elif args.all_workloads:
        for w in (1, 2, 3, 4, 5):  # one line per workload, the headline's among them
            args.workload = w
            print(json.dumps(run(args)), flush=True)
        return
    else:
        res = run(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
