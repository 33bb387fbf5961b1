#!/usr/bin/env python3
"""Decode-step benchmark of latent-KV attention (MLA / MLRA-n) on one MI355X.

One step = one full `mlra_decode` call (absorb_q with the split-KV plan ->
split-KV decode -> combine -> out_proj) for one layer over a batch of sequences whose caches are
already resident in HBM. The default workload is MLRA-4 at the DeepSeek-V3
attention shape, B=16, L=32768 (bf16 cache). Cache copies rotate between
steps so that no step is served from the 256 MB Infinity Cache.

Prints ONE JSON line: tokens/s (value), KV-cache GB/s, the roofline of the
split-KV decode kernel (timed live inside the timed region: the decode
dispatch of every N-th step stamps a pair of HIP events at its start and end)
and the float64 oracle timed on the host cores.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload NAME]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn tokens/s and KV-cache GB/s (% HBM peak) at B=16, L=32K, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "latent_decode_traffic.json")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_traffic.json")
KERNEL_SRC = {"prefill": "branch_rank_amd/csrc/prefill_branch.hip",
              "branch": "branch_rank_amd/csrc/decode_branch.hip",
              "wide": "branch_rank_amd/csrc/decode_wide.hip",
              "head_group": "branch_rank_amd/csrc/decode_mfma.hip",
              "portable": "branch_rank_amd/csrc/kernels_generic.hip"}
# headers each kernel's source includes (their text is part of the kernel)
_CSRC = "branch_rank_amd/csrc/"
KERNEL_DEPS = {"prefill": ["device_common.h", "internal.h"],
               "branch": ["branch_tiles.h", "device_common.h", "internal.h"],
               "wide": ["device_common.h", "internal.h"],
               "head_group": ["device_common.h", "internal.h"],
               "portable": ["internal.h", "plan_device.h"]}


def source_sha(kernel):
    """sha256 over a kernel's source file and the headers it includes, in a
    fixed order: a change to any of them makes counters taken before stale."""
    h = hashlib.sha256()
    for f in [KERNEL_SRC[kernel]] + [_CSRC + d for d in KERNEL_DEPS[kernel]]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mlra4_b16_l32k")
    ap.add_argument("--also", default="mla_b16_l32k,mla_b16_l4k,mlra4_b2_l128k,mla_b2_l128k,"
                                      "shard_b64_ragged",
                    help="comma-separated extra workloads reported beside (empty: none)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "portable", "head_group", "branch"],
                    help="split-KV decode kernel (auto: the library's choice)")
    ap.add_argument("--cache-bytes-min", type=float, default=2.0,
                    help="GiB of rotating cache copies (>= 8x the Infinity Cache)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the clock and power under load (rocm-smi)")
    ap.add_argument("--no-shards", action="store_true",
                    help="skip the per-device tensor-parallel shard comparison")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the causal prefill leg (MLRA-4, 4 prompts of 4096 tokens)")
    ap.add_argument("--prefill-workload", default="mlra4_prefill_b4_t4k")
    ap.add_argument("--mla-prefill-workload", default="mla_prefill_b4_t4k",
                    help="MLA prefill (unabsorbed form) also timed ('' = none)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill leg: print its JSON object and stop")
    ap.add_argument("--time-every", type=int, default=4,
                    help="stamp the decode dispatch's start/end events on every N-th timed step")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--fp8", default="mlra4_b16_l32k,mla_b16_l32k",
                    help="workloads also timed on an fp8 (E4M3) copy of their cache ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe-copy", action="store_true",
                    help="only run a 1 GiB device copy (scale factor for HBM counters)")
    ap.add_argument("--probe-read", action="store_true",
                    help="only run the HBM read-ceiling probe and print its JSON")
    ap.add_argument("--no-probe-read", action="store_true",
                    help="skip the read-ceiling probe in the full run")
    return ap.parse_args()


def kernel_flops_bytes(w, lens, fp8=False):
    """Algorithmic work of the split-KV decode kernel: every cached element is
    read once (the branches share the RoPE key and partition the latent), and
    per token each head does 2*(d_c + d_r) flop for the scores and 2*d_c for
    the value accumulation. fp8 caches hold one byte per element."""
    tokens = int(sum(int(x) for x in lens))
    row = w.d_c + w.d_r
    esz = 1 if fp8 else (2 if w.dtype == "bf16" else 4)
    return tokens * row * esz, tokens * w.heads * 2 * (row + w.d_c), tokens


def traffic_for(workload, kernel, path=TRAFFIC_FILE):
    """HBM bytes per launch from a committed counter summary (one record or a
    list of them), if one was taken on this workload, this kernel and the
    kernel's current source; else None."""
    try:
        with open(path) as f:
            recs = json.load(f)
        src = KERNEL_SRC[kernel]
        sha = source_sha(kernel)
        for t in recs if isinstance(recs, list) else [recs]:
            if (t.get("kernel_source") == src and t.get("kernel_sha256") == sha
                    and t.get("workload") == workload):
                return int(t["hbm_bytes_per_launch"])
        return None
    except (OSError, ValueError, KeyError):
        return None


def sample_clock(step, torch, limit_s=30.0):
    """Shader/memory clock and power while decode steps keep the GPU busy:
    rocm-smi runs as a child process after half a second of steps."""
    import re
    import subprocess
    import threading
    out = {}

    def probe():
        time.sleep(0.5)
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"],
                               capture_output=True, text=True, timeout=20)
            d = json.loads(r.stdout[r.stdout.index("{"):])
            for k, v in next(iter(d.values())).items():
                m = re.search(r"([0-9]+(\.[0-9]+)?)", str(v))
                if not m:
                    continue
                if "sclk clock speed" in k:
                    out["sclk_mhz"] = float(m.group(1))
                elif "mclk clock speed" in k:
                    out["mclk_mhz"] = float(m.group(1))
                elif "Power" in k and "(W)" in k:
                    out["power_w"] = float(m.group(1))
        except Exception as e:  # noqa: BLE001 - best effort, reported as such
            out["error"] = f"{type(e).__name__}: {str(e)[:120]}"

    th = threading.Thread(target=probe)
    th.start()
    t0, i = time.time(), 0
    while th.is_alive() and time.time() - t0 < limit_s:
        for _ in range(50):
            step(i)
            i += 1
        torch.cuda.synchronize()
    th.join()
    out["sampled_during"] = "back-to-back decode steps of the main workload"
    return out


def run_workload(name, steps, warmup, cache_gib, torch, br, synth, kernel="auto", every=4,
                 clock=False, fp8=False):
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w, parts=("q_nope", "q_rope", "w_uk", "w_uv"))
    lens = inp["lens"]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {k: torch.from_numpy(inp[k]).cuda().to(dt) for k in ("q_nope", "q_rope", "w_uk", "w_uv")}
    kv_bytes, flops, tokens = kernel_flops_bytes(w, lens, fp8)
    copies = max(2, min(16, math.ceil(cache_gib * 2**30 / max(kv_bytes, 1))))
    log(f"[bench] {name}: B={w.batch} tokens={tokens} cache={kv_bytes / 1e6:.1f} MB x {copies} copies")
    lens_dev = torch.from_numpy(lens).cuda()
    cfg = br.make_config(w.heads, w.d_c, w.d_r, w.d_n, w.d_v, n=w.n, sm_scale=w.tau,
                         alpha_q=w.alpha_q, alpha_kv=w.alpha_kv, theta=w.theta, dtype=w.dtype,
                         kernel=kernel)
    views, bufs = [], []
    for i in range(copies):
        buf, _ = synth.make_cache_device(w, seed=w.seed + 7919 * (i + 1), lens=lens)
        scales = None
        if fp8:  # E4M3 codes of the same cache, one scale per part
            buf, sc, sr = synth.fp8_device(buf, w.d_c)
            scales = (sc, sr)
        bufs.append(buf)
        views.append(br.cache_view(buf[..., :w.d_c], buf[..., w.d_c:], lens_dev, cfg,
                                   fp8_scales=scales))
    ws = br.alloc_workspace(cfg, w.batch, bufs[0].shape[1])
    kname = br.select_decode_kernel(cfg, views[0])
    out = torch.empty(w.batch, w.heads, w.d_v, dtype=torch.float32, device="cuda")

    def step(i):
        br.mlra_decode(cfg, w.n, dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"],
                       views[i % copies], ws, out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the decode dispatch of every `every`-th timed step stamps a pair of events
    # (hipExtLaunchKernel); such a dispatch is followed by a gap of a few us, so
    # the other steps run without events
    every = max(1, every)
    timed = list(range(0, steps, every))
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in timed]
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for a, b in kev:  # create the hipEvents outside the timed region
        a.record()
        b.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    for i in range(steps):
        if i % every == 0:
            br.set_kernel_timing(*kev[i // every])
        elif i % every == 1:
            br.set_kernel_timing(None, None)
        step(i)
    g1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    br.set_kernel_timing(None, None)
    ms_step = (t1 - t0) * 1e3 / steps
    gpu_ms_step = g0.elapsed_time(g1) / steps
    k_all = sorted(a.elapsed_time(b) for a, b in kev)
    k_ms = sum(k_all) / len(k_all)
    pct = lambda q: k_all[min(len(k_all) - 1, int(round(q * (len(k_all) - 1))))] * 1e3  # noqa: E731
    assert torch.isfinite(out).all().item(), "non-finite output"
    clk = sample_clock(step, torch) if clock else None  # after the timed region
    del bufs, views
    return dict(w=w, lens=lens, kv_bytes=kv_bytes, flops=flops, tokens=tokens, copies=copies,
                kernel=kname, timed_launches=len(kev),
                kernel_us_p10_p50_p90=[pct(0.1), pct(0.5), pct(0.9)], clock=clk,
                ms_step=ms_step, gpu_ms_step=gpu_ms_step, kernel_ms=k_ms)


def time_cache_append(w, steps, warmup, torch, br):
    """Mean time of one mlra_cache_append call (one token per sequence) at the
    workload's shape, on a cache with room: the step before each decode."""
    L = steps + warmup + 1
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    buf = torch.zeros(w.batch, L, w.d_c + w.d_r, dtype=dt, device="cuda")
    lens = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    rows = torch.randn(w.batch, w.d_c + w.d_r, dtype=torch.float32, device="cuda")
    cfg = br.make_config(w.heads, w.d_c, w.d_r, w.d_n, w.d_v, n=w.n, sm_scale=w.tau,
                         alpha_q=w.alpha_q, alpha_kv=w.alpha_kv, theta=w.theta, dtype=w.dtype)
    ckv, kr = buf[..., :w.d_c], buf[..., w.d_c:]
    for _ in range(warmup):
        br.cache_append(cfg, rows, ckv, kr, lens)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        br.cache_append(cfg, rows, ckv, kr, lens)
    e1.record()
    torch.cuda.synchronize()
    assert int(lens.min().item()) == steps + warmup
    return e0.elapsed_time(e1) * 1e3 / steps


def prefill_flops(w, lens):
    """Algorithmic work of the prefill kernel: each of the L(L+1)/2 (query,
    key) pairs of a sequence costs, per head, 2 d_c' flop per branch for the
    latent part of the score, 2 d_r once for the RoPE part (one dot product
    shared by the branches) and 2 d_c' per branch for the value: 2 (d_r +
    2 d_c) in all (2176 at the DeepSeek-V3 shape); each position and head
    adds the absorption (2 d_c d_n) and the output projection (2 d_c d_v).
    Returns (attention part, total, pairs, attention part with the RoPE dot
    counted once per branch, as a kernel that repeats it executes)."""
    pairs = sum(int(L) * (int(L) + 1) // 2 for L in lens)
    attn = pairs * w.heads * 2 * (w.d_r + 2 * w.d_c)
    attn_rep = pairs * w.heads * 2 * (w.n * w.d_r + 2 * w.d_c)
    rows = int(sum(int(L) for L in lens))
    proj = rows * w.heads * 2 * w.d_c * (w.d_n + w.d_v)
    return attn, attn + proj, pairs, attn_rep


def mha_prefill_flops(w, lens):
    """Algorithmic work of MLA's prefill in the unabsorbed (multi-head) form:
    each (query, key) pair costs, per head, 2 (d_n + d_r) flop for the score
    and 2 d_v for the value (640 at the DeepSeek-V3 shape); each cached row and
    head adds the up-projection 2 d_c (d_n + d_v). Returns (attention part,
    up-projection part, pairs)."""
    pairs = sum(int(L) * (int(L) + 1) // 2 for L in lens)
    attn = pairs * w.heads * 2 * (w.d_n + w.d_r + w.d_v)
    rows = int(sum(int(L) for L in lens))
    return attn, rows * w.heads * 2 * w.d_c * (w.d_n + w.d_v), pairs


def time_prefill(name, steps, warmup, torch, br, synth):
    """One prefill call per step over B full prompts: mlra_prefill (one
    kernel) for several branches, mla_prefill (the up-projection, then the
    attention kernel) for one. The attention dispatch stamps a pair of HIP
    events every step."""
    w = synth.WORKLOADS[name]
    T = w.cache_len
    inp = synth.make_inputs(w, parts=("w_uk", "w_uv"))
    lens = inp["lens"]
    buf, _ = synth.make_cache_device(w, seed=w.seed + 7919, lens=lens)
    lens_dev = torch.from_numpy(lens).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    qn = torch.randn(w.batch, T, w.heads, w.d_n, generator=gen, device="cuda").to(torch.bfloat16)
    qr = torch.randn(w.batch, T, w.heads, w.d_r, generator=gen, device="cuda").to(torch.bfloat16)
    wk = torch.from_numpy(inp["w_uk"]).cuda().to(torch.bfloat16)
    wv = torch.from_numpy(inp["w_uv"]).cuda().to(torch.bfloat16)
    cfg = br.make_config(w.heads, w.d_c, w.d_r, w.d_n, w.d_v, n=w.n, sm_scale=w.tau,
                         alpha_q=w.alpha_q, alpha_kv=w.alpha_kv, theta=w.theta, dtype=w.dtype)
    cache = br.cache_view(buf[..., :w.d_c], buf[..., w.d_c:], lens_dev, cfg)
    out = torch.empty(w.batch, T, w.heads, w.d_v, dtype=torch.bfloat16, device="cuda")
    log(f"[bench] prefill {name}: B={w.batch} T={T}")
    mha = w.n == 1
    ws = (torch.empty(br.mla_prefill_workspace_size(cfg, w.batch, T), dtype=torch.uint8,
                      device="cuda") if mha else None)

    def call():
        if mha:
            br.mla_prefill(cfg, qn, qr, wk, wv, cache, out, workspace=ws)
        else:
            br.mlra_prefill(cfg, w.n, qn, qr, wk, wv, cache, out)

    for _ in range(warmup):
        call()
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for x, y in kev:
        x.record()
        y.record()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record()
    for i in range(steps):
        br.set_kernel_timing(*kev[i])
        call()
    g1.record()
    torch.cuda.synchronize()
    br.set_kernel_timing(None, None)
    assert torch.isfinite(out.float()).all().item(), "non-finite prefill output"
    ms = g0.elapsed_time(g1) / steps
    k_ms = sum(x.elapsed_time(y) for x, y in kev) / steps
    if mha:
        attn, proj, pairs = mha_prefill_flops(w, lens)
        tf = attn / (k_ms / 1e3) / 1e12
        return {"workload": name, "batch": w.batch, "prompt_len": T, "heads": w.heads,
                "branches": w.n, "form": "unabsorbed (multi-head): up-projection + attention",
                "steps": steps, "ms_per_call": ms,
                "prompt_tokens_per_s": int(sum(int(L) for L in lens)) / (ms / 1e3),
                "attention_kernel_ms": k_ms, "up_projection_ms": ms - k_ms,
                "attention_flops": attn, "up_projection_flops": proj,
                "flop_count": "2 (d_n + d_r + d_v) flop per (query, key) pair and head; "
                              "2 d_c (d_n + d_v) per cached row and head",
                "tflops_whole_call": (attn + proj) / (ms / 1e3) / 1e12,
                "attn_pairs": pairs,
                "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                             "note": "attention kernel, fp16 MFMA (same peak as bf16)",
                             "traffic": None}}
    attn, total, pairs, attn_rep = prefill_flops(w, lens)
    tf = total / (k_ms / 1e3) / 1e12
    return {"workload": name, "batch": w.batch, "prompt_len": T, "heads": w.heads,
            "branches": w.n, "steps": steps, "ms_per_call": ms,
            "prompt_tokens_per_s": int(sum(int(L) for L in lens)) / (ms / 1e3),
            "kernel_ms": k_ms, "kernel_flops": total, "attention_flops": attn,
            "flop_count": "RoPE score counted once per (query, key, head): 2 (d_r + 2 d_c) "
                          "flop per pair and head",
            "kernel_tflops_rope_per_branch": (total - attn + attn_rep) / (k_ms / 1e3) / 1e12,
            "attn_pairs": pairs,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                         "traffic": traffic_for(name, "prefill", PREFILL_TRAFFIC_FILE)}}


def cpu_baseline(w, seconds):
    """The float64 oracle (unabsorbed definition) on host cores, one sequence
    at a time of the same workload recipe until `seconds` have elapsed. The
    BLAS threads are set to the CPUs this process may run on (its affinity
    mask), or to OMP_NUM_THREADS when that is set lower (the host's share
    per GPU); `cores` is the count the oracle ran with."""
    import oracle
    import synth
    affinity = len(os.sched_getaffinity(0))
    cores = affinity
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and 0 < int(omp) < cores:
        cores = int(omp)
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # noqa: BLE001
        limiter = None
    try:
        return _cpu_baseline_run(w, seconds, oracle, synth, cores, affinity)
    finally:
        if limiter is not None:
            limiter.restore_original_limits()


def _cpu_baseline_run(w, seconds, oracle, synth, cores, affinity):
    done, spent = 0, 0.0
    L = None
    while spent < seconds and done < w.batch:
        one = w.replace(batch=1)
        inp = synth.make_inputs(one, seed=w.seed + 104729 * (done + 1))
        L = int(inp["lens"][0])
        t0 = time.perf_counter()
        oracle.mlra_decode_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"], inp["ckv"],
                               inp["krope"], inp["lens"], w.n, tau=w.tau, alpha_q=w.alpha_q,
                               alpha_kv=w.alpha_kv, theta=w.theta)
        spent += time.perf_counter() - t0
        done += 1
        log(f"[bench] oracle: {done} sequence(s) in {spent:.1f} s")
    return {"value": done / spent, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {w.batch} sequences (L={L}, all {w.heads} heads, {w.n} branch(es)), "
                      f"float64 unabsorbed oracle, {spent:.1f} s, BLAS threads {cores} "
                      f"(affinity mask {affinity} CPUs)"}


def probe_read(torch, gib=4.0):
    """Measured HBM read ceiling (include/mlra_probe.h): every byte of a
    `gib` GiB buffer (16x the Infinity Cache) read once per launch, through
    VGPR loads and through LDS-DMA, over a few launch shapes; the best
    GB/s of each path. Each shape: one untimed launch, then 3 timed."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "branch_rank_amd", "libmlra_probe.so"))
    lib.mlra_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mlra_probe_read.restype = ctypes.c_int
    n = int(gib * 2**30)
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    # (mode, workgroups, waves, depth)
    shapes = [(0, 1024, 4, 4), (0, 2048, 4, 4), (0, 4096, 4, 2), (0, 1024, 8, 8), (0, 512, 16, 4),
              (1, 256, 8, 8), (1, 256, 8, 12), (1, 256, 16, 8), (1, 512, 8, 8), (1, 512, 4, 12),
              (1, 1024, 4, 8)]
    runs = []
    for mode, wgs, waves, depth in shapes:
        def go():
            rc = lib.mlra_probe_read(buf.data_ptr(), n, mode, wgs, waves, depth, sink.data_ptr(),
                                     stream)
            if rc != 0:
                raise RuntimeError(f"mlra_probe_read returned {rc}")
        go()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            go()
        e1.record()
        torch.cuda.synchronize()
        gbs = 3 * n / (e0.elapsed_time(e1) / 1e3) / 1e9
        runs.append({"path": "vgpr" if mode == 0 else "lds_dma", "workgroups": wgs,
                     "waves": waves, "depth": depth, "gbs": round(gbs, 1)})
        log(f"[bench] read probe {runs[-1]}")
    del buf
    best = {}
    for r in runs:
        if r["gbs"] > best.get(r["path"], {"gbs": 0})["gbs"]:
            best[r["path"]] = r
    return {"buffer_bytes": n, "best_gbs": max(r["gbs"] for r in runs), "vgpr": best["vgpr"],
            "lds_dma": best["lds_dma"], "runs": runs}


def probe_copy(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "launches": 3}))


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}, WORLD_SIZE {world}); "
              "this decode path has no multi-GPU leg.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import branch_rank_amd as br
    import synth
    br.lib()  # fails loudly when the HIP library is missing
    if a.probe_copy:
        probe_copy(torch)
        return
    if a.probe_read:
        print(json.dumps({"probe": "read", **probe_read(torch)}))
        return
    if a.prefill_only:
        print(json.dumps(time_prefill(a.prefill_workload, a.steps, a.warmup, torch, br, synth)))
        return
    main_r = run_workload(a.workload, a.steps, a.warmup, a.cache_bytes_min, torch, br, synth,
                          a.kernel, a.time_every, clock=not a.no_clock)
    extras = {}
    for name in [x for x in a.also.split(",") if x and x != a.workload]:
        r = run_workload(name, a.steps, a.warmup, a.cache_bytes_min, torch, br, synth, a.kernel
                         if a.kernel in ("auto", "portable") else "auto", a.time_every)
        extras[name] = {
            "tokens_per_s": r["w"].batch / (r["ms_step"] / 1e3),
            "ms_per_step": r["ms_step"],
            "decode_kernel": r["kernel"],
            "decode_kernel_us": r["kernel_ms"] * 1e3,
            "kv_cache_gbs_kernel": r["kv_bytes"] / (r["kernel_ms"] / 1e3) / 1e9,
            "kv_cache_gbs_step": r["kv_bytes"] / (r["ms_step"] / 1e3) / 1e9,
        }
    # quantised cache: the same workloads on E4M3 codes (half the bytes),
    # beside the bf16 decode kernel of the same run
    bf16_us = {a.workload: main_r["kernel_ms"] * 1e3,
               **{k: v["decode_kernel_us"] for k, v in extras.items()}}
    fp8 = {}
    for name in [x for x in a.fp8.split(",") if x]:
        r = run_workload(name, a.steps, a.warmup, a.cache_bytes_min, torch, br, synth, "auto",
                         a.time_every, fp8=True)
        k_us = r["kernel_ms"] * 1e3
        fp8[name] = {
            "tokens_per_s": r["w"].batch / (r["ms_step"] / 1e3),
            "ms_per_step": r["ms_step"],
            "decode_kernel": r["kernel"],
            "decode_kernel_us": k_us,
            "kv_bytes": r["kv_bytes"],
            "kv_cache_gbs_kernel": r["kv_bytes"] / (k_us / 1e6) / 1e9,
            "bf16_decode_kernel_us": bf16_us.get(name),
            "speedup_vs_bf16_kernel": bf16_us[name] / k_us if name in bf16_us else None,
        }
    append_us = time_cache_append(main_r["w"], a.steps, a.warmup, torch, br)
    prefill = prefill_mla = None
    if not a.no_prefill:
        prefill = time_prefill(a.prefill_workload, max(2, min(a.steps, 10)), 2, torch, br, synth)
        if a.mla_prefill_workload:
            prefill_mla = time_prefill(a.mla_prefill_workload, max(2, min(a.steps, 10)), 2, torch,
                                       br, synth)
    shards = None
    if not a.no_shards:
        shards = {}
        for tag in ("l32k", "l128k"):
            pair = {}
            for scheme, name in (("mla_tp4", f"mla_tp4_b16_{tag}"),
                                 ("mlra4_branch_shard", f"mlra4_shard_b16_{tag}")):
                r = run_workload(name, a.steps, a.warmup, a.cache_bytes_min, torch, br, synth,
                                 "auto", a.time_every)
                pair[scheme] = {"workload": name, "heads": r["w"].heads,
                                "row_bytes": (r["w"].d_c + r["w"].d_r) * 2,
                                "kv_bytes": r["kv_bytes"], "ms_per_step": r["ms_step"],
                                "decode_kernel": r["kernel"],
                                "decode_kernel_us": r["kernel_ms"] * 1e3,
                                "kv_cache_gbs_kernel": r["kv_bytes"] / (r["kernel_ms"] / 1e3) / 1e9}
            m, s_ = pair["mla_tp4"], pair["mlra4_branch_shard"]
            pair["byte_ratio"] = m["kv_bytes"] / s_["kv_bytes"]
            pair["step_time_ratio"] = m["ms_per_step"] / s_["ms_per_step"]
            pair["kernel_time_ratio"] = m["decode_kernel_us"] / s_["decode_kernel_us"]
            shards[tag] = pair
    ceiling = None if a.no_probe_read else probe_read(torch)
    w = main_r["w"]
    ms = main_r["ms_step"]
    k_s = main_r["kernel_ms"] / 1e3
    kv_gbs_kernel = main_r["kv_bytes"] / k_s / 1e9
    kv_gbs_step = main_r["kv_bytes"] / (ms / 1e3) / 1e9
    res = {
        "metric": METRIC,
        "value": w.batch / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; unit-RMS bf16 latent rows, N(0,1) K_RoPE, random-init W_UK/W_UV)",
        "config": {"workload": w.name, "batch": w.batch, "cache_len": w.cache_len,
                   "heads": w.heads, "d_c": w.d_c, "d_r": w.d_r, "d_nope": w.d_n, "d_v": w.d_v,
                   "branches": w.n, "alpha_q": round(w.alpha_q, 6),
                   "alpha_kv": round(w.alpha_kv, 6), "cache_copies": main_r["copies"],
                   "decode_kernel": main_r["kernel"],
                   "parallelism": "none (1 GPU)"},
        "kv_cache_gbs": kv_gbs_step,
        "kv_cache_frac_hbm_peak": kv_gbs_step / HBM_PEAK_GBS,
        "gpu_ms_per_step": main_r["gpu_ms_step"],
        "decode_kernel_us": main_r["kernel_ms"] * 1e3,
        "decode_kernel_timed_launches": main_r["timed_launches"],
        "decode_kernel_us_p10_p50_p90": main_r["kernel_us_p10_p50_p90"],
        "clock_under_load": main_r["clock"],
        "decode_kernel_kv_gbs": kv_gbs_kernel,
        "decode_kernel_mfma_tflops": main_r["flops"] / k_s / 1e12,
        "decode_kernel_mfma_frac": main_r["flops"] / k_s / 1e12 / BF16_PEAK_TFLOPS,
        "roofline": {"bound": "hbm", "achieved": kv_gbs_kernel, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kv_gbs_kernel / HBM_PEAK_GBS,
                     "traffic": traffic_for(w.name, main_r["kernel"])},
        "measured_read_ceiling": ceiling,
        "roofline_frac_of_measured_ceiling":
            kv_gbs_kernel / ceiling["best_gbs"] if ceiling else None,
        "cache_append_us": append_us,
        "also": extras,
        "shard_compare": shards,
        "fp8_cache": fp8,
        "prefill": prefill,
        "prefill_mla": prefill_mla,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


if __name__ == "__main__":
    main()
