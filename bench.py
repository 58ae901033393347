"""Benchmark of one TwoTower denoising step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the block attention of one denoiser attention layer (tt_block_attn) and the
confidence-unmask step (tt_unmask_reduce + tt_unmask_commit, which together
are tt_unmask_step), at the first refinement step of a block (every position
still masked, the most logits to read).  The default workload is the largest
single-GPU configuration: 64 sequences, prefix 4096, block 64, 32 query / 2 KV
heads, head_dim 128, bf16, vocabulary 131072 (4096 masked positions).
Inputs are resident in HBM before timing starts; independent input sets are
rotated so that the working set exceeds the 256 MB Infinity Cache and every
step streams from HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--graph]
    python bench.py --suite                      (supplementary workloads)
    python bench.py --attn-only --config NAME    (one attention workload, for counter runs)
    python bench.py --lmhead-only                (the fused LM head workloads, for traces)

Before the W warm-up steps, the step runs untimed for --prewarm-ms of wall
time: after the idle spell of input setup the GPU's clocks need about 20 ms
of load to ramp up, so the timed steps see steady clocks whatever W is.

Prints ONE JSON line: block-tokens/s over the timed steps; the roofline of
the dominant kernel of the step (the one with the longest average launch,
timed by HIP events around a back-to-back loop of that kernel alone on the
launch stream); both kernels' figures; the CPU oracle timed on a bounded
sample of the same workload on the host cores; and (default workload only,
--no-side skips them) the attention calls of the other configurations and
the step of the 256-token block, each with its fraction of the roof.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix, published
METRIC = "denoised block-tokens/s per denoising step; % HBM/MFMA peak"
DEFAULT_CONFIG = "highbatch_b64_p4096_l64"
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=200.0,
                    help="untimed steps for this much wall time before the warm-up steps "
                         "(the clocks ramp up over the first ~20 ms of load)")
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--prefix-len", type=int, default=None)
    ap.add_argument("--rotate", type=int, default=0, help="input sets rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the other configurations' attention calls and 256-token step")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per input set instead of eager calls")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the step: one JSON line per supplementary workload "
                         "(attention of every configuration, per-sequence prefixes, the "
                         "multi-block pass, selection rules, the fused LM head)")
    ap.add_argument("--attn-only", action="store_true",
                    help="instead of the step: only the attention call of --config "
                         "(and --prefix-len), timed as the suite times it (for counter runs)")
    ap.add_argument("--lmhead-only", action="store_true",
                    help="instead of the step: only the fused LM head workloads of the suite "
                         "(256 and 4096 masked rows), for kernel traces")
    ap.add_argument("--only", default="",
                    help="--suite sections to run, comma-separated: " + ", ".join(SUITE_SECTIONS))
    ap.add_argument("--kernel-reps", type=int, default=200,
                    help="back-to-back launches timed for the per-kernel roofline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of known size (1 GiB read + 1 GiB written),
    repeated 4 times.  rocprofv3 FETCH_SIZE / WRITE_SIZE read on this kernel
    give the scale factor from counter units to bytes."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "launches": 4}}))


# Kernel -> source file whose digest keys its committed counter profile.
KERNEL_SOURCES = {"vocab_reduce": "unmask.hip", "attn_mfma": "attn_mfma.hip"}


def code_digest(text: str) -> str:
    """Digest of C++/HIP source code with its // comments, indentation and
    blank lines removed: a change of wording in a comment keeps it, any change
    of code changes it."""
    lines = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].strip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def kernel_source_digest(kernel: str = "vocab_reduce") -> str:
    """Code digest of a kernel's source file; counter-derived traffic is only
    reported while it matches the digest recorded with the counters."""
    path = os.path.join(ROOT, "denoiser_attention_amd", "csrc", KERNEL_SOURCES[kernel])
    with open(path, encoding="utf-8") as fh:
        return code_digest(fh.read())


def recorded_traffic(workload: str, kernel: str = "vocab_reduce"):
    """HBM bytes per launch of `kernel` at `workload` from the committed
    rocprofv3 --pmc summary profiles/<kernel>_<workload>_traffic.md
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel factor), or None when
    absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    d = re.search(r"kernel_code_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not d or d.group(1) != kernel_source_digest(kernel):
        return None
    return float(m.group(1))


def host_cores() -> int:
    """Host cores this process may use, capped at 16 (the CPU share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_unmask_seq(task):
    """Worker: the oracle's unmask step on one sequence; returns its seconds."""
    import oracle
    x, m, k = task
    t0 = time.perf_counter()
    oracle.unmask_step(x, m, k)
    return time.perf_counter() - t0


def _worker_ready(_):
    import oracle  # noqa: F401
    return os.getpid()


def cpu_baseline(cfg, inp, lg, mask, attn_seqs=8, unmask_seqs=16):
    """The oracle as it stands, timed on the host cores over a bounded sample of
    one step of the workload, scaled to the whole step:
      attention: every query head of the first `attn_seqs` sequences, numpy
        fp64 with BLAS on the host cores; scaled by batch / attn_seqs;
      unmask: the first `unmask_seqs` sequences (every masked row, then the
        per-sequence top-k), one sequence per task in a pool of one process
        per host core (wall time of the pool, transfers included); scaled by
        batch / unmask_seqs.
    Runs before the process touches the GPU (the pool's workers are spawned
    interpreters that load only numpy and the oracle)."""
    import multiprocessing as mp

    import threadpoolctl

    import oracle
    cores = host_cores()
    B, L = mask.shape
    f = lambda a: oracle.decode_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)
    na = min(attn_seqs, B)
    with threadpoolctl.threadpool_limits(limits=cores, user_api="blas"):
        blas = [i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                if i.get("user_api") == "blas"]
        args = [f(inp[n][:na]) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")]
        t0 = time.perf_counter()
        oracle.block_attn(args[0], args[1], args[2], inp["prefix_len"], args[3], args[4],
                          inp["scale"])
        t_attn = time.perf_counter() - t0
    nu = min(unmask_seqs, B)
    tasks = [(lg[b:b + 1], mask[b:b + 1], cfg.k) for b in range(nu)]
    with mp.get_context("spawn").Pool(processes=cores) as pool:
        pool.map(_worker_ready, range(cores))
        t0 = time.perf_counter()
        per_seq = pool.map(_oracle_unmask_seq, tasks, chunksize=1)
        t_unmask = time.perf_counter() - t0
    t_step = t_attn * B / na + t_unmask * B / nu
    rows = int(mask[:nu].sum())
    return {
        "value": B * L / t_step, "unit": "block-tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"one step of {cfg.name}: attention of sequences 0..{na - 1} (all "
                   f"{cfg.n_q_heads} query heads) in numpy fp64, {t_attn:.2f} s with BLAS "
                   f"threads={max(blas) if blas else 1}, scaled x{B / na:g}; unmask of "
                   f"sequences 0..{nu - 1} ({rows} masked rows of {cfg.vocab} logits), "
                   f"{t_unmask:.2f} s wall in {cores} worker processes "
                   f"({sum(per_seq):.1f} s of worker time), scaled x{B / nu:g}"),
        "cores_per_leg": {"attention_blas_threads": max(blas) if blas else 1,
                          "unmask_processes": cores},
        "seconds": t_attn + t_unmask,
        "step_seconds_scaled": t_step,
    }


def _roof(bytes_, flops):
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return max(t_hbm, t_mfma), ("hbm" if t_hbm >= t_mfma else "mfma")


def time_calls_on(torch, stream, fns, n):
    """Average us per call over n back-to-back calls (rotating fns), HIP events
    on the launch stream, after at least 50 ms of untimed calls (the clocks
    ramp up under load)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < 0.05:
            for _ in range(8):
                fns[i % len(fns)]()
                i += 1
            stream.synchronize()
        e0.record(stream)
        for i in range(n):
            fns[i % len(fns)]()
        e1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / n


def rotated_sets(set_bytes, cap=48):
    """Independent input sets whose one pass exceeds 1 GB (four times the
    Infinity Cache), so that every call streams its inputs from HBM."""
    return int(min(cap, max(2, np.ceil(1.0e9 / set_bytes))))


def attn_bytes_flops(B, Hq, Hkv, D, L, P, s=2):
    """Algorithmic bytes and flops of one attention call."""
    return (s * (2 * B * Hq * L * D + 2 * B * Hkv * (P + L) * D), 4 * B * Hq * L * (P + L) * D)


def attention_calls(torch, tt, dev, stream, B, Hq, Hkv, D, L, P, scale, path="auto", n_sets=None):
    """Prepared attention calls over rotated N(0,1) bf16 input sets drawn on the
    device; returns (calls, buffers to keep alive)."""
    n_sets = n_sets or rotated_sets(attn_bytes_flops(B, Hq, Hkv, D, L, P)[0])

    def rnd(*shape):
        return torch.randn(*shape, device=dev, dtype=torch.float32).to(torch.bfloat16)

    fns, keep = [], []
    for _ in range(n_sets):
        t = dict(q=rnd(B, Hq, L, D), k_ctx=rnd(B, Hkv, P, D), v_ctx=rnd(B, Hkv, P, D),
                 k_blk=rnd(B, Hkv, L, D), v_blk=rnd(B, Hkv, L, D))
        out = torch.empty_like(t["q"])
        with torch.cuda.stream(stream):
            fns.append(tt.prepare_block_attn(t["q"], t["k_ctx"], t["v_ctx"], P, t["k_blk"],
                                             t["v_blk"], scale, out, path=path, stream=stream))
        keep.append((t, out))
    torch.cuda.synchronize()
    return fns, keep


# Attention calls of the other configurations, timed in the default run.
SIDE_ATTENTION = (("decode_b8_p2048_l32", {}), ("block256_b16_p1024", {}),
                  ("gen8k_b4_l256", {"prefix_len": 16128}), ("decode_l16", {}), ("decode_l1", {}))


def side_workloads(torch, tt, synth, dev, stream, logits_sets, reps=40):
    """The other configurations' attention calls, and the step of the 256-token
    block (its attention plus the unmask of its 4096 positions, read from the
    same 4096 logit rows as the default workload's), so that the default run
    records every workload's roof fraction.  The --suite lines cover them in
    more depth (every step of a block, the measured roofs)."""
    lines, block = [], None
    for name, kw in SIDE_ATTENTION:
        c = synth.get_config(name, **kw)
        B, Hq, Hkv, D, L, P = (c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block_len,
                               c.prefix_len)
        bytes_, flops = attn_bytes_flops(B, Hq, Hkv, D, L, P)
        fns, keep = attention_calls(torch, tt, dev, stream, B, Hq, Hkv, D, L, P, c.softmax_scale,
                                    n_sets=rotated_sets(bytes_, cap=16))
        us = time_calls_on(torch, stream, fns, reps)
        roof_s, bound = _roof(bytes_, flops)
        lines.append({"workload": name + (f" P={P}" if kw else ""), "op": "attention",
                      "avg_call_us": us, "bound": bound, "roof_us": roof_s * 1e6,
                      "roof_frac": roof_s * 1e6 / us, "TFLOPs": flops / us / 1e6,
                      "GBps": bytes_ / us / 1e3})
        if name == "block256_b16_p1024":
            block = (c, fns, keep, us)
        else:
            del fns, keep
    c, fns, keep, attn_us = block
    B, L, V = c.batch, c.block_len, c.vocab
    assert all(x.numel() == B * L * V for x in logits_sets)
    mask = torch.ones((B, L), dtype=torch.uint8, device=dev)
    mask_out = torch.empty_like(mask)
    tokens = torch.full((B, L), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        reds = [tt.prepare_unmask_reduce(x.view(B, L, V), mask, ws, stream=stream)
                for x in logits_sets]
        com = tt.prepare_unmask_commit(mask, c.k, tokens, mask_out, V, ws, stream=stream)
    torch.cuda.synchronize()
    n = max(len(fns), len(reds))
    steps = []
    for j in range(n):
        def one(a=fns[j % len(fns)], r=reds[j % len(reds)]):
            a()
            r()
            com()
        steps.append(one)
    us = time_calls_on(torch, stream, steps, reps)
    lines.append({"workload": c.name, "op": "step (attention + unmask of all 4096 positions, k=32)",
                  "avg_step_us": us, "block_tokens_per_s": B * L / (us * 1e-6),
                  "attention_us": attn_us})
    del fns, keep, reds
    return lines


SUITE_SECTIONS = ("probes", "attention", "gen8k_sweep", "varlen", "multiblock", "unmask",
                  "selection", "trace8k", "layers6", "crossover", "lmhead")


def suite(args):
    """Supplementary measurements, one JSON line each (not the headline).

    Sections (``--only a,b``; default all): roof probes (what this chip
    sustains: HBM streaming read, back-to-back bf16 MFMA), attention at every
    configuration and the prefix-bound shapes, the 8K-generation prefix sweep,
    per-sequence prefixes, the multi-block pass, the unmask at every
    configuration over every step of a block, the selection rules, the
    8K-token generation trace (32 blocks of 256), the step with six attention
    layers, the MFMA / wavefront-shuffle crossover, and the fused LM head.
    Every line carries its fraction of the datasheet roof and, once the probes
    have run, of the measured roof.  Inputs are drawn on the device
    (N(0,1) bf16 Q/K/V, N(0,3) fp32 logits): timings do not depend on values."""
    import ctypes

    import torch

    sys.path.insert(0, ROOT)
    import denoiser_attention_amd as tt
    from denoiser_attention_amd import synth

    only = set(SUITE_SECTIONS if not args.only else args.only.split(","))
    unknown = only - set(SUITE_SECTIONS)
    if unknown:
        raise SystemExit(f"bench.py: unknown suite sections {sorted(unknown)}")
    if args.attn_only:
        only = {"attn_only"}
    if args.lmhead_only:
        only = {"lmhead"}

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    reps = max(10, args.kernel_reps // 4)
    measured = {}    # measured roofs: "hbm" GB/s, "mfma" TFLOP/s

    def time_calls(fns, n=reps):
        return time_calls_on(torch, stream, fns, n)

    def fracs(us, bytes_, flops):
        roof_s, bound = _roof(bytes_, flops)
        out = {"bound": bound, "roof_us": roof_s * 1e6, "roof_frac": roof_s * 1e6 / us}
        if measured:
            t_m = max(bytes_ / (measured["hbm"] * 1e9), flops / (measured["mfma"] * 1e12))
            out["measured_roof_us"] = t_m * 1e6
            out["measured_roof_frac"] = t_m * 1e6 / us
        return out

    def emit(name, us, bytes_, flops, **extra):
        line = {"suite": name, "avg_us": us}
        line.update(fracs(us, bytes_, flops))
        line.update({"GBps": bytes_ / us / 1e3, "TFLOPs": flops / us / 1e6})
        line.update(extra)
        print(json.dumps(line), flush=True)

    n_rotate = rotated_sets

    def randn_bf16(*shape):
        return torch.randn(*shape, device=dev, dtype=torch.float32).to(torch.bfloat16)

    def attn_case(name, B, Hq, Hkv, D, L, P, scale=None, path="auto", extra=None, n=None):
        scale = 1.0 / np.sqrt(D) if scale is None else scale
        bytes_, flops = attn_bytes_flops(B, Hq, Hkv, D, L, P)
        n_sets = n_rotate(bytes_)
        fns, keep = attention_calls(torch, tt, dev, stream, B, Hq, Hkv, D, L, P, scale, path,
                                    n_sets)
        us = time_calls(fns, n=n or reps)
        ex = dict(kind="attention", B=B, P=P, L=L, Hq=Hq, Hkv=Hkv, D=D, path=path,
                  workspace_bytes=tt.attn_workspace_bytes(B, P, L, Hq, Hkv, D, torch.bfloat16,
                                                          path=path),
                  input_sets=n_sets)
        ex.update(extra or {})
        emit(name, us, bytes_, flops, **ex)
        del keep, fns
        return us

    def cfg_attn(name, **kw):
        c = synth.get_config(name, **kw)
        return attn_case(f"attn {name} P={c.prefix_len}", c.batch, c.n_q_heads, c.n_kv_heads,
                         c.head_dim, c.block_len, c.prefix_len)

    # ---- roof probes ----------------------------------------------------------
    if "probes" in only:
        probe = ctypes.CDLL(os.path.join(ROOT, "denoiser_attention_amd", "libtt_probes.so"))
        probe.tt_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_void_p]
        probe.tt_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
        probe.tt_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        probe.tt_probe_mfma_bf16_flops.restype = ctypes.c_double
        sink = torch.zeros(1024, dtype=torch.int32, device=dev)
        nbytes = 1 << 30
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(2)]
        torch.cuda.synchronize()

        def hbm_call(b):
            def f():
                if probe.tt_probe_hbm_read(b.data_ptr(), nbytes, sink.data_ptr(),
                                           stream.cuda_stream) != 0:
                    raise RuntimeError("tt_probe_hbm_read failed")
            return f
        us = time_calls([hbm_call(b) for b in bufs], n=40)
        measured_hbm = nbytes / us / 1e3
        emit("probe hbm streaming read 1 GiB (16 B non-temporal loads, 16 KB per workgroup)", us,
             nbytes, 0, kind="probe", measured_GBps=measured_hbm)
        del bufs
        n_wg, iters = 512, 4096
        flops = probe.tt_probe_mfma_bf16_flops(n_wg, iters)
        rates = {}
        for rnd in (0, 1):
            def mfma_call(rnd=rnd):
                if probe.tt_probe_mfma_bf16(n_wg, iters, rnd, sink.data_ptr(),
                                            stream.cuda_stream) != 0:
                    raise RuntimeError("tt_probe_mfma_bf16 failed")
            us = time_calls([mfma_call], n=40)
            rates[rnd] = flops / us / 1e6
            kind = "random operands" if rnd else "low-entropy operands"
            emit(f"probe bf16 mfma 32x32x16 {kind}, {n_wg} workgroups x 4 waves x {iters} x 4 "
                 "chains", us, 0, flops, kind="probe", measured_TFLOPs=rates[rnd])
        # The measured MFMA roof: random operands, as attention tiles are.
        measured_mfma = rates[1]
        measured.update(hbm=measured_hbm, mfma=measured_mfma)

    if "attn_only" in only:
        kw = {} if args.prefix_len is None else {"prefix_len": args.prefix_len}
        cfg_attn(args.config, **kw)
        return

    # ---- attention at every configuration and the prefix-bound shapes ---------
    if "attention" in only:
        for name, kw in (("decode_b8_p2048_l32", {}), ("block256_b16_p1024", {}),
                         ("gen8k_b4_l256", dict(prefix_len=512)),
                         ("gen8k_b4_l256", dict(prefix_len=8192)),
                         ("gen8k_b4_l256", dict(prefix_len=16128)),
                         ("highbatch_b64_p4096_l64", {}), ("decode_l16", {}), ("decode_l1", {}),
                         ("decode_b64_p4096_l1", {}), ("decode_b128_p2048_l1", {})):
            cfg_attn(name, **kw)

    if "gen8k_sweep" in only:
        for P in synth.GEN8K_SWEEP:
            cfg_attn("gen8k_b4_l256", prefix_len=P)

    # ---- per-sequence prefix lengths ---------------------------------------------
    if "varlen" in only:
        cfg = synth.get_config("decode_b8_p2048_l32")
        inp = synth.varlen_inputs(cfg, seed=0, max_prefix_len=2048)
        t = {n: torch.from_numpy(inp[n].view(np.int16)).to(dev).view(torch.bfloat16)
             for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
        lens = torch.from_numpy(inp["prefix_lens"]).to(dev)
        out = torch.empty_like(t["q"])
        with torch.cuda.stream(stream):
            fn = tt.prepare_block_attn_varlen(t["q"], t["k_ctx"], t["v_ctx"], lens, 2048,
                                              t["k_blk"], t["v_blk"], cfg.softmax_scale, out,
                                              stream=stream)
        torch.cuda.synchronize()
        us = time_calls([fn])
        Ps = inp["prefix_lens"].astype(np.int64)
        B, Hq, Hkv, D, L = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_len
        emit("attn varlen decode_b8 lens=" + ",".join(map(str, Ps.tolist())), us,
             2 * (2 * B * Hq * L * D + 2 * Hkv * int((Ps + L).sum()) * D),
             4 * Hq * L * int((Ps + L).sum()) * D, kind="attention varlen")
        del t, out

    # ---- training-style pass over all noisy blocks ------------------------------
    if "multiblock" in only:
        Hq, Hkv, D, S = 32, 2, 128, 256
        for nb in (8, 32):
            T = nb * S
            q, kn, vn = randn_bf16(1, Hq, T, D), randn_bf16(1, Hkv, T, D), randn_bf16(1, Hkv, T, D)
            kc, vc = randn_bf16(1, Hkv, T, D), randn_bf16(1, Hkv, T, D)
            out = torch.empty_like(q)
            with torch.cuda.stream(stream):
                fn = tt.prepare_block_attn_multiblock(q, kc, vc, kn, vn, S, 1.0 / np.sqrt(D), out,
                                                      stream=stream)
            torch.cuda.synchronize()
            us = time_calls([fn], n=max(5, reps // 4))
            keys = sum(j * S + S for j in range(nb))
            emit(f"attn multiblock {nb}x256 batch=1", us,
                 2 * (2 * Hq * nb * S * D + 2 * Hkv * (nb * S + (nb - 1) * S) * D),
                 4 * Hq * S * keys * D, kind="attention multiblock")
            del q, kn, vn, kc, vc, out

    # ---- unmask at every configuration over every step of a block ---------------
    def unmask_steps(name, B, L, V, k, T, n_sets):
        """Step r of T: the reduce and commit over the masked set the kernels
        themselves left after steps 1..r-1 (top-k, k per step)."""
        xs = [torch.randn(B, L, V, device=dev) * 3.0 for _ in range(n_sets)]
        mask = torch.ones((B, L), dtype=torch.uint8, device=dev)
        tok = torch.zeros((B, L), dtype=torch.int32, device=dev)
        ws = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        total_us = 0.0
        for r in range(1, T + 1):
            n_masked = int(mask.sum().item())
            mo = torch.empty_like(mask)
            with torch.cuda.stream(stream):
                reds = [tt.prepare_unmask_reduce(x, mask, ws, stream=stream) for x in xs]
                com = tt.prepare_unmask_commit(mask, k, tok, mo, V, ws, stream=stream)
            torch.cuda.synchronize()
            us_r = time_calls(reds)
            us_c = time_calls([com])
            total_us += us_r + us_c
            emit(f"unmask {name} step {r}/{T} reduce", us_r, n_masked * V * 4 + B * L, 0,
                 kind="vocabulary pass", masked=n_masked, commit_us=us_c, input_sets=n_sets)
            with torch.cuda.stream(stream):
                reds[0]()
                com()
            torch.cuda.synchronize()
            mask = mo
        return total_us

    if "unmask" in only:
        for name in ("decode_b8_p2048_l32", "block256_b16_p1024", "gen8k_b4_l256",
                     "highbatch_b64_p4096_l64"):
            c = synth.get_config(name)
            n_sets = 2 if c.batch * c.block_len * c.vocab * 4 > 4.0e8 else 8
            tot = unmask_steps(name, c.batch, c.block_len, c.vocab, c.k, c.steps, n_sets)
            print(json.dumps({"suite": f"unmask {name} whole block ({c.steps} steps)",
                              "avg_us": tot, "kind": "unmask block",
                              "committed_tokens": c.batch * c.block_len}), flush=True)

    # ---- selection rules (decode workload, all positions masked) ---------------
    if "selection" in only:
        cfg = synth.get_config("decode_b8_p2048_l32")
        B, L, V = cfg.batch, cfg.block_len, cfg.vocab
        x = torch.randn(B, L, V, device=dev) * 3.0
        mask = torch.ones((B, L), dtype=torch.uint8, device=dev)
        tok = torch.zeros((B, L), dtype=torch.int32, device=dev)
        mo = torch.empty_like(mask)
        ws = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=dev)
        with torch.cuda.stream(stream):
            tt.prepare_unmask_reduce(x, mask, ws, stream=stream)()
        for mode, params in (("top_k", dict(k=8)), ("threshold", dict(gamma=0.8, steps_left=4)),
                             ("schedule", dict(step=1, n_steps=4)), ("leftmost", dict(k=1))):
            with torch.cuda.stream(stream):
                c = tt.prepare_unmask_commit_ex(mask, tt.select_rule(mode, **params), tok, mo, V,
                                                ws, stream=stream)
            emit(f"unmask commit {mode} decode_b8", time_calls([c]), B * L * 16 * 16 + 2 * B * L,
                 0, kind="selection")
        del x

    # ---- 8K tokens generated as 32 blocks of 256 ---------------------------------
    if "trace8k" in only:
        cfg = synth.get_config("gen8k_b4_l256")
        B, L, Hq, Hkv, D, V, k = (cfg.batch, cfg.block_len, cfg.n_q_heads, cfg.n_kv_heads,
                                  cfg.head_dim, cfg.vocab, cfg.k)
        prompt, n_blocks, T = 8192, 32, cfg.steps
        cap = prompt + L * n_blocks
        kc, vc = randn_bf16(B, Hkv, cap, D), randn_bf16(B, Hkv, cap, D)
        qs = [randn_bf16(B, Hq, L, D) for _ in range(2)]
        kbs = [randn_bf16(B, Hkv, L, D) for _ in range(2)]
        vbs = [randn_bf16(B, Hkv, L, D) for _ in range(2)]
        xs = [torch.randn(B, L, V, device=dev) * 3.0 for _ in range(2)]
        out = torch.empty_like(qs[0])
        tok = torch.zeros((B, L), dtype=torch.int32, device=dev)
        masks = [torch.empty((B, L), dtype=torch.uint8, device=dev) for _ in range(T + 1)]
        ws_u = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=dev)
        ws_a = torch.empty(max(1, max(tt.attn_workspace_bytes(B, prompt + L * b, L, Hq, Hkv, D,
                                                              torch.bfloat16)
                                      for b in range(n_blocks))), dtype=torch.uint8, device=dev)
        scale = 1.0 / np.sqrt(D)

        # Every call validated once up front (one prepared call per block's
        # prefix length, per step's masks and per logits set); the trace then
        # costs one ctypes call per launch on the host.
        with torch.cuda.stream(stream):
            attn_calls = [[tt.prepare_block_attn(qs[j], kc, vc, prompt + L * b, kbs[j], vbs[j],
                                                 scale, out, workspace=ws_a, stream=stream)
                           for j in range(2)] for b in range(n_blocks)]
            red_calls = [[tt.prepare_unmask_reduce(xs[j], masks[r], ws_u, stream=stream)
                          for j in range(2)] for r in range(T)]
            com_calls = [tt.prepare_unmask_commit(masks[r], k, tok, masks[r + 1], V, ws_u,
                                                  stream=stream) for r in range(T)]
            reset = masks[0].fill_
        torch.cuda.synchronize()

        def trace(layers=1):
            i = 0
            for b in range(n_blocks):
                reset(1)
                for r in range(T):
                    for _ in range(layers):
                        attn_calls[b][i % 2]()
                    red_calls[r][i % 2]()
                    com_calls[r]()
                    i += 1

        roof_s = 0.0
        roof_bytes = roof_flops = 0
        n_masked = [L - k * r for r in range(T)]
        for b in range(n_blocks):
            P = prompt + L * b
            ab, af = attn_bytes_flops(B, Hq, Hkv, D, L, P)
            for r in range(T):
                roof_s += _roof(ab, af)[0] + _roof(B * n_masked[r] * V * 4 + B * L, 0)[0]
                roof_bytes += ab + B * n_masked[r] * V * 4 + B * L
                roof_flops += af
        for layers in (1, 6):
            with torch.cuda.stream(stream):
                trace(layers)      # warm
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                trace(layers)
                e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            if layers == 1:
                roof_l = roof_s
            else:
                roof_l = 0.0
                for b in range(n_blocks):
                    ab, af = attn_bytes_flops(B, Hq, Hkv, D, L, prompt + L * b)
                    for r in range(T):
                        roof_l += 6 * _roof(ab, af)[0] + _roof(B * n_masked[r] * V * 4, 0)[0]
            tokens = B * L * n_blocks
            print(json.dumps({
                "suite": f"generation trace gen8k: {n_blocks} blocks of {L} after a {prompt}-token "
                         f"prompt, {T} unmask steps of k={k} per block, {layers} attention "
                         f"layer(s) per step",
                "ms": ms, "committed_tokens": tokens, "committed_tokens_per_s": tokens / (ms * 1e-3),
                "block_tokens_per_s": B * L * n_blocks * T / (ms * 1e-3),
                "roof_ms": roof_l * 1e3, "roof_frac": roof_l * 1e3 / ms,
                "kind": "generation trace"}), flush=True)
        del kc, vc, xs

    # ---- the step with six attention layers ----------------------------------------
    if "layers6" in only:
        for name in ("highbatch_b64_p4096_l64", "decode_b8_p2048_l32", "block256_b16_p1024"):
            c = synth.get_config(name)
            B, L, V, Hq, Hkv, D, P = (c.batch, c.block_len, c.vocab, c.n_q_heads, c.n_kv_heads,
                                      c.head_dim, c.prefix_len)
            layers = [dict(q=randn_bf16(B, Hq, L, D), kc=randn_bf16(B, Hkv, P, D),
                           vc=randn_bf16(B, Hkv, P, D), kb=randn_bf16(B, Hkv, L, D),
                           vb=randn_bf16(B, Hkv, L, D)) for _ in range(6)]
            x = torch.randn(B, L, V, device=dev) * 3.0
            mask = torch.ones((B, L), dtype=torch.uint8, device=dev)
            mo = torch.empty_like(mask)
            tok = torch.zeros((B, L), dtype=torch.int32, device=dev)
            out = torch.empty_like(layers[0]["q"])
            ws_a = torch.empty(max(1, tt.attn_workspace_bytes(B, P, L, Hq, Hkv, D, torch.bfloat16)),
                               dtype=torch.uint8, device=dev)
            ws_u = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=dev)
            with torch.cuda.stream(stream):
                calls = [tt.prepare_block_attn(l["q"], l["kc"], l["vc"], P, l["kb"], l["vb"],
                                               c.softmax_scale, out, workspace=ws_a, stream=stream)
                         for l in layers]
                calls.append(tt.prepare_unmask_reduce(x, mask, ws_u, stream=stream))
                calls.append(tt.prepare_unmask_commit(mask, c.k, tok, mo, V, ws_u, stream=stream))

            def step6():
                for f in calls:
                    f()
            us = time_calls([step6], n=max(10, reps // 2))
            ab, af = attn_bytes_flops(B, Hq, Hkv, D, L, P)
            ub = B * L * V * 4 + B * L
            roof = 6 * _roof(ab, af)[0] + _roof(ub, 0)[0]
            print(json.dumps({
                "suite": f"step with 6 attention layers {name}", "avg_us": us,
                "block_tokens_per_s": B * L / (us * 1e-6), "roof_us": roof * 1e6,
                "roof_frac": roof * 1e6 / us, "kind": "step x6 layers"}), flush=True)
            del layers, x

    # ---- MFMA / wavefront-shuffle crossover (G*L packed rows per KV head) --------
    if "crossover" in only:
        B, Hkv, D, P = 64, 2, 128, 4096
        for G, L in ((1, 1), (2, 1), (4, 1), (8, 1), (12, 1), (16, 1), (24, 1), (32, 1),
                     (4, 4), (8, 2), (16, 2)):
            for path in ("mfma", "shuffle"):
                attn_case(f"crossover G*L={G * L} (G={G}, L={L}) B{B} P{P} {path}", B, G * Hkv, Hkv,
                          D, L, P, path=path, extra=dict(kind="crossover", rows_per_kv_head=G * L))

    # ---- fused LM head + unmask vs the library GEMM + this unmask ---------------
    if "lmhead" in only:
        d = synth.LM_D_MODEL
        for name, B, L in (("decode_b8", 8, 32), ("block256_b16", 16, 256)):
            V = 131072
            torch.manual_seed(0)
            h = torch.randn(B, L, d, device=dev).to(torch.bfloat16)
            w = (torch.randn(V, d, device=dev) * (3.0 / d ** 0.5)).to(torch.bfloat16)
            mask = torch.ones((B, L), dtype=torch.uint8, device=dev)
            tok = torch.zeros((B, L), dtype=torch.int32, device=dev)
            mo = torch.empty_like(mask)
            with torch.cuda.stream(stream):
                call = tt.prepare_lmhead_unmask_step(h, w, mask, tt.select_rule("top_k", k=8), tok,
                                                     mo, stream=stream)
            us = time_calls([call], n=10)
            rows = B * L
            logits = torch.empty((rows, V), dtype=torch.float32, device=dev)
            ws = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=dev)

            def unfused():
                logits.copy_(torch.matmul(h.view(rows, d), w.t()))
                tt.unmask_step(logits.view(B, L, V), mask, 8, tok, mask_out=mo, workspace=ws,
                               stream=stream)
            us_u = time_calls([unfused], n=10)
            emit(f"lmhead+unmask {name} rows={rows} V={V} d={d}", us, V * d * 2 + rows * d * 2,
                 2.0 * rows * V * d, kind="fused LM head", unfused_library_gemm_us=us_u)
            del h, w, logits


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); the "
              "denoising step shards over sequences with no exchange, so throughput at N GPUs "
              "is N independent copies of this measurement.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.suite or args.attn_only or args.lmhead_only:
        suite(args)
        return

    sys.path.insert(0, ROOT)
    from denoiser_attention_amd import synth

    kw = {} if args.prefix_len is None else {"prefix_len": args.prefix_len}
    cfg = synth.get_config(args.config, **kw)
    B, L, V = cfg.batch, cfg.block_len, cfg.vocab
    Hq, Hkv, D, P = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.prefix_len
    s = 2 if cfg.dtype == "bf16" else 4

    attn_bytes = s * (2 * B * Hq * L * D + 2 * B * Hkv * (P + L) * D)
    attn_flops = 4 * B * Hq * L * (P + L) * D
    logits_bytes = B * L * V * 4
    set_bytes = attn_bytes + logits_bytes
    R = args.rotate or max(2, int(np.ceil(1.0e9 / set_bytes)))
    R = min(R, 8)

    # Host inputs of the first set; the CPU oracle is timed on them before the
    # process touches the GPU.
    first = (synth.attn_inputs(cfg, seed=0, step=0), synth.logits(cfg, seed=0, step=0))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, first[0], first[1], np.ones((B, L), np.uint8))

    import torch

    import denoiser_attention_amd as tt

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sets = []
    for r in range(R):
        inp, lg = first if r == 0 else (synth.attn_inputs(cfg, seed=0, step=r),
                                          synth.logits(cfg, seed=0, step=r))
        t = {n: up(inp[n]) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
        t["logits"] = up(lg)
        sets.append(t)
        del inp, lg
    del first
    mask = torch.ones((B, L), dtype=torch.uint8, device=dev)
    mask_out = torch.empty_like(mask)
    tokens = torch.full((B, L), -1, dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, L, D), dtype=sets[0]["q"].dtype, device=dev)
    dt = sets[0]["q"].dtype
    attn_ws_n = tt.attn_workspace_bytes(B, P, L, Hq, Hkv, D, dt)
    attn_ws = torch.empty(max(attn_ws_n, 1), dtype=torch.uint8, device=dev)
    um_ws = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=dev)
    # A stream of our own (default priority): the graphs are captured on it
    # and every timed launch goes to it.
    stream = torch.cuda.Stream(dev)

    # Validate every call once; a step then costs three ctypes calls on the host.
    calls = []
    with torch.cuda.stream(stream):
        for t in sets:
            calls.append((
                tt.prepare_block_attn(t["q"], t["k_ctx"], t["v_ctx"], P, t["k_blk"], t["v_blk"],
                                      cfg.softmax_scale, out,
                                      workspace=attn_ws if attn_ws_n else None, stream=stream),
                tt.prepare_unmask_reduce(t["logits"], mask, um_ws, stream=stream),
                tt.prepare_unmask_commit(mask, cfg.k, tokens, mask_out, V, um_ws, stream=stream),
            ))
    torch.cuda.synchronize()

    def eager_step(i):
        for c in calls[i % R]:
            c()

    graphs = None
    if args.graph:
        graphs = []
        for i in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                eager_step(i)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(i):
        if graphs is None:
            eager_step(i)
        else:
            graphs[i % R].replay()

    # Untimed pre-warm for a fixed wall time (clock ramp), then W warm-up steps.
    prewarm_steps = 0
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        while (time.perf_counter() - t0) * 1e3 < args.prewarm_ms:
            for _ in range(4):
                step(prewarm_steps)
                prewarm_steps += 1
            stream.synchronize()
    prewarm_s = time.perf_counter() - t0
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        t_start.record(stream)
        for i in range(args.steps):
            step(i)
        t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps

    # Graph replays must reproduce an eager step bit for bit.
    graph_check = None
    if graphs is not None:
        tokens.fill_(-1)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            eager_step(0)
        torch.cuda.synchronize()
        ref = (out.clone(), tokens.clone(), mask_out.clone())
        for _ in range(2):
            out.fill_(0)
            tokens.fill_(-1)
            mask_out.fill_(7)
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                graphs[0].replay()
            torch.cuda.synchronize()
            ok = (torch.equal(out.view(torch.int16), ref[0].view(torch.int16))
                  and torch.equal(tokens, ref[1]) and torch.equal(mask_out, ref[2]))
            if not ok:
                print("bench.py: graph replay differs from the eager step", file=sys.stderr)
                sys.exit(1)
        graph_check = "graph replays == eager step (bitwise, 2 replays)"

    def kernel_loop_us(which):
        """Average duration of one launch of call `which` (0 attention, 1
        vocabulary pass, 2 commit) over back-to-back launches on rotated input
        sets, between two HIP events on the launch stream."""
        n = args.kernel_reps
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            for i in range(5):
                calls[i % R][which]()
            e0.record(stream)
            for i in range(n):
                calls[i % R][which]()
            e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    reduce_us = kernel_loop_us(1)
    attn_us = kernel_loop_us(0)
    commit_us = kernel_loop_us(2)

    n_masked = B * L
    reduce_bytes = n_masked * V * 4 + B * L          # masked logit rows + mask bytes
    reduce_gbs = reduce_bytes / (reduce_us * 1e-6) / 1e9
    attn_tflops = attn_flops / (attn_us * 1e-6) / 1e12
    attn_t_roof, attn_bound = _roof(attn_bytes, attn_flops)
    attn_mfma = attn_bound == "mfma"

    vocab_line = {
        "kernel": "vocab_reduce_kernel (tt_unmask_reduce)", "avg_launch_us": reduce_us,
        "bound": "hbm", "GBps": reduce_gbs, "frac": reduce_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_launch": reduce_bytes,
        "traffic": recorded_traffic(cfg.name, "vocab_reduce"),
    }
    attn_line = {
        "kernel": "attn_mfma_kernel (+ split merge when planned) (tt_block_attn)",
        "avg_call_us": attn_us, "tflops": attn_tflops,
        "mfma_frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS, "bound": attn_bound,
        "roof_us": attn_t_roof * 1e6, "roof_frac": attn_t_roof * 1e6 / attn_us,
        "algorithmic_bytes": attn_bytes, "flops": attn_flops,
        "workspace_bytes": attn_ws_n,
        "traffic": recorded_traffic(cfg.name, "attn_mfma") if attn_ws_n == 0 else None,
    }
    timing = (f"HIP events around {args.kernel_reps} back-to-back launches on the launch "
              "stream, rotated input sets")
    if reduce_us >= attn_us:
        roofline = {
            "kernel": vocab_line["kernel"], "bound": "hbm", "achieved": reduce_gbs,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": reduce_gbs / HBM_PEAK_GBS,
            "traffic": vocab_line["traffic"], "algorithmic_bytes_per_launch": reduce_bytes,
            "avg_launch_us": reduce_us, "timing": timing,
        }
    elif attn_mfma:
        roofline = {
            "kernel": attn_line["kernel"], "bound": "mfma", "achieved": attn_tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": attn_line["traffic"],
            "algorithmic_flops_per_launch": attn_flops,
            "algorithmic_bytes_per_launch": attn_bytes, "avg_launch_us": attn_us,
            "timing": timing,
        }
    else:
        gbs = attn_bytes / (attn_us * 1e-6) / 1e9
        roofline = {
            "kernel": attn_line["kernel"], "bound": "hbm", "achieved": gbs,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": attn_line["traffic"], "algorithmic_bytes_per_launch": attn_bytes,
            "avg_launch_us": attn_us, "timing": timing,
        }

    side = None
    if not args.no_side and cfg.name == DEFAULT_CONFIG:
        side = side_workloads(torch, tt, synth, dev, stream, [t["logits"] for t in sets])

    result = {
        "metric": METRIC,
        "value": B * L / (ms_step * 1e-3),
        "unit": "block-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp32" if cfg.dtype == "bf16" else "fp32",
        "data": ("synthetic (seeded N(0,1) Q/K/V"
                 + (", 1% K/V outlier channels x10" if cfg.outlier_frac else "")
                 + ", N(0,3) logits"
                 + (" with planted peaks" if cfg.plant_peaks else "")
                 + (", 5% injected ties" if cfg.tie_frac else "")
                 + f"; {R} input sets rotated)"),
        "config": {
            "workload": cfg.name, "batch": B, "prefix_len": P, "block_len": L,
            "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "vocab": V, "k": cfg.k,
            "masked_positions": n_masked, "attention_layers_per_step": 1,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "attention": attn_line,
        "vocab_pass": vocab_line,
        "commit_us": commit_us,
        "prewarm": {"seconds": prewarm_s, "steps": prewarm_steps},
        "step_launch": "HIP graph replay per step" if graphs is not None else "eager calls",
        "graph_check": graph_check,
        "cpu_baseline": cpu,
        "other_workloads": side,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
