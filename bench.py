"""Benchmark of one TwoTower denoising step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the block attention of one denoiser attention layer (tt_block_attn) and the
confidence-unmask step (tt_unmask_reduce + tt_unmask_commit, which together
are tt_unmask_step), at the first refinement step of a block (every position
still masked, the most logits to read).  Inputs are resident in HBM before
timing starts; several independent input sets are rotated so that the working
set exceeds the 256 MB Infinity Cache and every step streams from HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--graph]
    python bench.py --suite                      (supplementary workloads)
    python bench.py --attn-only --config NAME    (one attention workload, for counter runs)
    python bench.py --lmhead-only                (the fused LM head workloads, for traces)

The timed loop issues each step's three library calls on one stream.  With
--graph each input set's step is captured once into a HIP graph and the loop
replays the graphs instead (checked bit for bit against an eager step; on
this stack the replays have measured slower than the eager calls).

Prints ONE JSON line: block-tokens/s over the timed steps, the roofline of the
dominant kernel (the vocabulary pass, HBM-bound; its duration from HIP events
around a back-to-back loop of that kernel alone on the launch stream), the
attention call measured the same way, and the CPU oracle timed on the host.
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
DEFAULT_CONFIG = "decode_b8_p2048_l32"
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    # The GPU's clocks ramp up over the first ~20 ms of load after an idle
    # spell (input setup): 2000 warm-up steps (~0.1 s) time the steady state.
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--prefix-len", type=int, default=None)
    ap.add_argument("--rotate", type=int, default=0, help="input sets rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


def kernel_source_digest() -> str:
    """Digest of the vocabulary-pass kernel source; counter-derived traffic is
    only reported while it matches the digest recorded with the counters."""
    with open(os.path.join(ROOT, "denoiser_attention_amd", "csrc", "unmask.hip"), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch of the vocabulary pass from the committed rocprofv3
    --pmc summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel factor),
    or None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"vocab_reduce_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    d = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not d or d.group(1) != kernel_source_digest():
        return None
    return float(m.group(1))


def cpu_baseline(cfg, host_sets, mask, min_seconds=10.0):
    """The oracle as it stands, on the host cores, over whole steps of the same
    workload (all heads of the attention call, all masked rows), repeated over
    the rotated input sets until about min_seconds have passed."""
    import threadpoolctl

    import oracle
    blas = [i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
            if i.get("user_api") == "blas"]
    threads = max(blas) if blas else 1
    f = lambda a: oracle.decode_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)
    t_attn = t_unmask = 0.0
    steps = 0
    while steps < len(host_sets) and (steps == 0 or t_attn + t_unmask < min_seconds):
        inp, lg = host_sets[steps]
        t0 = time.perf_counter()
        oracle.block_attn(f(inp["q"]), f(inp["k_ctx"]), f(inp["v_ctx"]), inp["prefix_len"],
                          f(inp["k_blk"]), f(inp["v_blk"]), inp["scale"])
        t_attn += time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.unmask_step(lg, mask, cfg.k)
        t_unmask += time.perf_counter() - t0
        steps += 1
    t_step = (t_attn + t_unmask) / steps
    B, L = mask.shape
    return {
        "value": B * L / t_step, "unit": "block-tokens/s", "cores": threads, "kind": "oracle",
        "sample": (f"{steps} full steps of {cfg.name} (distinct input sets): attention over all "
                   f"{cfg.batch}x{cfg.n_q_heads} (batch, head) pairs in numpy fp64 "
                   f"({t_attn:.2f} s, BLAS threads={threads}), unmask of all {int(mask.sum())} "
                   f"masked rows per step ({t_unmask:.2f} s, one thread)"),
        "seconds": t_attn + t_unmask,
    }


def _roof(bytes_, flops):
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return max(t_hbm, t_mfma), ("hbm" if t_hbm >= t_mfma else "mfma")


def suite(args):
    """Supplementary measurements, one JSON line each (not the headline)."""
    import torch

    sys.path.insert(0, ROOT)
    import denoiser_attention_amd as tt
    from denoiser_attention_amd import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    reps = max(10, args.kernel_reps // 4)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def time_calls(fns, n=reps):
        """Average us per call over back-to-back calls (rotating fns), HIP events,
        after at least 50 ms of untimed calls (the clocks ramp up under load)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            t0 = time.perf_counter()
            i = 0
            while time.perf_counter() - t0 < 0.05:
                for _ in range(8):
                    fns[i % len(fns)]()
                    i += 1
                torch.cuda.synchronize()
            e0.record(stream)
            for i in range(n):
                fns[i % len(fns)]()
            e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    def emit(name, us, bytes_, flops, **extra):
        roof_s, bound = _roof(bytes_, flops)
        line = {"suite": name, "avg_us": us, "bound": bound, "roof_us": roof_s * 1e6,
                "roof_frac": roof_s * 1e6 / us, "GBps": bytes_ / us / 1e3,
                "TFLOPs": flops / us / 1e6}
        line.update(extra)
        print(json.dumps(line), flush=True)

    def n_rotate(set_bytes):
        # Enough independent input sets that one pass over them exceeds 1 GB
        # (four times the Infinity Cache), as in the step benchmark.
        return int(min(48, max(2, np.ceil(1.0e9 / set_bytes))))

    def attn_case(name, cfg, **kw):
        B, Hq, Hkv, D, L = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_len
        P = cfg.prefix_len if "prefix_len" not in kw else kw["prefix_len"]
        n_sets = n_rotate(2 * (2 * B * Hq * L * D + 2 * B * Hkv * (P + L) * D))
        fns, keep = [], []
        for r in range(n_sets):
            inp = synth.attn_inputs(cfg, seed=0, step=r, **kw)
            t = {n: up(inp[n]) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
            out = torch.empty_like(t["q"])
            with torch.cuda.stream(stream):
                fns.append(tt.prepare_block_attn(t["q"], t["k_ctx"], t["v_ctx"], P, t["k_blk"],
                                                 t["v_blk"], cfg.softmax_scale, out, stream=stream))
            keep.append((t, out))
        us = time_calls(fns)
        s = 2
        emit(name, us, s * (2 * B * Hq * L * D + 2 * B * Hkv * (P + L) * D),
             4 * B * Hq * L * (P + L) * D, kind="attention", B=B, P=P, L=L, Hq=Hq, Hkv=Hkv, D=D,
             input_sets=n_sets)
        del keep, fns

    def lmhead_section():
        # Fused LM head + unmask vs the library GEMM + this unmask.
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
                call = tt.prepare_lmhead_unmask_step(h, w, mask, tt.select_rule("top_k", k=8), tok, mo,
                                                     stream=stream)
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


    if args.lmhead_only:
        lmhead_section()
        return

    if args.attn_only:
        kw = {} if args.prefix_len is None else {"prefix_len": args.prefix_len}
        cfg = synth.get_config(args.config, **kw)
        attn_case(f"attn {args.config} P={cfg.prefix_len}", cfg)
        return

    # Attention at every configuration (bf16) and the prefix-bound shapes.
    for name, kw in (("decode_b8_p2048_l32", {}), ("block256_b16_p1024", {}),
                     ("gen8k_b4_l256", dict(prefix_len=512)), ("gen8k_b4_l256", dict(prefix_len=8192)),
                     ("gen8k_b4_l256", dict(prefix_len=16128)), ("highbatch_b64_p4096_l64", {}),
                     ("decode_l16", {}), ("decode_l1", {}), ("decode_b64_p4096_l1", {}),
                     ("decode_b128_p2048_l1", {})):
        cfg = synth.get_config(name, **kw)
        attn_case(f"attn {name} P={cfg.prefix_len}", cfg)

    # Per-sequence prefix lengths (decode geometry, lengths mixed in [0, 2048]).
    cfg = synth.get_config("decode_b8_p2048_l32")
    inp = synth.varlen_inputs(cfg, seed=0, max_prefix_len=2048)
    t = {n: up(inp[n]) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
    lens = torch.from_numpy(inp["prefix_lens"]).to(dev)
    out = torch.empty_like(t["q"])
    fn = lambda: tt.block_attn_varlen(t["q"], t["k_ctx"], t["v_ctx"], lens, 2048, t["k_blk"],
                                      t["v_blk"], cfg.softmax_scale, out=out, stream=stream)
    us = time_calls([fn])
    Ps = inp["prefix_lens"].astype(np.int64)
    B, Hq, Hkv, D, L = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_len
    emit("attn varlen decode_b8 lens=" + ",".join(map(str, Ps.tolist())), us,
         2 * (2 * B * Hq * L * D + 2 * Hkv * int((Ps + L).sum()) * D),
         4 * Hq * L * int((Ps + L).sum()) * D, kind="attention varlen")
    del t, out

    # Training-style pass over all noisy blocks: 8 and 32 blocks of 256.
    for nb, bsz in ((8, 1), (32, 1)):
        cfg = synth.get_config("block256_b16_p1024")
        mb = synth.multiblock_inputs(cfg, nb, 256, seed=0, batch=bsz)
        t = {n: up(mb[n]) for n in ("q", "k_ctx", "v_ctx", "k_noisy", "v_noisy")}
        out = torch.empty_like(t["q"])
        fn = lambda: tt.block_attn_multiblock(t["q"], t["k_ctx"], t["v_ctx"], t["k_noisy"],
                                              t["v_noisy"], 256, cfg.softmax_scale, out=out,
                                              stream=stream)
        us = time_calls([fn], n=max(5, reps // 4))
        Hq, Hkv, D, S = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, 256
        keys = sum(j * S + S for j in range(nb))        # visible keys per query row, summed over blocks
        emit(f"attn multiblock {nb}x256 batch={bsz}", us,
             2 * bsz * (2 * Hq * nb * S * D + 2 * Hkv * (nb * S + (nb - 1) * S) * D),
             4 * bsz * Hq * S * keys * D, kind="attention multiblock")
        del t, out

    # Vocabulary pass and the selection rules (decode workload, all positions masked).
    cfg = synth.get_config("decode_b8_p2048_l32")
    B, L, V = cfg.batch, cfg.block_len, cfg.vocab
    n_sets = n_rotate(B * L * V * 4)
    xs = [up(synth.logits(cfg, seed=0, step=r)) for r in range(n_sets)]
    mask = torch.ones((B, L), dtype=torch.uint8, device=dev)
    tok = torch.zeros((B, L), dtype=torch.int32, device=dev)
    mo = torch.empty_like(mask)
    ws = torch.empty(tt.unmask_workspace_bytes(B, L, V), dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        reds = [tt.prepare_unmask_reduce(x, mask, ws, stream=stream) for x in xs]
        reds[0]()
    emit("unmask reduce decode_b8", time_calls(reds), B * L * V * 4 + B * L, 0,
         kind="vocabulary pass", input_sets=n_sets)
    for mode, params in (("top_k", dict(k=8)), ("threshold", dict(gamma=0.8, steps_left=4)),
                         ("schedule", dict(step=1, n_steps=4)), ("leftmost", dict(k=1))):
        with torch.cuda.stream(stream):
            c = tt.prepare_unmask_commit_ex(mask, tt.select_rule(mode, **params), tok, mo, V, ws,
                                            stream=stream)
        emit(f"unmask commit {mode} decode_b8", time_calls([c]), B * L * 16 * 16 + 2 * B * L, 0,
             kind="selection")
    del xs, reds
    lmhead_section()


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

    import torch

    sys.path.insert(0, ROOT)
    import denoiser_attention_amd as tt
    from denoiser_attention_amd import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sets = []
    host_sets = []
    for r in range(R):
        inp = synth.attn_inputs(cfg, seed=0, step=r)
        lg = synth.logits(cfg, seed=0, step=r)
        if r < 3 and not args.no_cpu_baseline:
            host_sets.append((inp, lg))
        t = {n: up(inp[n]) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk")}
        t["logits"] = up(lg)
        sets.append(t)
        del lg
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
        vocabulary pass) over back-to-back launches on rotated input sets,
        between two HIP events on the launch stream."""
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

    n_masked = B * L
    reduce_bytes = n_masked * V * 4 + B * L          # masked logit rows + mask bytes
    achieved_gbs = reduce_bytes / (reduce_us * 1e-6) / 1e9
    attn_tflops = attn_flops / (attn_us * 1e-6) / 1e12
    attn_t_roof = max(attn_bytes / (HBM_PEAK_GBS * 1e9), attn_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))

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
        "data": "synthetic (seeded N(0,1) Q/K/V, N(0,3) logits with planted peaks; "
                f"{R} input sets rotated)",
        "config": {
            "workload": cfg.name, "batch": B, "prefix_len": P, "block_len": L,
            "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "vocab": V, "k": cfg.k,
            "masked_positions": n_masked, "attention_layers_per_step": 1,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "vocab_reduce_kernel (tt_unmask_reduce)",
            "bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": recorded_traffic(cfg.name),
            "algorithmic_bytes_per_launch": reduce_bytes,
            "avg_launch_us": reduce_us,
            "timing": f"HIP events around {args.kernel_reps} back-to-back launches on the "
                      "launch stream",
        },
        "attention": {
            "avg_call_us": attn_us, "tflops": attn_tflops,
            "mfma_frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS,
            "roof_us": attn_t_roof * 1e6, "roof_frac": attn_t_roof * 1e6 / attn_us,
            "algorithmic_bytes": attn_bytes, "flops": attn_flops,
        },
        "step_launch": "HIP graph replay per step" if graphs is not None else "eager calls",
        "graph_check": graph_check,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, host_sets, np.ones((B, L), np.uint8))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
