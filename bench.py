"""Benchmark of the sparse sampling step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c3_t2i_4k] [--no-cpu-baseline]

A bench "step" is one whole generation of the workload: the prompt prefetch
and all sampling steps (every step runs the full hot path: KV append, step
attention, subset logits with confidence/argmax, unmask selection) over the
batch.  The generation is captured once as a HIP graph; W replays warm up,
then K replays are timed between device synchronisations.

value  = tokens unmasked per second = batch * generated length * K / seconds.
roofline: the dominant call is the step attention (k_attn_bf16, plus
          k_attn_combine on steps whose key range is split).  Its average
          duration comes from HIP events recorded around every call of an
          eager generation on the stream the kernels run on; `achieved`
          counts only algorithmic bytes (K and V of the visible cache once per
          (sequence, kv head), the transient table rows, Q rows, fp32 O) per
          call, against the 8 TB/s HBM peak (the step's arithmetic intensity
          is below the MFMA/HBM ridge).  The algorithmic MFMA fraction is
          reported alongside.  `traffic` is the counter-measured HBM bytes per
          call from the committed summary when it was taken on the current
          kernel sources, else null.
cpu_baseline: the CPU oracle (float64 NumPy) timed on this host on a bounded
          sample: sequence 0 of the same workload, from the prompt through as
          many sampling steps as fit in the time budget.

Training-form attention (the block-mask forward of the same method):
    python bench.py --block-attention [--workload train_t2i_4k|train_text]
        one JSON line: algorithmic TFLOP/s of mdm_block_attention against the
        bf16 MFMA peak, timed with HIP events over K launches, and the CPU
        oracle on a bounded sample.

Speed-up switches (page 1, ablation Table 6: cache prompt / cache res /
truncate res, and the plain bidirectional dense MDM):
    python bench.py --ablation [--ablation-steps K]
        one JSON line per setting: tokens unmasked/s of whole generations of
        the workload under that setting (HIP-graph replays, as above) and its
        speed-up over the setting with every switch off.

Profiling helpers (used to produce profiles/):
    python bench.py --profile-steps N         N eager generations, nothing else
    python bench.py --copy-calibration        one plain 1 GiB device copy
    python bench.py --traffic-summary FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
        reads rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv output of a
        --profile-steps 1 run and of a --copy-calibration run and writes the
        per-call HBM traffic of the step attention to profiles/.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E
METRIC = "tokens unmasked/sec at 4096-tok T2I; step-attn+logits % of MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_c3_t2i_4k_traffic.json")
CSRC = os.path.join(ROOT, "masked_discrete_diffusion_amd", "csrc")
ATTN_SOURCES = [os.path.join(CSRC, f) for f in ("attention.hip", "common.hpp", "kernels.hpp")]
COPY_BYTES = 1 << 30


ATT_REPEAT = 3          # back-to-back launches of each step's attention between its timing events


def attention_work(cfg, plan):
    """Algorithmic FLOPs and HBM bytes of every attention launch."""
    flops, nbytes = [], []
    d, H, Hkv, B, R = cfg.head_dim, cfg.n_heads, cfg.n_kv_heads, cfg.batch, cfg.n_registers
    esz = 2 if cfg.precision == "bf16" else 4
    S = cfg.prompt_len
    for st in plan:
        S += st.n_d
        s_tot = S + st.n_c + R
        pairs = st.n_d * S + (st.n_c + R) * s_tot
        flops.append(4.0 * d * pairs * H * B)
        n_q = st.n_d + st.n_c + R
        kv = 2.0 * S * Hkv * d * esz                      # cached K and V read once per (b, kv head)
        tables = (n_q * H * d + 2 * (st.n_c + R) * Hkv * d) * esz
        out = 4.0 * n_q * H * d
        nbytes.append(B * (kv + tables + out))
    return np.array(flops), np.array(nbytes)


def logits_work(cfg, plan):
    hidden, V = cfg.hidden, cfg.vocab
    esz = 2 if cfg.precision == "bf16" else 4
    flops = np.array([2.0 * cfg.batch * st.n_c * hidden * V for st in plan])
    nbytes = np.array([V * hidden * esz + cfg.batch * st.n_c * hidden * 4.0 for st in plan])
    return flops, nbytes


def device_reference(stream):
    """Context for the roofline fractions, measured on this device: compute
    units and name as the runtime reports them, and the bandwidth of a plain
    1 GiB device copy (bytes read + written over the HIP-event time of 10
    back-to-back copies), the HBM rate an ordinary stream attains here."""
    import torch
    props = torch.cuda.get_device_properties(0)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(2):
            dst.copy_(src)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        t1.record(stream)
    t1.synchronize()
    gbs = 10 * 2 * COPY_BYTES / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del src, dst
    return {"name": props.name, "compute_units": props.multi_processor_count,
            "copy_gbs": round(gbs, 1), "copy_frac_of_peak": round(gbs / HBM_PEAK_GBS, 3)}


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


TRAFFIC_WORKLOAD = "c3_t2i_4k"     # the workload the committed counter runs measured


def load_traffic(workload):
    """Counter-derived HBM bytes per attention call, if measured on this
    workload and these sources (None otherwise)."""
    if workload != TRAFFIC_WORKLOAD:
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attention_source_sha") != source_sha(ATTN_SOURCES):
        return None
    return t.get("hbm_bytes_per_call")


def _pmc_dispatches(d, counter):
    """{kernel name: {dispatch id: value}} for one counter of a rocprofv3 --pmc csv run."""
    import csv
    import glob
    tab = {}
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            per = tab.setdefault(r["Kernel_Name"], {})
            disp = int(r["Dispatch_Id"])
            per[disp] = per.get(disp, 0.0) + float(r["Counter_Value"])
    return tab


def traffic_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Per-call HBM traffic of the step attention from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what its counter reads for a plain copy
    of COPY_BYTES (which reads and writes COPY_BYTES)."""
    def largest(d, counter):
        vals = [v for per in _pmc_dispatches(d, counter).values() for v in per.values()]
        return max(vals) if vals else float("nan")

    def attention_kib(d, counter):
        tot, calls = 0.0, 0
        for name, per in _pmc_dispatches(d, counter).items():
            if "k_attn_bf16" in name or "k_attn_combine" in name:
                tot += sum(per.values())
                if "k_attn_bf16" in name:
                    calls += len(per)
        return tot, calls

    f_scale = COPY_BYTES / 1024.0 / largest(copy_fetch_dir, "FETCH_SIZE")
    w_scale = COPY_BYTES / 1024.0 / largest(copy_write_dir, "WRITE_SIZE")
    fk, calls = attention_kib(fetch_dir, "FETCH_SIZE")
    wk, _ = attention_kib(write_dir, "WRITE_SIZE")
    calls = max(calls, 1)
    t = {"attention_source_sha": source_sha(ATTN_SOURCES), "calls": calls,
         "fetch_kib_per_call": fk / calls, "write_kib_per_call": wk / calls,
         "copy_scale_fetch": f_scale, "copy_scale_write": w_scale,
         "hbm_bytes_per_call": (fk * f_scale + wk * w_scale) * 1024.0 / calls}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(t))


def _trace_durations(trace_dir):
    """{kernel name: [durations in ns in dispatch order]} from a --kernel-trace csv."""
    import csv
    import glob
    out = {}
    for f in sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)):
        rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            out.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def _short(name):
    n = name.replace("void ", "").replace("mdm::(anonymous namespace)::", "")
    return n.split("(")[0]


def pmc_summary(trace_dir, sq_dir, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload="c3_t2i_4k"):
    """Per-kernel counter summary of one eager generation (--profile-steps 1
    runs under rocprofv3 --pmc) with durations from a --kernel-trace run of
    two generations: MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over every
    SIMD's cycles of the traced duration at 2.4 GHz), VALU instructions, and
    HBM bytes (FETCH_SIZE / WRITE_SIZE scaled by a plain copy) against the
    algorithmic bytes of the same calls."""
    from mdm_inputs import get_config, make_workload
    from masked_discrete_diffusion_amd.sampler import make_plan
    cfg = get_config(workload)
    wl = make_workload(cfg, tables=False)
    plan = make_plan(wl)
    a_flops, a_bytes = attention_work(cfg, plan)
    l_flops, l_bytes = logits_work(cfg, plan)

    def largest(d, counter):
        vals = [v for per in _pmc_dispatches(d, counter).values() for v in per.values()]
        return max(vals)
    f_scale = COPY_BYTES / 1024.0 / largest(copy_fetch_dir, "FETCH_SIZE")
    w_scale = COPY_BYTES / 1024.0 / largest(copy_write_dir, "WRITE_SIZE")
    groups = {"step attention (k_attn_bf16, all variants)": "k_attn_bf16",
              "vocabulary screen (k_screen_bf16, all variants)": "k_screen_bf16",
              "wide vocabulary screen (k_screen_wide, all variants)": "k_screen_wide",
              "screen split reduce (k_screen_reduce)": "k_screen_reduce",
              "decision (k_decide)": "k_decide"}
    dur = _trace_durations(trace_dir)
    tabs = {c: _pmc_dispatches(d, c) for c, d in (("SQ_VALU_MFMA_BUSY_CYCLES", sq_dir), ("SQ_INSTS_VALU", sq_dir),
                                                  ("SQ_WAVES", sq_dir), ("FETCH_SIZE", fetch_dir),
                                                  ("WRITE_SIZE", write_dir))}
    lines = []
    for label, key in groups.items():
        ds = [v for n, vs in dur.items() if key in n for v in vs]
        n_calls = len(ds) // 2                       # two generations traced
        if not n_calls:
            continue
        mean_ns = sum(ds) / len(ds)
        per = {}
        for c, tab in tabs.items():
            vals = [v for n, pv in tab.items() if key in n for v in pv.values()]
            per[c] = sum(vals) / max(len(vals), 1)
        mfma = per["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * mean_ns * 2.4)
        hbm = per["FETCH_SIZE"] * f_scale * 1024 + per["WRITE_SIZE"] * w_scale * 1024
        if key == "k_attn_bf16":
            alg, fl = a_bytes.mean(), a_flops.mean()
        elif key in ("k_screen_bf16", "k_screen_wide"):
            alg, fl = l_bytes.mean(), l_flops.mean()
        else:
            alg, fl = float("nan"), float("nan")
        variants = sorted({_short(n) for n in dur if key in n})
        lines.append(f"{label}\n"
                     f"  variants                 {', '.join(variants)}\n"
                     f"  calls per generation     {n_calls}\n"
                     f"  mean duration            {mean_ns / 1e3:.2f} us (kernel trace)\n"
                     f"  MFMA busy                {mfma:.3f} of all SIMD cycles\n"
                     f"  VALU instructions        {per['SQ_INSTS_VALU']:.4g} per call ({per['SQ_WAVES']:.0f} waves)\n"
                     f"  HBM fetch + write        {hbm / 1e6:.2f} MB per call (FETCH_SIZE x{f_scale:.3f}, "
                     f"WRITE_SIZE x{w_scale:.3f})\n"
                     + (f"  algorithmic bytes        {alg / 1e6:.2f} MB per call (measured / algorithmic "
                        f"{hbm / alg:.2f})\n"
                        f"  algorithmic FLOP         {fl / 1e9:.2f} GFLOP per call = "
                        f"{fl / (mean_ns * 1e-9) / 1e12:.1f} TFLOP/s, {fl / (mean_ns * 1e-9) / 1e12 / MFMA_BF16_PEAK_TFLOPS:.3f}"
                        f" of the bf16 peak; {alg / (mean_ns * 1e-9) / 1e9:.0f} GB/s, "
                        f"{alg / (mean_ns * 1e-9) / 1e9 / HBM_PEAK_GBS:.3f} of 8 TB/s\n" if alg == alg else ""))
    text = "\n".join(lines)
    print(text)
    return text


def cpu_threads(n):
    """Context that caps the BLAS thread pools at n threads (n <= 0: no cap)."""
    import contextlib
    if n <= 0:
        return contextlib.nullcontext()
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=n)


def cpu_baseline(cfg, budget_s):
    """The oracle's whole generation of the workload's sequences 0, 1, ... (round
    robin), step by step, until budget_s seconds have passed."""
    from threadpoolctl import threadpool_info
    from mdm_inputs import make_workload
    from oracle.step import Model, SequenceOracle, select_all, select_by_confidence, step_candidates
    from oracle.logits import decide, subset_logits

    wl = make_workload(cfg)
    model = Model.from_workload(wl)
    t0 = time.perf_counter()
    tokens = steps = gens = 0
    b = 0
    while True:
        seq = SequenceOracle(model, wl.prompt_ids[b], wl.prompt_pos[b])
        seq.prefill()
        d = (np.empty(0, np.int64), np.empty(0, np.int64))
        remaining = {b: None}
        done = True
        for k in range(cfg.n_steps):
            c_pos = step_candidates(wl, k, b, remaining)
            out = seq.forward(d[0], d[1], c_pos)
            tok, conf32 = decide(subset_logits(out.h, model.w))[:2]
            if cfg.schedule == "semi_ar":
                sel, rem = select_by_confidence(c_pos, conf32, wl.semi_ar[k].n_select)
                remaining[b] = c_pos[rem]
            else:
                sel, _ = select_all(c_pos)
            seq.write_tokens(c_pos[sel], tok[sel])
            d = (tok[sel], c_pos[sel])
            tokens += int(np.size(c_pos[sel]))
            steps += 1
            if time.perf_counter() - t0 > budget_s:
                done = k + 1 == cfg.n_steps
                break
        gens += done
        b = (b + 1) % cfg.batch
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{cfg.name}: sequences taken in turn, each a prompt prefetch + its {cfg.n_steps} sampling "
                      f"steps; {gens} whole generations, {steps} steps, {tokens} tokens unmasked in {dt:.1f} s, "
                      f"float64 NumPy on {cpu}"}


def block_attention_pairs(blocks, m):
    """Visible (query, key) pairs of one sequence under the block rule, from
    the block sizes: a clean block i sees blocks j <= i, a masked block i
    sees itself and blocks j <= m."""
    ids, sizes = np.unique(blocks, return_counts=True)
    clean = ids <= m
    total = 0
    for i, sz in zip(ids, sizes):
        seen = sizes[ids <= i].sum() if i <= m else sizes[clean].sum() + sz
        total += int(sz) * int(seen)
    return total


def block_attention_bench(args):
    """Training-form attention (mdm_block_attention) on one training batch:
    W untimed launches, then K launches bracketed by HIP events on the stream
    they run on.  value = algorithmic TFLOP/s = 4 d H * visible pairs per
    launch / mean launch time (MFMA-bound: the contraction over a 64-key tile
    does 128 FLOP per byte of K and V read)."""
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    from mdm_inputs.training import get_train_config, make_train_attn_inputs

    cfg = get_train_config(args.workload if args.workload.startswith("train_") else "train_t2i_4k")
    inp = make_train_attn_inputs(cfg)
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    q, k, v = t(inp.q), t(inp.k), t(inp.v)
    blocks = torch.from_numpy(inp.blocks).to(dev)
    n_clean = torch.from_numpy(inp.n_clean).to(dev)
    shape = L.MdmBlockAttnShape(batch=cfg.batch, n_rows=cfg.n_rows, n_heads=cfg.n_heads,
                                n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim)
    ws_bytes = L.mdm_block_attention_workspace_bytes(shape)
    ws = torch.zeros(ws_bytes // 4 + 1, dtype=torch.int32, device=dev)
    out = torch.empty((cfg.batch, cfg.n_rows, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch():
        L.mdm_block_attention(shape, q, k, v, blocks, n_clean, out, ws, ws_bytes, stream.cuda_stream)

    print(f"[bench] {cfg.name}: batch {cfg.batch}, {cfg.n_rows} rows, inputs ready", file=sys.stderr, flush=True)
    if args.profile_steps:
        for _ in range(args.profile_steps):
            launch()
        torch.cuda.synchronize()
        print(f"[bench] profiled {args.profile_steps} launches", file=sys.stderr, flush=True)
        return
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        launch()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    pairs = sum(block_attention_pairs(inp.blocks[b], int(inp.n_clean[b])) for b in range(cfg.batch))
    flops = 4.0 * cfg.head_dim * cfg.n_heads * pairs
    nbytes = 2.0 * cfg.batch * cfg.n_rows * cfg.head_dim * (cfg.n_heads + 2 * cfg.n_kv_heads) \
        + 4.0 * cfg.batch * cfg.n_rows * cfg.n_heads * cfg.head_dim
    tflops = flops / (ms / 1e3) / 1e12
    res = {
        "metric": "training-form block-mask attention, algorithmic TFLOP/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "rows": cfg.n_rows, "prompt_tokens": cfg.prompt_len,
                   "generated_tokens": cfg.gen_len, "registers_per_masked_block": cfg.n_registers,
                   "clean_blocks": cfg.clean_blocks, "masked_blocks": cfg.masked_blocks,
                   "heads": cfg.n_heads, "kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "parallelism": "none"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "mdm_block_attention: k_tile_ranges + k_block_attn",
                     "visible_pairs_per_query_head": pairs, "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes,
                     "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        with cpu_threads(args.cpu_threads):
            res["cpu_baseline"] = block_attention_cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res))


def block_attention_cpu_baseline(inp, budget_s):
    """The oracle (float64 NumPy attention under the block mask) on sequence 0,
    one query head after another until the budget is spent."""
    from threadpoolctl import threadpool_info
    from mdm_inputs.generate import bf16_bits_to_f32
    from oracle.attention import attend
    from oracle.masks import block_mask

    cfg = inp.cfg
    blk = inp.blocks[0]
    m = int(inp.n_clean[0])
    G = cfg.n_heads // cfg.n_kv_heads
    f64 = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    t0 = time.perf_counter()
    vis = block_mask(blk, blk, m)
    heads = 0
    for h in range(cfg.n_heads):
        kvh = h // G
        attend(f64(inp.q[0][:, h:h + 1]), f64(inp.k[0][:, kvh:kvh + 1]), f64(inp.v[0][:, kvh:kvh + 1]), vis)
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * cfg.head_dim * heads * block_attention_pairs(blk, m)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"sequence 0 of {cfg.name}: {heads} of {cfg.n_heads} query heads "
                      f"({cfg.n_rows} rows each) in {dt:.1f} s, float64 NumPy"}


def library_gemm_bench(args):
    """Context for the vocabulary screen: the vendor GEMM (torch.matmul on
    bf16 operands, bf16 out) of the workload's logits products h W^T at the
    step sizes of its schedule, timed beside this library's whole logits call
    (screen + split reduce + proven decision) at the same row counts, both
    over 20 back-to-back calls between HIP events.  Not part of the product
    path; h is seeded N(0, 1)."""
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    from mdm_inputs import get_config, make_workload

    cfg = get_config(args.workload)
    wl = make_workload(cfg)
    run = SparseStepRunner(wl, device="cuda:0")
    ns = sorted({st.n_c for st in run.plan if st.n_c})
    picks = sorted({ns[0], ns[len(ns) // 4], ns[len(ns) // 2], ns[(3 * len(ns)) // 4], ns[-1]})
    w = torch.from_numpy(wl.w_vocab.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(7)
    reps = 20

    def timed(fn, stream):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    print(f"# {cfg.name}: logits products [M x {cfg.hidden}] x [{cfg.vocab} x {cfg.hidden}]^T")
    print("#    M  vendor GEMM (us)  TFLOP/s   this library's logits call (us)  TFLOP/s")
    for n_c in picks:
        M = cfg.batch * n_c
        h = torch.randn(M * cfg.hidden, generator=gen, device="cuda:0", dtype=torch.float32)
        hb = h.view(M, cfg.hidden).to(torch.bfloat16)
        t_lib = timed(lambda: torch.matmul(hb, w.t()), torch.cuda.current_stream())
        t_own = timed(lambda: L.mdm_subset_logits_confidence(run.ctx, h, n_c * cfg.hidden, n_c, run.conf, run.token,
                                                             None), run.stream)
        fl = 2.0 * M * cfg.hidden * cfg.vocab
        print(f"  {M:5d}  {t_lib:16.1f}  {fl / t_lib / 1e6:7.0f}   {t_own:31.1f}  {fl / t_own / 1e6:7.0f}",
              flush=True)
    L.mdm_device_status(run.ctx)
    run.close()


def ablation_bench(args):
    """Every setting of the speed-up switches on the workload, each timed as
    whole generations replayed from a HIP graph."""
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    from masked_discrete_diffusion_amd.ablation import ALL_SWITCHES, AblationRunner, switch_work
    from mdm_inputs import get_config, make_workload

    cfg = get_config(args.workload)
    wl = make_workload(cfg)
    print(f"[bench] {cfg.name}: switch settings, workload ready", file=sys.stderr, flush=True)
    base = None
    for sw in ALL_SWITCHES:
        run = AblationRunner(wl, sw, device="cuda:0")
        run.generate()
        torch.cuda.synchronize()
        L.mdm_device_status(run.ctx)
        graph = run.capture_graph()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.ablation_steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        L.mdm_device_status(run.ctx)
        value = cfg.batch * cfg.gen_len * args.ablation_steps / elapsed
        if base is None:
            base = value
        res = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
               "steps": args.ablation_steps, "warmup": args.warmup,
               "ms_per_step": round(elapsed / args.ablation_steps * 1e3, 4), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if cfg.precision == "bf16" else "fp32",
               "data": "synthetic",
               "config": {"workload": f"{cfg.name}/{sw.name}", "batch": cfg.batch, "prompt_tokens": cfg.prompt_len,
                          "image_tokens": cfg.gen_len, "sampling_steps": cfg.n_steps,
                          "registers": run.n_registers, "cache_prompt": sw.cache_prompt,
                          "cache_res": sw.cache_res, "truncate": sw.truncate,
                          "bidirectional": sw.bidirectional, "parallelism": "none"},
               "speedup_vs_all_off": round(value / base, 3)}
        att, head = switch_work(cfg, run.counts, sw)
        gen_s = elapsed / args.ablation_steps
        res["algorithmic_tflop_per_generation"] = {"attention": round(att / 1e12, 3), "head": round(head / 1e12, 3)}
        res["mfma_frac"] = round((att + head) / gen_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        print(json.dumps(res), flush=True)
        del graph
        run.close()
        del run
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3_t2i_4k")
    ap.add_argument("--layers", type=int, default=1,
                    help="attention layers (upper layers project the previous layer's outputs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="limit the CPU baseline's BLAS threads (0: as many as the host gives)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run only this many eager generations (for profilers) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain device copy of 1 GiB (counter calibration) and exit")
    ap.add_argument("--block-attention", action="store_true",
                    help="time the training-form block-mask attention (workload train_t2i_4k or train_text)")
    ap.add_argument("--ablation", action="store_true",
                    help="time every setting of the speed-up switches (cache prompt / cache res / truncate)")
    ap.add_argument("--ablation-steps", type=int, default=5)
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the vendor GEMM on the workload's logits products beside the logits call")
    ap.add_argument("--pmc-summary", nargs=6, metavar="DIR",
                    help="TRACE SQ FETCH WRITE COPY_FETCH COPY_WRITE: per-kernel counter summary (stdout)")
    ap.add_argument("--traffic-summary", nargs=4, metavar="DIR",
                    help="FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR: write the attention traffic summary")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              f"(sequences are independent and would shard across GPUs with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {COPY_BYTES} bytes", file=sys.stderr, flush=True)
        return
    if args.block_attention:
        block_attention_bench(args)
        return
    if args.library_gemm:
        library_gemm_bench(args)
        return
    if args.ablation:
        ablation_bench(args)
        return
    from masked_discrete_diffusion_amd import _lib as L
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    from mdm_inputs import get_config, make_workload

    cfg = get_config(args.workload)
    if args.layers != 1:
        cfg = cfg.replace(layers=args.layers)
    wl = make_workload(cfg)
    run = SparseStepRunner(wl, device="cuda:0")
    print(f"[bench] {cfg.name}: batch {cfg.batch}, {cfg.n_steps} steps, workload ready", file=sys.stderr, flush=True)

    if args.profile_steps:
        for _ in range(args.profile_steps):
            run.generate()
        torch.cuda.synchronize()
        L.mdm_device_status(run.ctx)
        print(f"[bench] profiled {args.profile_steps} eager generations", file=sys.stderr, flush=True)
        return

    run.generate()
    torch.cuda.synchronize()
    L.mdm_device_status(run.ctx)
    graph = run.capture_graph()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tokens = cfg.batch * cfg.gen_len * args.steps
    print(f"[bench] {args.steps} graph replays in {elapsed:.3f} s", file=sys.stderr, flush=True)

    # per-kernel durations: HIP events around every attention / logits launch of
    # eager generations, on the stream the kernels run on
    stream = run.stream
    n = len(run.plan)
    reps = 3
    att_ms = np.zeros(n)
    log_ms = np.zeros(n)
    proj_ms = np.zeros(n)
    up_att_ms = np.zeros(n)
    # each step's attention is launched ATT_REPEAT times back to back between
    # its two events (the call is idempotent): a lone launch between events also
    # times the dispatch of the kernel, which back-to-back launches (and the
    # graph replays) overlap with the previous kernel
    for _ in range(reps):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        evu = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(cfg.layers - 1)]
               for _ in range(n)]
        with torch.cuda.stream(stream):
            run.prefill()
        for k, st in enumerate(run.plan):
            if st.n_d:
                L.mdm_kv_append(run.ctx, run.d_tok[st.d_buf], run.d_pos[st.d_buf], st.n_d, st.n_d)
            c_ptr, c_stride = run._c_src(st)
            ev[k][0].record(stream)
            for _ in range(ATT_REPEAT):
                L.mdm_step_attention(run.ctx, run.d_tok[st.d_buf], run.d_pos[st.d_buf], st.n_d, st.n_d,
                                     c_ptr, c_stride, st.n_c, run.out)
            ev[k][1].record(stream)
            for li, layer in enumerate(range(2, cfg.layers + 1)):
                src, dst = run.outs[(layer - 2) % 2], run.outs[(layer - 1) % 2]
                evu[k][li][0].record(stream)
                L.mdm_layer_project(run.ctx, layer, src, 0, run.d_pos[st.d_buf], st.n_d, st.n_d, c_ptr, c_stride,
                                    st.n_c)
                evu[k][li][1].record(stream)
                L.mdm_layer_attention(run.ctx, layer, st.n_d, st.n_c, dst)
                evu[k][li][2].record(stream)
            n_q = st.n_d + st.n_c + cfg.n_registers
            h_ptr = run.out.data_ptr() + 4 * st.n_d * cfg.hidden
            ev[k][2].record(stream)
            L.mdm_subset_logits_confidence(run.ctx, h_ptr, n_q * cfg.hidden, st.n_c, run.conf, run.token, None)
            ev[k][3].record(stream)
            rem = run.rem[st.rem_out] if st.rem_out >= 0 else None
            L.mdm_unmask_select(run.ctx, c_ptr, c_stride, run.conf, run.token, st.n_c, st.n_sel, st.mode,
                                run.d_tok[st.out_buf], run.d_pos[st.out_buf], rem, run.seq_tokens)
        torch.cuda.synchronize()
        att_ms += np.array([e[0].elapsed_time(e[1]) for e in ev]) / ATT_REPEAT
        log_ms += np.array([e[2].elapsed_time(e[3]) for e in ev])
        proj_ms += np.array([sum(u[0].elapsed_time(u[1]) for u in eu) for eu in evu])
        up_att_ms += np.array([sum(u[1].elapsed_time(u[2]) for u in eu) for eu in evu])
    att_ms /= reps
    log_ms /= reps
    proj_ms /= reps
    up_att_ms /= reps
    L.mdm_device_status(run.ctx)

    a_flops, a_bytes = attention_work(cfg, run.plan)
    l_flops, l_bytes = logits_work(cfg, run.plan)
    att_s = att_ms.sum() / 1e3
    achieved = a_bytes.sum() / att_s / 1e9               # = mean algorithmic bytes per call / mean call time
    mfma_tflops = a_flops.sum() / att_s / 1e12
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if args.layers != 1 else load_traffic(cfg.name),
                "kernel": "mdm_step_attention: k_attn_bf16<128, pair | lag | quad> (+ k_attn_combine<128> on key-split steps)",
                "calls": n,
                "launches_per_event_pair": ATT_REPEAT,
                "avg_call_us": round(att_ms.mean() * 1e3, 2),
                "algorithmic_bytes_per_call": round(float(a_bytes.mean()), 0),
                "algorithmic_tflops": round(mfma_tflops, 2),
                "mfma_frac": round(mfma_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    if cfg.layers > 1 and proj_ms.sum() > att_ms.sum():
        # the upper layers' projection dominates: 2 M N hidden FLOP per call
        # (M = B n_q query rows, N = (H + 2 H_kv) d outputs), MFMA-bound
        n_up = cfg.layers - 1
        p_flops = np.array([2.0 * cfg.batch * (st.n_d + st.n_c + cfg.n_registers) * cfg.proj_rows * cfg.hidden
                            for st in run.plan]) * n_up
        p_s = proj_ms.sum() / 1e3
        p_tflops = p_flops.sum() / p_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(p_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(p_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "mdm_layer_project: k_pack + k_screen_bf16 | k_screen_wide (raw product, h hi + lo) + k_rope_scatter",
                    "calls": n * n_up, "avg_call_us": round(proj_ms.mean() / n_up * 1e3, 2),
                    "algorithmic_flops_per_call": round(float(p_flops.mean() / n_up), 0),
                    "first_layer_attention": roofline}
    # the logits call (screen, split reduce, decision): per step, the time the
    # roofline allows is the larger of its W + h stream at the HBM peak and its
    # product at the bf16 MFMA peak
    l_roof_s = np.maximum(l_bytes / (HBM_PEAK_GBS * 1e9), l_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    l_s = log_ms.sum() / 1e3
    logits_roofline = {"bound": "hbm below ~300 rows per step, mfma above (per step: the larger)",
                       "frac": round(float(l_roof_s.sum() / l_s), 4),
                       "roofline_ms": round(float(l_roof_s.sum() * 1e3), 4), "measured_ms": round(l_s * 1e3, 4),
                       "achieved_tflops": round(float(l_flops.sum() / l_s / 1e12), 2),
                       "achieved_gbs": round(float(l_bytes.sum() / l_s / 1e9), 1),
                       "avg_call_us": round(float(log_ms.mean() * 1e3), 2),
                       "kernel": "mdm_subset_logits_confidence: k_screen_bf16 | k_screen_wide (+ k_screen_reduce) + k_decide"}
    both_s = att_s + log_ms.sum() / 1e3
    step_frac = (a_flops.sum() + l_flops.sum()) / both_s / 1e12 / MFMA_BF16_PEAK_TFLOPS

    out = {
        "metric": METRIC,
        "value": round(tokens / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.precision == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "prompt_tokens": cfg.prompt_len,
                   "image_tokens": cfg.gen_len, "registers": cfg.n_registers, "sampling_steps": cfg.n_steps,
                   "heads": cfg.n_heads, "kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "vocab": cfg.vocab, "schedule": cfg.schedule, "order": cfg.order, "layers": cfg.layers,
                   "parallelism": "none"},
        "roofline": roofline,
        "logits_roofline": logits_roofline,
        "step_attn_logits_mfma_frac": round(step_frac, 4),
        "kernel_ms_per_generation": {"attention": round(att_ms.sum(), 4), "logits": round(log_ms.sum(), 4),
                                     **({"upper_projection": round(proj_ms.sum(), 4),
                                         "upper_attention": round(up_att_ms.sum(), 4)} if cfg.layers > 1 else {})},
    }
    out["device"] = device_reference(stream)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        with cpu_threads(args.cpu_threads):
            out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    run.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
