#!/usr/bin/env python3
"""Benchmark of folded-GQA decode attention (and Quest) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Prints ONE JSON line.  A "step" is one pass of the hot path over one batch of
synthetic inputs already resident in HBM.

* long_context (default): the long-context Quest GQA workload, B 8, Hq 32,
  Hkv 8, D 128, L 131072 (contiguous fp16 cache [8, 8, 131072, 128], 16
  planted pages per KV head).  The headline step is folded decode attention
  over the whole context with the step's K/V row appended at slot 131071
  (gqa_decode_attn: decode kernel + split merge); `value` is its KV GB/s and
  `roofline` its achieved rate.  Beside it: the Quest step at the same shape
  (K/V row and page-metadata append fused into the page scores, then top-K +
  attention over the 256 chosen pages + split merge), its stages, each
  kernel's fraction of peak, and its time over the dense step next to the
  byte model 1/S + B/L = 3/32.  Secondary legs (shorter runs): the EXAONE-
  shaped 30-layer step, the batched paged decode, the 32K Llama2-7B-shaped
  Quest step and one GQA layer.
* exaone30:    30 sequential decode-attention layers shaped like EXAONE 4.0
  1.2B (Hq 32, Hkv 8, D 64, fp16 cache [8, 4096, 64] per layer, 3000 valid
  keys, the step's K/V row appended at slot 2999 inside the attention
  kernel), captured once in a HIP graph and replayed per step.
* gqa1:        one layer, B 1, Hq 32, Hkv 8, D 64, 4096 keys.
* paged:       B 64, Hq 32, Hkv 8, D 128, page size 16, lengths U[1024, 32768].
* quest32k:    Llama2-7B-shaped, B 1, H 32, D 128, L 32768, budget 2048:
               page score + top-K + sparse attention (dense at the same
               shape is reported beside it).
* quest128k:   the Quest step of the long-context workload as the line.

Before every timed step a 1 GiB buffer is written (outside the step's events)
so that neither L2 nor the 256 MiB Infinity Cache holds the inputs.  A step
of at most three calls is launched directly on the stream (the host enqueues
it while the flush kernel runs); a longer step is captured once in a HIP graph
and replayed.  Step time is the median over the K steps of HIP events around
the step on the launching stream.  `value` is the KV bytes the step must read
divided by the step time.  One attention call runs the attention kernel and
the small split-merge kernel (or the score and top-K kernels), so both count.
The CPU baseline is the fp64 NumPy oracle on a bounded sample of the same
workload, timed on the host's cores (one worker thread per sampled unit, up
to the cores available, one BLAS thread each; median of 3 passes).
"""

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TENSORS = ("q", "k", "v", "seqlens", "k_new", "v_new")
FLUSH_BYTES = 1 << 30


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_context",
                    choices=["long_context", "exaone30", "gqa1", "paged", "quest32k",
                             "quest128k", "repeat_kv_ab", "quest_sweep", "multi_query"])
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the secondary workloads of the default line")
    ap.add_argument("--seed", type=int, default=2)
    return ap.parse_args()


# ---------------------------------------------------------------- workloads


class Stage:
    """Calls captured into one graph: `calls` launches of one C-ABI entry
    point (each running `kernels`), moving `bytes` algorithmic bytes."""

    def __init__(self, name, fns, nbytes, kernels):
        self.name = name
        self.fns = fns
        self.bytes = nbytes
        self.kernels = kernels


class Step:
    """One pass of the hot path: its stages and its byte accounting."""

    def __init__(self, name, config, kv_bytes, algo_bytes, stages):
        self.name = name
        self.config = config
        self.kv_bytes = kv_bytes            # K/V (and metadata) bytes the step must read
        self.algo_bytes = algo_bytes        # every byte the method must move
        self.stages = stages


def exaone30(da, torch, seed, dev):
    from decode_attention_folded_amd import workloads
    layers, hq, hkv, d, cap, L = 30, 32, 8, 64, 4096, 3000
    data = []
    for l in range(layers):
        c = workloads.device_dense(seed * 100 + l, 1, hq, hkv, d, cap, L, dev, with_new=True)
        c["out"] = torch.empty_like(c["q"])
        data.append(c)
    ws = da.Workspace(dev)
    seqlens = data[0]["seqlens"]

    def one(l):
        c = data[l]
        da.gqa_decode_attn(c["q"], c["k"], c["v"], seqlens, k_new=c["k_new"],
                           v_new=c["v_new"], out=c["out"], workspace=ws)

    kv_layer = 2 * hkv * L * d * 2
    per_launch = kv_layer + 2 * hkv * d * 2 + 2 * hq * d * 2   # KV + appended row + Q/out
    cfg = {"workload": "exaone1.2b_30layer_decode_hq32_hkv8_d64_cap4096_len3000_append",
           "layers": layers, "batch": 1, "num_q_heads": hq, "num_kv_heads": hkv,
           "head_dim": d, "capacity": cap, "valid_len": L, "dtype_cache": "fp16"}
    st = Stage("attention", [lambda l=l: one(l) for l in range(layers)], layers * per_launch,
               "decode_kernel + merge_kernel (gqa_decode_attn)")
    step = Step("exaone30", cfg, layers * kv_layer, layers * per_launch, [st])
    step.kernels_per_step = 2 * layers  # attention + split merge per layer
    return step, data


def gqa1(da, torch, seed, dev):
    from decode_attention_folded_amd import workloads
    hq, hkv, d, L = 32, 8, 64, 4096
    c = workloads.device_dense(seed, 1, hq, hkv, d, L, L, dev)
    c["out"] = torch.empty_like(c["q"])
    ws = da.Workspace(dev)

    def one():
        da.gqa_decode_attn(c["q"], c["k"], c["v"], c["seqlens"], out=c["out"], workspace=ws)

    kv = 2 * hkv * L * d * 2
    cfg = {"workload": "gqa_decode_b1_hq32_hkv8_d64_ctx4096", "batch": 1, "num_q_heads": hq,
           "num_kv_heads": hkv, "head_dim": d, "valid_len": L}
    st = Stage("attention", [one], kv + 2 * hq * d * 2,
               "decode_kernel + merge_kernel (gqa_decode_attn)")
    step = Step("gqa1", cfg, kv, kv + 2 * hq * d * 2, [st])
    step.kernels_per_step = 2
    return step, c


def paged(da, torch, seed, dev):
    import numpy as np
    from decode_attention_folded_amd import workloads
    b, hq, hkv, d, s, mp = 64, 32, 8, 128, 16, 2048
    lens = workloads.draw_seqlens(3, b, 1024, 32768)
    c = workloads.device_paged(seed, b, hq, hkv, d, s, mp, lens, dev)
    c["out"] = torch.empty_like(c["q"])
    ws = da.Workspace(dev)

    def one():
        da.gqa_decode_attn(c["q"], c["k"], c["v"], c["seqlens"], page_table=c["page_table"],
                           page_size=s, out=c["out"], workspace=ws)

    kv = int(2 * hkv * d * 2 * int(np.sum(lens)))
    per = kv + 2 * b * hq * d * 2 + b * mp * 4
    cfg = {"workload": "paged_gqa_decode_b64_hq32_hkv8_d128_s16_len1k-32k", "batch": b,
           "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d, "page_size": s,
           "total_tokens": int(np.sum(lens))}
    st = Stage("attention", [one], per, "paged_persist_kernel + merge_kernel (gqa_decode_attn)")
    return Step("paged", cfg, kv, per, [st]), c


def quest(da, torch, seed, dev, long_ctx):
    from decode_attention_folded_amd import workloads
    if long_ctx:
        b, hq, hkv, d, L, s, budget, plant = 8, 32, 8, 128, 131072, 16, 4096, 16
        name = "quest_gqa_b8_hq32_hkv8_d128_L131072_s16_budget4096_append"
    else:
        b, hq, hkv, d, L, s, budget, plant = 1, 32, 32, 128, 32768, 16, 2048, 8
        name = "quest_llama2-7b_b1_h32_d128_L32768_s16_budget2048"
    c = workloads.device_dense(seed, b, hq, hkv, d, L, L, dev, plant_pages=plant,
                               plant_page_size=s, with_new=long_ctx)
    P = L // s
    meta = torch.zeros((b, hkv, P, 2, d), dtype=torch.float16, device=dev)
    # the metadata state before the step: with an append, the step's token is
    # key L - 1, so the state covers keys [0, L - 1) (the slot the append
    # overwrites is not a key yet)
    built = c["seqlens"] - 1 if long_ctx else c["seqlens"]
    da.quest_meta_append(c["k"], c["v"], meta, built, n_new=L, page_size=s)
    k_sel = budget // s
    idx = torch.empty((b, hkv, k_sel), dtype=torch.int32, device=dev)
    scores = torch.empty((b, hkv, P), dtype=torch.float32, device=dev)
    out = torch.empty_like(c["q"])
    dense_out = torch.empty_like(c["q"])
    ws = da.Workspace(dev)
    dws = da.Workspace(dev)

    def append():
        da.quest_meta_append(c["k"], c["v"], meta, c["seqlens"], 1, page_size=s,
                             k_new=c["k_new"], v_new=c["v_new"])

    def append_select():   # the step's append fused into the score launch
        da.quest_append_score_topk(c["q"], c["k"], c["v"], meta, c["seqlens"], c["k_new"],
                                   c["v_new"], page_size=s, budget_tokens=budget,
                                   page_idx=idx, page_scores=scores)

    def select():
        da.quest_page_score_topk(c["q"], meta, c["seqlens"], page_size=s, budget_tokens=budget,
                                 page_idx=idx, page_scores=scores)

    def attend():
        da.quest_sparse_decode_attn(c["q"], c["k"], c["v"], c["seqlens"], idx,
                                    budget_tokens=budget, page_size=s, out=out, workspace=ws)

    # The step as launched by default: scores (with the step's append at 128K),
    # then the top-K fused into the selected-page attention.
    def append_score():
        da.quest_append_score_topk(c["q"], c["k"], c["v"], meta, c["seqlens"], c["k_new"],
                                   c["v_new"], page_size=s, budget_tokens=budget,
                                   page_scores=scores, select=False)

    def score():
        da.quest_page_score_topk(c["q"], meta, c["seqlens"], page_size=s, budget_tokens=budget,
                                 page_scores=scores, select=False)

    def select_attend():
        da.quest_select_sparse_decode_attn(c["q"], c["k"], c["v"], c["seqlens"], scores,
                                           budget_tokens=budget, page_size=s, page_idx=idx,
                                           out=out, workspace=ws)

    def dense():
        da.gqa_decode_attn(c["q"], c["k"], c["v"], c["seqlens"], out=dense_out, workspace=dws)

    def dense_append():   # dense decode attention with the step's K/V row appended
        da.gqa_decode_attn(c["q"], c["k"], c["v"], c["seqlens"], k_new=c["k_new"],
                           v_new=c["v_new"], out=dense_out, workspace=dws)

    units = b * hkv
    meta_bytes = units * P * 2 * d * 2
    sel_bytes = units * k_sel * s * 2 * d * 2
    dense_bytes = units * L * 2 * d * 2
    kv_bytes = meta_bytes + sel_bytes
    qo_bytes = 2 * b * hq * d * 2
    # scores written by the score stage and read by the selecting attention;
    # the chosen pages written by it
    score_bytes = meta_bytes + units * P * 4 + b * hq * d * 2
    attend_bytes = sel_bytes + qo_bytes + units * P * 4 + units * k_sel * 4
    # append: the new K/V row (read + write) and the touched page's min/max
    append_bytes = units * (2 * 2 * d * 2 + 2 * 2 * d * 2)
    algo = score_bytes + attend_bytes + (append_bytes if long_ctx else 0)
    if long_ctx:
        stages = [Stage("append_score", [append_score], score_bytes + append_bytes,
                        "page_score_kernel with the append (quest_append_score_topk, "
                        "scores only)")]
    else:
        stages = [Stage("score", [score], score_bytes,
                        "page_score_kernel (quest_page_score_topk, scores only)")]
    stages.append(Stage("select_sparse_attention", [select_attend], attend_bytes,
                        "decode_kernel selecting its pages + merge_kernel "
                        "(quest_select_sparse_decode_attn)"))
    cfg = {"workload": name, "batch": b, "num_q_heads": hq, "num_kv_heads": hkv,
           "head_dim": d, "seq_len": L, "page_size": s, "budget_tokens": budget,
           "k_pages": k_sel}
    st = Step("quest128k" if long_ctx else "quest32k", cfg, kv_bytes, algo, stages)
    st.kernels_per_step = 3  # page scores, selecting attention, split merge
    st.dense_fn = dense_append if long_ctx else dense
    c["quest_out"], c["dense_out"], c["idx"], c["scores"], c["meta"] = (out, dense_out, idx,
                                                                        scores, meta)
    # the same step with the top-K as its own launch, and (128K) with the
    # append as its own launch too, for comparison
    st.variants = {"separate_topk": [append_select if long_ctx else select, attend]}
    if long_ctx:
        st.variants["separate_append"] = [append, select, attend]
    st.dense_bytes = dense_bytes
    # the dense step's algorithmic bytes: K/V of every valid key, the appended
    # row (read from k_new/v_new and written), Q and the output
    st.dense_algo_bytes = dense_bytes + (units * 2 * 2 * d * 2 if long_ctx else 0) + qo_bytes
    st.byte_model = {"meta_bytes": meta_bytes, "selected_bytes": sel_bytes,
                     "dense_bytes": dense_bytes,
                     "ratio_model": 1.0 / s + budget / L}
    return st, c


# ---------------------------------------------------------------- timing


def capture(torch, fns):
    """Capture the launches of one step into a HIP graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for f in fns:
                f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


DIRECT_MAX_CALLS = 3   # steps of at most this many calls are launched directly


def time_direct(torch, fns, steps, warmup, flush):
    """Launch the calls directly on the stream, warmup + steps times, with a
    cache flush before each step (outside the events).  The host enqueues the
    calls while the flush kernel (about 150 us) runs, so neither host launch
    overhead nor a graph launch sits between the events.  Returns per-step ms."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    out = []
    for i in range(warmup + steps):
        if flush is not None:
            flush.zero_()
        a.record()
        for f in fns:
            f()
        b.record()
        torch.cuda.synchronize()
        if i >= warmup:
            out.append(a.elapsed_time(b))
    return out


def time_calls(torch, fns, steps, warmup, flush):
    """Per-step ms of the calls `fns`: launched directly when there are at most
    DIRECT_MAX_CALLS of them, otherwise replayed from one captured graph."""
    if len(fns) <= DIRECT_MAX_CALLS:
        return time_direct(torch, fns, steps, warmup, flush), "direct"
    return time_stages(torch, [capture(torch, fns)], steps, warmup, flush)[0], "graph"


def time_stages(torch, graphs, steps, warmup, flush):
    """Replay the stage graphs back to back, warmup + steps times, with a cache
    flush before each step (outside the events) and HIP events between the
    stages on the launching stream.  Returns per-step ms and per-stage ms."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(graphs) + 1)]
    step_ms, stage_ms = [], [[] for _ in graphs]
    for i in range(warmup + steps):
        if flush is not None:
            flush.zero_()
        ev[0].record()
        for j, g in enumerate(graphs):
            g.replay()
            ev[j + 1].record()
        torch.cuda.synchronize()
        if i >= warmup:
            step_ms.append(ev[0].elapsed_time(ev[-1]))
            for j in range(len(graphs)):
                stage_ms[j].append(ev[j].elapsed_time(ev[j + 1]))
    return step_ms, stage_ms


def cpu_baseline(step, data, seed):
    """The fp64 oracle on a bounded sample of a secondary workload, in one
    thread with one BLAS thread (the default line's baseline is
    long_context_cpu_baseline)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        return _cpu_baseline(step, data)


def _cpu_baseline(step, data):
    import numpy as np
    import oracle
    from oracle import quest as oquest
    t0 = time.perf_counter()
    sample = ""
    bytes_done = 0
    reps = 0
    if step.name == "exaone30":
        host = [{k: v.cpu().numpy() for k, v in c.items() if k in TENSORS} for c in data]
        t0 = time.perf_counter()
        while True:   # whole steps until about 10 s of CPU work
            for c in host:
                k2, v2 = oracle.append_kv(c["k"], c["v"], c["seqlens"], c["k_new"], c["v_new"])
                oracle.decode_attention(c["q"], k2, v2, c["seqlens"], 1 / 8.0)
            reps += 1
            bytes_done += step.kv_bytes
            if time.perf_counter() - t0 > 10.0 or reps >= 30:
                break
        sample = f"{reps} full 30-layer step(s) (append + repeat_kv attention, fp64)"
    elif step.name in ("gqa1",):
        c = {k: v.cpu().numpy() for k, v in data.items() if k in TENSORS}
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 10.0 and reps < 20:
            oracle.decode_attention(c["q"], c["k"], c["v"], c["seqlens"], 1 / 8.0)
            reps += 1
            bytes_done += step.kv_bytes
        sample = f"{reps} full step(s)"
    elif step.name == "paged":
        # a few sequences of the batch
        lens = data["seqlens_host"]
        table = data["page_table_host"]
        t0 = None
        for b in range(4):
            n = (int(lens[b]) + 15) // 16
            pages = table[b, :n]
            k = data["k"][torch_index(pages)].cpu().numpy()
            v = data["v"][torch_index(pages)].cpu().numpy()
            q = data["q"][b:b + 1].cpu().numpy()
            kc = k.transpose(1, 0, 2, 3).reshape(1, k.shape[1], n * 16, k.shape[3])
            vc = v.transpose(1, 0, 2, 3).reshape(1, v.shape[1], n * 16, v.shape[3])
            s0 = time.perf_counter()
            oracle.decode_attention(q, kc, vc, [int(lens[b])], 1 / math.sqrt(128))
            t0 = (t0 or 0.0) + time.perf_counter() - s0
            bytes_done += 2 * 8 * int(lens[b]) * 128 * 2
        sample = "4 of the 64 sequences"
        return _baseline(bytes_done, t0, sample)
    else:
        # Quest: one or two (b, kv) units through every step of the method
        b_units = [(0, 0), (0, 1)]
        c = data
        S = step.config["page_size"]
        budget = step.config["budget_tokens"]
        L = step.config["seq_len"]
        G = step.config["num_q_heads"] // step.config["num_kv_heads"]
        elapsed = 0.0
        for (b, kv) in b_units:
            q = c["q"][b:b + 1, kv * G:(kv + 1) * G].cpu().numpy()
            k = c["k"][b:b + 1, kv:kv + 1].cpu().numpy()
            v = c["v"][b:b + 1, kv:kv + 1].cpu().numpy()
            lens = np.array([L], np.int32)
            s0 = time.perf_counter()
            meta = oquest.build_metadata(k, lens, S, L // S)
            u = oquest.page_scores(q, meta, lens, S)
            idx = oquest.select_pages(u, lens, S, budget // S)
            oquest.sparse_decode_attention(q, k, v, lens, idx, S, 1 / math.sqrt(128))
            elapsed += time.perf_counter() - s0
            bytes_done += step.kv_bytes // (step.config["batch"] * step.config["num_kv_heads"])
        sample = f"{len(b_units)} (b, kv) units, metadata build + score + top-K + sparse attention"
        return _baseline(bytes_done, elapsed, sample)
    elapsed = time.perf_counter() - t0
    return _baseline(bytes_done, elapsed, sample)


def torch_index(pages):
    import torch
    return torch.from_numpy(pages.astype("int64"))


def _baseline(bytes_done, elapsed, sample):
    # these workloads' oracle legs run in one thread with one BLAS thread
    return {"value": round(bytes_done / elapsed / 1e9, 6), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": sample, "seconds": round(elapsed, 3),
            "host_cores": len(os.sched_getaffinity(0)), "blas_threads": 1}


def _code_only(text):
    """Source text without comments and with whitespace collapsed, so that
    editing a comment does not change the digest."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(root=None):
    """Hash of the kernel sources' code (comments and whitespace ignored): the
    committed counter summary is used only while it was taken on these exact
    kernels."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(root or ROOT, "decode_attention_folded_amd", "csrc")
    for name in ("attention_impl.h", "decode_kernel.hip", "decode_select.hip", "topk.h",
                 "quest_kernels.hip", "device_common.h", "kernels.h"):
        with open(os.path.join(csrc, name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload, stage):
    """HBM bytes per call of one stage (its kernels summed) from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE runs, scaled by a
    reference copy), or None if missing or taken on different kernel
    sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
    try:
        text = open(path).read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None
    entry = data.get("workloads", {}).get(workload)
    if not entry or data.get("kernel_source_digest") != kernel_source_digest():
        return None
    return entry.get("stages", {}).get(stage, {}).get("bytes_per_call")


def measure(torch, da, dev, step, steps, warmup, flush):
    """Time the step: a step of at most DIRECT_MAX_CALLS calls is launched
    directly on the stream after the cache flush (HIP events around it);
    longer steps are captured once in a HIP graph and replayed (a graph
    launch costs about 12 us before its first kernel, which a long step
    amortises and a short one would not).  With several stages, each stage is
    timed the same way to find the dominant one; a single-stage step is its
    own dominant stage, timed in the same loop."""
    for st in step.stages:       # eager warm-up allocates every workspace first
        for f in st.fns:
            f()
    if hasattr(step, "dense_fn"):
        step.dense_fn()
    torch.cuda.synchronize()

    def run(fns, reps, warm):
        return time_calls(torch, fns, reps, warm, flush)

    all_fns = [f for st in step.stages for f in st.fns]
    t_wall0 = time.perf_counter()
    step_ms, how = run(all_fns, steps, warmup)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms = statistics.median(step_ms)
    if len(step.stages) == 1:
        med = [ms]
    else:
        med = []
        for st in step.stages:
            st_ms = run(st.fns, max(10, steps // 2), 2)[0]
            med.append(statistics.median(st_ms))
            if os.environ.get("BENCH_BOTH_LAUNCH_MODES"):
                print(st.name, [round(x * 1e3, 2) for x in st_ms], file=sys.stderr)
    dom = max(range(len(med)), key=lambda j: med[j])
    dst = step.stages[dom]
    res = {
        "ms": ms,
        "launch": how,
        "gbs": step.kv_bytes / (ms * 1e-3) / 1e9,
        "dominant": dst,
        "stage_ms": med[dom],
        "achieved": dst.bytes / (med[dom] * 1e-3) / 1e9,
        "us_per_step": round(ms * 1e3, 3),
        "us_p10": round(sorted(step_ms)[len(step_ms) // 10] * 1e3, 3),
        "us_p90": round(sorted(step_ms)[(len(step_ms) * 9) // 10] * 1e3, 3),
        "timed_wall_s": round(t_wall, 3),
        "stage_us": {st.name: round(m * 1e3, 3) for st, m in zip(step.stages, med)},
    }
    for name, fns in getattr(step, "variants", {}).items():
        res["step_us_" + name] = round(statistics.median(run(fns, steps, 2)[0]) * 1e3, 3)
    if hasattr(step, "dense_fn"):
        dense_ms = statistics.median(run([step.dense_fn], max(10, steps // 2), 2)[0])
        res["dense_same_shape_us"] = round(dense_ms * 1e3, 3)
        res["dense_same_shape_gbs"] = round(step.dense_bytes / (dense_ms * 1e-3) / 1e9, 1)
        res["dense_same_shape_pct_peak"] = round(
            100 * step.dense_bytes / (dense_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)
        res["quest_over_dense_time"] = round(ms / dense_ms, 4)
        res["byte_model"] = step.byte_model
    if os.environ.get("BENCH_BOTH_LAUNCH_MODES"):
        g = capture(torch, all_fns)
        res["us_per_step_graph"] = round(
            statistics.median(time_stages(torch, [g], steps, warmup, flush)[0]) * 1e3, 3)
    return res


def repeat_kv_ab(da, torch, seed, dev, steps, warmup, flush):
    """The fold against the materialised repeat_kv path ([CoreML-GQA] section
    4's comparison) at the single-layer, 30-layer EXAONE-shaped and batched
    paged shapes.  Materialised = gqa_repeat_kv (each KV head copied to its G
    query heads) + the same attention kernel at G = 1.  Both sides read the
    same valid rows and skip the append (the materialised side has no
    separate append path)."""
    from decode_attention_folded_amd import workloads
    import numpy as np

    def timed(fns, reps):
        return statistics.median(time_calls(torch, fns, reps, 2, flush)[0]) * 1e3

    out = {}
    cases = []
    # single layer and the 30-layer step (B=1, Hq=32, Hkv=8, D=64)
    for name, layers, L, cap in (("gqa_layer_ctx4096", 1, 4096, 4096),
                                 ("exaone_30_layers_len3000", 30, 3000, 4096)):
        data = [workloads.device_dense(seed * 100 + l, 1, 32, 8, 64, cap, L, dev)
                for l in range(layers)]
        for c in data:
            c["kr"] = torch.empty((1, 32, cap, 64), dtype=torch.float16, device=dev)
            c["vr"] = torch.empty_like(c["kr"])
            c["out"] = torch.empty_like(c["q"])
        kv_bytes = layers * 2 * 8 * L * 64 * 2
        cases.append((name, data, None, 16, kv_bytes, 4))
    # batched paged decode (B=64, Hq=32, Hkv=8, D=128, S=16, U[1K, 32K])
    lens = workloads.draw_seqlens(3, 64, 1024, 32768)
    pc = workloads.device_paged(seed, 64, 32, 8, 128, 16, 2048, lens, dev)
    pc["kr"] = torch.empty((64, 32, 2048 * 16, 128), dtype=torch.float16, device=dev)
    pc["vr"] = torch.empty_like(pc["kr"])
    pc["out"] = torch.empty_like(pc["q"])
    cases.append(("paged_b64_len1k-32k", [pc], pc["page_table"], 16,
                  int(2 * 8 * 128 * 2 * int(np.sum(lens))), 4))
    for name, data, table, s, kv_bytes, g in cases:
        ws = da.Workspace(dev)
        fold = [lambda c=c: da.gqa_decode_attn(c["q"], c["k"], c["v"], c["seqlens"],
                                               page_table=table, page_size=s, out=c["out"],
                                               workspace=ws) for c in data]
        copy = [lambda c=c: da.gqa_repeat_kv(c["k"], c["v"], c["seqlens"], 32, page_table=table,
                                             page_size=s, k_out=c["kr"], v_out=c["vr"])
                for c in data]
        attn1 = [lambda c=c: da.gqa_decode_attn(c["q"], c["kr"], c["vr"], c["seqlens"],
                                                out=c["out"], workspace=ws) for c in data]
        for f in fold + copy + attn1:
            f()
        torch.cuda.synchronize()
        reps = max(5, steps // 2) if name.startswith("paged") else steps
        t_fold = timed(fold, reps)
        t_copy = timed(copy, reps)
        t_attn1 = timed(attn1, reps)
        t_both = timed(copy + attn1, reps)
        out[name] = {
            "fold_us": round(t_fold, 3),
            "materialised_us": round(t_both, 3),
            "repeat_kv_copy_us": round(t_copy, 3),
            "attention_g1_us": round(t_attn1, 3),
            "materialised_over_fold": round(t_both / t_fold, 3),
            "kv_bytes": kv_bytes,
            "copy_bytes": kv_bytes * (1 + g),
            "copy_gbs": round(kv_bytes * (1 + g) / (t_copy * 1e-6) / 1e9, 1),
            "byte_model_materialised_over_fold": 1 + 2 * g,
        }
        for c in data:
            del c["kr"], c["vr"]
        del data
        torch.cuda.empty_cache()
    return out


def multi_query(da, torch, seed, dev, steps, warmup, flush):
    """The fold with q_len > 1 query positions per head (group and sequence
    axes merged, causal alignment per row): the K/V bytes of a step stay the
    same while the rows per KV head grow from G to G * q_len."""
    from decode_attention_folded_amd import workloads

    def timed(fns, reps):
        return statistics.median(time_calls(torch, fns, reps, 2, flush)[0]) * 1e3

    out = {}
    shapes = (("exaone_30_layers_len3000", 30, 1, 32, 8, 64, 4096, 3000, (1, 2)),
              ("dense_b1_h32_g1_d128_L32768", 1, 1, 32, 32, 128, 32768, 32768, (1, 2, 4, 8)),
              ("dense_b8_hq32_hkv8_d128_L131072", 1, 8, 32, 8, 128, 131072, 131072, (1, 2)))
    for name, layers, b, hq, hkv, d, cap, L, qlens in shapes:
        data = [workloads.device_dense(seed * 100 + l, b, hq, hkv, d, cap, L, dev)
                for l in range(layers)]
        ws = da.Workspace(dev)
        kv_bytes = layers * b * hkv * L * 2 * d * 2
        res = {}
        for lq in qlens:
            qs = [torch.randn((b, hq, lq, d), device=dev).to(torch.float16) for _ in data]
            outs = [torch.empty_like(q) for q in qs]
            fns = [lambda c=c, q=q, o=o: da.gqa_decode_attn_multi(q, c["k"], c["v"], c["seqlens"],
                                                                  out=o, workspace=ws)
                   for c, q, o in zip(data, qs, outs)]
            for f in fns:
                f()
            torch.cuda.synchronize()
            us = timed(fns, steps if L < 100000 else max(10, steps // 2))
            res[f"q_len_{lq}"] = {"rows_per_kv_head": hq // hkv * lq, "step_us": round(us, 3),
                                  "kv_gbs": round(kv_bytes / (us * 1e-6) / 1e9, 1)}
        out[name] = res
        del data
        torch.cuda.empty_cache()
    return out


def quest_sweep(da, torch, seed, dev, steps, warmup, flush):
    """Quest page-size sweep at the Llama2-7B shape (B=1, H=32, D=128,
    L=32768) for S in {8, 16, 32, 64}, at a fixed token budget (2048) and at
    a fixed page count (K=128), against the byte model 1/S + B/L and dense
    attention ([Quest-review], "is page size 16 always optimal"); and a
    32-layer stack of that shape whose first two layers stay dense (the
    paper's layer policy the review cites) against 32 dense layers."""
    from decode_attention_folded_amd import workloads
    import numpy as np
    b, h, d, L = 1, 32, 128, 32768

    def timed(fns, reps):
        return statistics.median(time_calls(torch, fns, reps, 2, flush)[0]) * 1e3

    c = workloads.device_dense(seed, b, h, h, d, L, L, dev, plant_pages=8, plant_page_size=16)
    planted = c["planted"]
    ws = da.Workspace(dev)
    out = torch.empty_like(c["q"])
    dense_us = timed([lambda: da.gqa_decode_attn(c["q"], c["k"], c["v"], c["seqlens"], out=out,
                                                 workspace=ws)], steps)
    dense_bytes = b * h * L * 2 * d * 2
    sweep = {}
    for S in (8, 16, 32, 64):
        P = L // S
        meta = torch.zeros((b, h, P, 2, d), dtype=torch.float16, device=dev)
        da.quest_meta_append(c["k"], c["v"], meta, c["seqlens"], n_new=L, page_size=S)
        for mode, budget in (("fixed_budget_2048", 2048), ("fixed_k_128", 128 * S)):
            kp = budget // S
            idx = torch.empty((b, h, kp), dtype=torch.int32, device=dev)
            scores = torch.empty((b, h, P), dtype=torch.float32, device=dev)
            # the Quest step as launched by default: scores, then the top-K
            # fused into the selected-page attention
            fns = [lambda: da.quest_page_score_topk(c["q"], meta, c["seqlens"], page_size=S,
                                                    budget_tokens=budget, page_scores=scores,
                                                    select=False),
                   lambda: da.quest_select_sparse_decode_attn(c["q"], c["k"], c["v"], c["seqlens"],
                                                              scores, budget_tokens=budget,
                                                              page_size=S, page_idx=idx,
                                                              out=out, workspace=ws)]
            for f in fns:
                f()
            torch.cuda.synchronize()
            us = timed(fns, steps)
            # planted 16-token blocks covered by the chosen pages (a statistic)
            sel = idx.cpu().numpy()
            hit = tot = 0
            for (bb, hh), pages in planted.items():
                chosen = set(int(p) for p in sel[bb, hh] if p >= 0)
                for p16 in pages:
                    toks = range(16 * p16, 16 * p16 + 16)
                    hit += sum(1 for t in toks if t // S in chosen)
                    tot += 16
            model = 1.0 / S + budget / L
            sweep[f"S{S}_{mode}"] = {
                "page_size": S, "budget_tokens": budget, "k_pages": kp,
                "step_us": round(us, 3), "over_dense_time": round(us / dense_us, 4),
                "byte_model_ratio": round(model, 5),
                "bytes": int(dense_bytes * model),
                "gbs": round(dense_bytes * model / (us * 1e-6) / 1e9, 1),
                "planted_token_recall": round(hit / tot, 4),
            }
        del meta
        torch.cuda.empty_cache()
    del c
    torch.cuda.empty_cache()

    # 32 layers of the same shape: all dense, or two dense + 30 Quest (S=16,
    # budget 2048) layers
    layers = []
    for l in range(32):
        cl = workloads.device_dense(seed * 1000 + l, b, h, h, d, L, L, dev)
        cl["out"] = torch.empty_like(cl["q"])
        if l >= 2:
            cl["meta"] = torch.zeros((b, h, L // 16, 2, d), dtype=torch.float16, device=dev)
            da.quest_meta_append(cl["k"], cl["v"], cl["meta"], cl["seqlens"], n_new=L,
                                 page_size=16)
            cl["idx"] = torch.empty((b, h, 128), dtype=torch.int32, device=dev)
            cl["scores"] = torch.empty((b, h, L // 16), dtype=torch.float32, device=dev)
        layers.append(cl)

    def dense_layer(cl):
        da.gqa_decode_attn(cl["q"], cl["k"], cl["v"], cl["seqlens"], out=cl["out"], workspace=ws)

    def quest_layer(cl):
        da.quest_page_score_topk(cl["q"], cl["meta"], cl["seqlens"], page_size=16,
                                 budget_tokens=2048, page_scores=cl["scores"], select=False)
        da.quest_select_sparse_decode_attn(cl["q"], cl["k"], cl["v"], cl["seqlens"], cl["scores"],
                                           budget_tokens=2048, page_size=16, page_idx=cl["idx"],
                                           out=cl["out"], workspace=ws)

    all_dense = [lambda cl=cl: dense_layer(cl) for cl in layers]
    policy = [lambda cl=cl, l=l: dense_layer(cl) if l < 2 else quest_layer(cl)
              for l, cl in enumerate(layers)]
    for f in all_dense + policy:
        f()
    torch.cuda.synchronize()
    reps = max(5, steps // 5)
    t_dense = timed(all_dense, reps)
    t_policy = timed(policy, reps)
    stack = {"layers": 32, "dense_layers": 2, "page_size": 16, "budget_tokens": 2048,
             "all_dense_us": round(t_dense, 3), "two_dense_then_quest_us": round(t_policy, 3),
             "ratio": round(t_policy / t_dense, 4),
             "byte_model_ratio": round((2 + 30 * (1 / 16 + 2048 / L)) / 32, 5)}
    del layers
    torch.cuda.empty_cache()
    return {"dense_us": round(dense_us, 3), "dense_gbs": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
            "sweep": sweep, "stack_32_layers": stack}


def sample_units(batch, hkv, n):
    """(b, kv) units spread over the batch and the KV heads."""
    units = []
    for i in range(n):
        b = i % batch
        units.append((b, (3 * i + 1 + i // batch) % hkv))
    return units


def host_threads():
    """Cores this process may run on, and the BLAS threads NumPy would use."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"), default=1)
    except ImportError:
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return cores, blas


def long_context_cpu_baseline(step, c, units, reps=3):
    """The fp64 oracle on sampled (b, kv) units of the long-context workload,
    and the GPU's results on those units checked against it.

    One oracle step per unit: the K/V row append and repeat_kv attention over
    the whole context (the dense step); and the Quest step: metadata update
    for the new key, page scores, top-K, attention over the chosen pages.  The
    units run in parallel worker threads (NumPy releases the GIL in its array
    loops), one per unit up to the host's cores, each with one BLAS thread.
    Each of the dense and Quest passes is timed three times; the median
    counts.  The GPU outputs are those of the last timed step (the inputs do
    not change between steps and the append is idempotent)."""
    import concurrent.futures
    import numpy as np
    import oracle
    from oracle import quest as oquest
    from threadpoolctl import threadpool_limits

    cfg = step.config
    L, S, D = cfg["seq_len"], cfg["page_size"], cfg["head_dim"]
    G = cfg["num_q_heads"] // cfg["num_kv_heads"]
    K = cfg["budget_tokens"] // S
    P = L // S
    scale = 1.0 / math.sqrt(D)
    host = []
    for (b, kv) in units:   # host copies of the unit (outside the timed passes)
        u = {"q": c["q"][b:b + 1, kv * G:(kv + 1) * G].cpu().numpy(),
             "k": c["k"][b:b + 1, kv:kv + 1].cpu().numpy(),
             "v": c["v"][b:b + 1, kv:kv + 1].cpu().numpy(),
             "k_new": c["k_new"][b:b + 1, kv:kv + 1].cpu().numpy(),
             "v_new": c["v_new"][b:b + 1, kv:kv + 1].cpu().numpy(),
             "lens": np.array([L], np.int32),
             "gpu_dense": c["dense_out"][b, kv * G:(kv + 1) * G].float().cpu().numpy(),
             "gpu_quest": c["quest_out"][b, kv * G:(kv + 1) * G].float().cpu().numpy(),
             "gpu_idx": c["idx"][b:b + 1, kv:kv + 1].cpu().numpy()}
        # the resident metadata state the step updates (built once, untimed)
        u["meta"] = oquest.build_metadata(u["k"], u["lens"], S, P)
        host.append(u)

    def dense_unit(u):
        k2, v2 = oracle.append_kv(u["k"], u["v"], u["lens"], u["k_new"], u["v_new"])
        return oracle.decode_attention(u["q"], k2, v2, u["lens"], scale)[0]

    def quest_unit(u):
        k2, v2 = oracle.append_kv(u["k"], u["v"], u["lens"], u["k_new"], u["v_new"])
        meta = oquest.append_metadata(u["meta"], k2, u["lens"], 1, S)
        scores = oquest.page_scores(u["q"], meta, u["lens"], S)
        idx = oquest.select_pages(scores, u["lens"], S, K)
        out = oquest.sparse_decode_attention(u["q"], k2, v2, u["lens"], idx, S, scale)[0]
        return scores, idx, out, k2, v2

    cores, _ = host_threads()
    workers = max(1, min(cores, len(host)))

    def timed_pass(fn):
        times, res = [], None
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            for _ in range(reps):
                t0 = time.perf_counter()
                res = list(ex.map(fn, host))
                times.append(time.perf_counter() - t0)
        return statistics.median(times), res

    with threadpool_limits(1):
        t_dense, dense_res = timed_pass(dense_unit)
        t_quest, quest_res = timed_pass(quest_unit)
        # attention over the GPU's own choice (untimed; the parity check)
        quest_err = 0.0
        idx_exact = swaps = violations = 0
        for u, (scores, idx, out, k2, v2) in zip(host, quest_res):
            g = [int(p) for p in u["gpu_idx"][0, 0] if p >= 0]
            w = [int(p) for p in idx[0, 0] if p >= 0]
            if g == w:
                idx_exact += 1
                want = out
            else:
                kth = np.sort(scores[0, 0])[::-1][K - 1]
                diff = set(g) ^ set(w)
                swaps += len(diff) // 2
                violations += sum(1 for p in diff
                                  if abs(scores[0, 0, p] - kth) > 1e-5 * abs(kth))
                # the oracle's attention over the pages the GPU chose
                want = oquest.sparse_decode_attention(u["q"], k2, v2, u["lens"], u["gpu_idx"],
                                                      S, scale)[0]
            quest_err = max(quest_err, float(np.max(np.abs(u["gpu_quest"] - want))))
    dense_err = max(float(np.max(np.abs(u["gpu_dense"] - r))) for u, r in zip(host, dense_res))
    unit_kv = L * 2 * D * 2
    quest_unit_bytes = step.kv_bytes // (cfg["batch"] * cfg["num_kv_heads"])
    cores, blas = host_threads()
    return {
        "value": round(len(host) * unit_kv / t_dense / 1e9, 6), "unit": "GB/s",
        "cores": workers, "kind": "oracle",
        "sample": (f"{len(host)} of the {cfg['batch'] * cfg['num_kv_heads']} (b, kv) units, "
                   f"one oracle step each (append + repeat_kv attention over {L} keys, fp64); "
                   "median of 3 passes"),
        "seconds": round(t_dense, 3),
        "host_cores": cores, "blas_threads": 1, "worker_threads": workers,
        "quest": {"gbs": round(len(host) * quest_unit_bytes / t_quest / 1e9, 6),
                  "seconds": round(t_quest, 3),
                  "sample": "the same units: append, new-key metadata update, page scores, "
                            "top-K, attention over the chosen pages (fp64); median of 3"},
        "parity": {"units": [list(u) for u in units],
                   "dense_max_abs_err": dense_err,
                   "quest_max_abs_err": quest_err,
                   "idx_exact": idx_exact, "idx_units": len(host),
                   "idx_near_tie_swaps": swaps, "idx_rule_violations": violations,
                   "tolerance": 2e-3},
    }


def summarize_leg(name, step, r):
    """The short record of a secondary workload in the default line."""
    out = {"workload": step.config["workload"], "us_per_step": r["us_per_step"],
           "kv_gbs": round(r["gbs"], 1), "pct_hbm_peak": round(100 * r["gbs"] / HBM_PEAK_GBS, 2),
           "launch": r["launch"], "stage_us": r["stage_us"],
           "algorithmic_bytes_per_step": step.algo_bytes}
    for key in ("quest_over_dense_time", "dense_same_shape_us", "dense_same_shape_pct_peak"):
        if key in r:
            out[key] = r[key]
    if "byte_model" in r:
        out["byte_model_ratio"] = r["byte_model"]["ratio_model"]
    return out


def long_context_line(args, torch, da, dev, flush):
    """The default line: dense decode attention on the long-context workload
    (value, roofline), the Quest step beside it, secondary legs, CPU
    baseline."""
    step, c = MAKERS["quest128k"](da, torch, args.seed, dev)
    units = step.config["batch"] * step.config["num_kv_heads"]
    # warm-up calls allocate every workspace before the timed loops
    step.dense_fn()
    for st in step.stages:
        for f in st.fns:
            f()
    torch.cuda.synchronize()

    # the headline step: one gqa_decode_attn call (decode kernel + merge)
    t0 = time.perf_counter()
    dense_ms = time_direct(torch, [step.dense_fn], args.steps, args.warmup, flush)
    dense_wall = time.perf_counter() - t0
    ms = statistics.median(dense_ms)
    # the Quest step at the same shape
    qr = measure(torch, da, dev, step, args.steps, args.warmup, flush)
    stage_bytes = {st.name: st.bytes for st in step.stages}
    quest_stages = {}
    for name, us in qr["stage_us"].items():
        gbs = stage_bytes[name] / (us * 1e-6) / 1e9
        quest_stages[name] = {"us": us, "bytes": stage_bytes[name], "gbs": round(gbs, 1),
                              "frac": round(gbs / HBM_PEAK_GBS, 4)}
    quest_ms = qr["ms"]
    model = step.byte_model["ratio_model"]

    # reference copy of known size (scales the FETCH/WRITE counters in the
    # counter runs); not part of the timed region
    src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    cal = read_calibration(da, torch, dev, flush)
    achieved = step.dense_algo_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "decode-attn KV GB/s (% HBM peak) + us/step; Quest score+topK+attn us/step",
        "value": round(step.dense_bytes / (ms * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in, f32 accumulate",
        "data": "synthetic N(0,1) fp16, seeded; 16 planted pages per KV head",
        "config": {"workload": "long_context_gqa_b8_hq32_hkv8_d128_L131072_append",
                   "batch": 8, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                   "seq_len": step.config["seq_len"], "capacity": step.config["seq_len"],
                   "append_slot": step.config["seq_len"] - 1,
                   "step": "gqa_decode_attn over every valid key with the step's K/V row "
                           "appended (decode kernel + split merge)"},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic("long_context", "dense_attention"),
            "frac_of_calibration": round(achieved / cal["read_gbs"], 4),
            "kernel": "decode_kernel<128,4> + merge_kernel (gqa_decode_attn)",
            "stage": "dense_attention",
            "calls_per_step": 1,
            "us_per_call": round(ms * 1e3, 3),
            "bytes_per_call": step.dense_algo_bytes,
            "time_source": "HIP events around the call on its stream in the timed region "
                           "(median over steps); the call is the decode kernel and the "
                           "split merge",
        },
        "us_per_step": round(ms * 1e3, 3),
        "us_p10": round(sorted(dense_ms)[len(dense_ms) // 10] * 1e3, 3),
        "us_p90": round(sorted(dense_ms)[(len(dense_ms) * 9) // 10] * 1e3, 3),
        "kv_bytes_per_step": step.dense_bytes,
        "algorithmic_bytes_per_step": step.dense_algo_bytes,
        "pct_hbm_peak": round(100 * step.dense_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "cache_flush_between_steps": flush is not None,
        "launch": "the step's call launched directly on the stream",
        "timed_wall_s": round(dense_wall, 3),
        "quest": {
            "workload": step.config["workload"],
            "us_per_step": qr["us_per_step"],
            "us_p10": qr["us_p10"],
            "us_p90": qr["us_p90"],
            "kv_bytes_per_step": step.kv_bytes,
            "algorithmic_bytes_per_step": step.algo_bytes,
            "gbs": round(step.algo_bytes / (quest_ms * 1e-3) / 1e9, 1),
            "frac": round(step.algo_bytes / (quest_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "stages": quest_stages,
            "stage_time_source": "HIP events around each stage's call alone after a cache "
                                 "flush (median); each carries its own first-launch latency",
            "us_per_step_separate_topk": qr["step_us_separate_topk"],
            "us_per_step_separate_append": qr["step_us_separate_append"],
            "quest_over_dense_time": round(quest_ms / ms, 4),
            "byte_model_ratio": model,
            "over_byte_model": round(quest_ms / ms / model, 3),
            "target_us_at_70pct": round(step.kv_bytes / (0.7 * HBM_PEAK_GBS * 1e3), 3),
            "units": units,
        },
        "calibration": cal,
        "dense_pct_calibration": round(100 * step.dense_bytes / (ms * 1e-3) / 1e9
                                       / cal["read_gbs"], 2),
    }
    fl = launch_floor(torch, dev, flush, step.kernels_per_step, max(10, args.steps // 2))
    fl["bytes_at_calibrated_rate_us"] = round(step.algo_bytes / (cal["read_gbs"] * 1e3), 3)
    line["quest"]["launch_floor"] = fl
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = long_context_cpu_baseline(
            step, c, sample_units(step.config["batch"], step.config["num_kv_heads"], 16))
    del c
    torch.cuda.empty_cache()

    if not args.no_legs:
        legs = {}
        for name in ("exaone30", "paged", "quest32k", "gqa1"):
            lstep, ldata = MAKERS[name](da, torch, args.seed, dev)
            # half the line's steps and warm-up: with only a few warm-up steps
            # the first timed steps of a long leg run slow while the clocks settle
            r = measure(torch, da, dev, lstep, max(10, args.steps // 2), max(3, args.warmup // 2),
                        flush)
            legs[name] = summarize_leg(name, lstep, r)
            if hasattr(lstep, "kernels_per_step"):
                lf = launch_floor(torch, dev, flush, lstep.kernels_per_step, 10)
                legs[name]["launch_floor_us"] = lf["us_per_step"]
            del ldata
            torch.cuda.empty_cache()
        line["legs"] = legs
    return line


MAKERS = {
    "exaone30": exaone30, "gqa1": gqa1, "paged": paged,
    "quest32k": lambda *a: quest(*a, long_ctx=False),
    "quest128k": lambda *a: quest(*a, long_ctx=True),
}


CAL_BYTES = 4 << 30


def launch_floor(torch, dev, flush, n_kernels, steps):
    """Step time of `n_kernels` one-element fill kernels launched the way the
    step's calls are (directly, or replayed from one captured graph), with the
    same cache flush: the launch-only floor of a step with that many dependent
    kernels, none of which moves data."""
    t = torch.zeros(1, dtype=torch.float32, device=dev)
    fns = [lambda: t.fill_(1.0)] * n_kernels
    ms, how = time_calls(torch, fns, steps, 3, flush)
    return {"kernels": n_kernels, "kernel": "one-element fill (torch)", "launch": how,
            "us_per_step": round(statistics.median(ms) * 1e3, 3)}


def read_calibration(da, torch, dev, flush, reps=10):
    """HBM read rate of the library's streaming-read calibration kernel over a
    4 GiB buffer (cache flushed before each rep, median): the practical read
    ceiling on this part, reported next to the nominal peak."""
    buf = torch.full((CAL_BYTES,), 0x5A, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(reps + 2):
        if flush is not None:
            flush.zero_()
        a.record()
        da.read_calibration(buf, sink)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            times.append(a.elapsed_time(b) * 1e-3)
    del buf, sink
    torch.cuda.empty_cache()
    sec = statistics.median(times)
    return {"read_gbs": round(CAL_BYTES / sec / 1e9, 1), "bytes": CAL_BYTES,
            "kernel": "read_calibration_kernel (da_read_calibration)",
            "pct_of_peak": round(100 * CAL_BYTES / sec / 1e9 / HBM_PEAK_GBS, 2)}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "there is no multi-GPU path", file=sys.stderr)
        return 2
    import torch
    import decode_attention_folded_amd as da
    da.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = None if args.no_flush else torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    if args.workload == "repeat_kv_ab":
        ab = repeat_kv_ab(da, torch, args.seed, dev, args.steps, args.warmup, flush)
        ex = ab["exaone_30_layers_len3000"]
        big = ab["paged_b64_len1k-32k"]
        line = {
            "metric": "fold vs materialised repeat_kv (copy + G=1 attention): time ratio",
            "value": ex["materialised_over_fold"], "unit": "x", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ex["fold_us"] * 1e-3, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16 in, f32 accumulate",
            "data": "synthetic N(0,1) fp16, seeded",
            "config": {"workload": "repeat_kv_ab: gqa layer, exaone 30 layers, paged b64"},
            "roofline": {"bound": "hbm", "achieved": big["copy_gbs"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(big["copy_gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": None, "kernel": "repeat_kv_kernel (gqa_repeat_kv)",
                         "stage": "repeat_kv copy, paged b64",
                         "bytes_per_call": big["copy_bytes"],
                         "us_per_call": big["repeat_kv_copy_us"],
                         "time_source": "HIP events around the call after a cache flush "
                                        "(median)"},
            "repeat_kv_ab": ab,
            "cache_flush_between_steps": flush is not None,
        }
        print(json.dumps(line), flush=True)
        return 0
    if args.workload == "multi_query":
        mq = multi_query(da, torch, args.seed, dev, args.steps, args.warmup, flush)
        ex = mq["exaone_30_layers_len3000"]
        line = {
            "metric": "decode-attn KV GB/s with q_len > 1 queries per head (fold, causal)",
            "value": ex["q_len_2"]["kv_gbs"], "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ex["q_len_2"]["step_us"] * 1e-3, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16 in, f32 accumulate",
            "data": "synthetic N(0,1) fp16, seeded",
            "config": {"workload": "multi_query: exaone 30 layers, dense 32K G=1, dense 128K G=4",
                       "value_is": "exaone 30 layers at q_len 2"},
            "multi_query": mq,
            "cache_flush_between_steps": flush is not None,
        }
        print(json.dumps(line), flush=True)
        return 0
    if args.workload == "quest_sweep":
        sw = quest_sweep(da, torch, args.seed, dev, args.steps, args.warmup, flush)
        base = sw["sweep"]["S16_fixed_budget_2048"]
        line = {
            "metric": "Quest score+topK+attn us/step (page-size sweep, 32K Llama2-7B shape)",
            "value": base["step_us"], "unit": "us", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(base["step_us"] * 1e-3, 6),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16 in, f32 accumulate", "data": "synthetic N(0,1) fp16, seeded",
            "config": {"workload": "quest_sweep_b1_h32_d128_L32768_S8-64",
                       "value_is": "S=16, budget 2048"},
            "quest_sweep": sw,
            "cache_flush_between_steps": flush is not None,
        }
        print(json.dumps(line), flush=True)
        return 0
    if args.workload == "long_context":
        print(json.dumps(long_context_line(args, torch, da, dev, flush)), flush=True)
        return 0
    step, data = MAKERS[args.workload](da, torch, args.seed, dev)
    r = measure(torch, da, dev, step, args.steps, args.warmup, flush)

    # reference copy of known size (scales the FETCH/WRITE counters in the
    # counter runs); not part of the timed region
    src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    traffic = counter_traffic(args.workload, r["dominant"].name)
    cal = read_calibration(da, torch, dev, flush)
    line = {
        "metric": "decode-attn KV GB/s (% HBM peak) + us/step",
        "value": round(r["gbs"], 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in, f32 accumulate",
        "data": "synthetic N(0,1) fp16, seeded",
        "config": step.config,
        "roofline": {
            "bound": "hbm",
            "achieved": round(r["achieved"], 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "frac_of_calibration": round(r["achieved"] / cal["read_gbs"], 4),
            "kernel": r["dominant"].kernels,
            "stage": r["dominant"].name,
            "calls_per_step": len(r["dominant"].fns),
            "us_per_call": round(r["stage_ms"] * 1e3 / len(r["dominant"].fns), 3),
            "bytes_per_call": r["dominant"].bytes // len(r["dominant"].fns),
            "time_source": ("HIP events around the step in the timed region (median over "
                            "steps), divided by its calls" if len(step.stages) == 1 else
                            "HIP events around the stage's calls alone after a cache "
                            "flush (median), divided by its calls"),
        },
        "us_per_step": r["us_per_step"],
        "us_p10": r["us_p10"],
        "us_p90": r["us_p90"],
        "kv_bytes_per_step": step.kv_bytes,
        "algorithmic_bytes_per_step": step.algo_bytes,
        "pct_hbm_peak": round(100 * r["gbs"] / HBM_PEAK_GBS, 2),
        "cache_flush_between_steps": flush is not None,
        "launch": ("the step replayed from one captured HIP graph" if r["launch"] == "graph"
                   else "the step's calls launched directly on the stream"),
        "timed_wall_s": r["timed_wall_s"],
        "stage_us": r["stage_us"],
        "calibration": cal,
    }
    for key in ("dense_same_shape_us", "dense_same_shape_gbs", "dense_same_shape_pct_peak",
                "quest_over_dense_time", "byte_model", "step_us_separate_topk",
                "step_us_separate_append", "us_per_step_graph"):
        if key in r:
            line[key] = r[key]
    if hasattr(step, "kernels_per_step"):
        # what the same number of dependent launches costs with no data, and
        # what the step's bytes cost at the calibrated read rate
        fl = launch_floor(torch, dev, flush, step.kernels_per_step, max(10, args.steps // 2))
        fl["bytes_at_calibrated_rate_us"] = round(step.algo_bytes / (cal["read_gbs"] * 1e3), 3)
        line["launch_floor"] = fl
    if "dense_same_shape_gbs" in r:
        line["dense_same_shape_pct_calibration"] = round(
            100 * r["dense_same_shape_gbs"] / cal["read_gbs"], 2)

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(step, data, args.seed)

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
