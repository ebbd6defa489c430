#!/usr/bin/env python3
"""Benchmark of the GPT-OSS attention hot path on one MI355X.

Step = one pass of the prefill hot path over the dense BSHD workload
(B=4, S=4096, 64 query / 8 KV heads of width 64, bf16 N(0,1) inputs, fp32
N(0,1) sinks): build the YaRN cos/sin table for the 4096 positions, then one
full-causal layer and one sliding-window-128 layer, each with q and k rotated
inside the attention call. `value` is unmasked prefill TFLOP/s over the step
(4 * D * Hq FLOPs per visible (query, key) pair). The decode half of the metric
(64 sequences, cache lengths uniform in [1024, 32768], full and window-128
layers) is timed in the same run and reported under "decode", with the same
decode over a paged cache (64-row pages in a shuffled pool) and over 128-slot
ring caches for the window layer, and the cache append, under "decode.kv_cache".

Timing uses HIP events recorded on the stream the library launches on, around
every call inside the timed region; the whole region is bracketed by device
synchronisation. Before its timed calls every section runs its own calls for
--settle-seconds (default 0.3 s) and then W untimed warm-up iterations: from
idle, this GPU needs a few tens of milliseconds of sustained load before its
clock settles, and calls timed earlier run up to 20 % slower. The timed work is
the same either way; the JSON states the settle time. The window-layer decode
(a 17.8 MB working set, inside the 256 MB last-level cache) has a 512 MiB buffer
written between its timed calls, outside the timed events, so its rate is not
served from that cache. A 1 GiB device copy is timed as well, so that HBM rates
can be read against achievable as well as against the 8 TB/s of the data sheet.
The CPU baseline is the fp64 oracle on time-bounded samples of every workload
(query rows of each prefill config and layer, whole sequences of the decode),
on this host's cores.

The same two layers over 16 packed THD sequences (lengths uniform in [128, 8192])
and over one 131072-token sequence are timed under "prefill_thd_and_long".

The backward pass of both layers (dq, dk, dv, dsinks) is timed after the step and
reported under "backward" (not part of `value`). The q/k/v projections of the
same tokens (hidden 2880, Linear with bias) with the RoPE in their epilogue are
timed under "projection", next to torch's linear (hipBLASLt) followed by the
standalone rotation, as context. One step of a context-parallel prefill (a
128K-token sequence over 8 ranks: a 16384-token query shard against a
16384-token key shard) and the merge of 8 partial results are timed under
"context_parallel" (one GPU's share of the ring; the exchange is not built).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-backward] [--settle SECONDS]
       python bench.py --profile {step,prefill-full,prefill-window,decode-full,copy,backward-full,backward-window,
                                  decode-paged,decode-ring,kv-append,proj-rope,proj,cp-step} --steps K
       (the --profile modes run only the named call, for rocprofv3)
"""

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (%MFMA peak) + decode KV GB/s (%HBM peak), 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
WINDOW = 128
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {   # the sources a kernel's counters depend on
    "prefill": ["attention_yarn_rope_amd/csrc/prefill.hip", "attention_yarn_rope_amd/csrc/common.h"],
    "decode": ["attention_yarn_rope_amd/csrc/decode.hip", "attention_yarn_rope_amd/csrc/common.h"],
    "window": ["attention_yarn_rope_amd/csrc/window.hip", "attention_yarn_rope_amd/csrc/common.h"],
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_traffic(name, kernel):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None.

    profiles/<name>.counters.json holds FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) for the kernel, the same counters for a plain copy kernel of known
    size (the calibration factor), and the hash of the kernel sources at the
    time; a changed kernel makes the figure stale (None).
    """
    path = os.path.join(PROFILES, f"{name}.counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return c["traffic_bytes_per_launch"]


def ensure_built():
    from attention_yarn_rope_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from attention_yarn_rope_amd import build
        build.build(verbose=False)


class Timer:
    """Per-call HIP event pairs on the current (library) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        stream = self.torch.cuda.current_stream()
        s.record(stream)
        fn()
        e.record(stream)
        self.pairs.setdefault(name, []).append((s, e))

    def mean_ms(self, name):
        v = [s.elapsed_time(e) for s, e in self.pairs.get(name, [])]
        return sum(v) / len(v) if v else float("nan")


def settle_clock(torch, dev, seconds):
    """Sustained bf16 matrix-core load for `seconds`, so that a profiled kernel's launches all run at
    the settled clock (from idle this GPU needs tens of milliseconds of load to reach it)."""
    if seconds <= 0:
        return
    a = torch.randn((4096, 4096), device=dev).to(torch.bfloat16)
    torch.mm(a, a)   # library set-up happens here, outside the timed load
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            torch.mm(a, a)
        torch.cuda.synchronize()


def settle(torch, fns, warmup, seconds):
    """Untimed: the section's own calls for `seconds` (the clock settles under sustained load),
    then `warmup` more rounds of them."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for fn in fns:
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        for fn in fns:
            fn()
    torch.cuda.synchronize()


def host_cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class _RowsF64:
    """Indexable view of a CPU bf16 tensor that converts only the indexed rows to fp64."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        import numpy as np
        import torch
        return self.t[torch.as_tensor(np.asarray(idx))].double().numpy()


def cpu_baseline(samples, budget_s):
    """The oracle, as it stands, timed on bounded samples of every workload on the host's cores.

    samples: (config, layer, kind, data). kind "rows": data = (q, k, v, sinks, window, rows) for one
    sequence, rows in the order they are taken, a few at a time, until the entry's share of budget_s
    is spent; kind "decode": data = (q, k_cache, v_cache, lengths, sinks, window), whole sequences in
    order. Returns the aggregate rate and, per (config, layer), rows or sequences done, seconds and
    GFLOP/s on unmasked FLOPs (4 * 64 * 64 per visible (query, key) pair and head)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    per = budget_s / max(len(samples), 1)
    flops_all, secs_all, table = 0, 0.0, {}
    for config, layer, kind, data in samples:
        flops, done, t0 = 0, 0, time.perf_counter()
        if kind == "rows":
            q, k, v, sinks, w, rows = data
            step = 1 if (w == 0 and len(rows) <= 512 and q.shape[0] > 8192) else 8
            while done < len(rows) and time.perf_counter() - t0 < per:
                rs = np.sort(np.asarray(rows[done:done + step]))
                oracle.prefill_rows(q, k, v, sinks, 0.125, w, rs)
                flops += sum(4 * 64 * 64 * (min(int(r) + 1, w) if w else int(r) + 1) for r in rs)
                done += len(rs)
            unit = "query rows x 64 heads"
        else:
            q, kc, vc, lengths, sinks, w = data
            while done < len(lengths) and time.perf_counter() - t0 < per:
                L = int(lengths[done])
                lo = 0 if w <= 0 else max(0, L - w)
                oracle.decode(q[done:done + 1].double().numpy(), kc[done:done + 1, :L].double().numpy(),
                              vc[done:done + 1, :L].double().numpy(), [L], sinks, 0.125, w)
                flops += 4 * 64 * 64 * (L - lo)
                done += 1
            unit = "sequences x 64 heads"
        secs = time.perf_counter() - t0
        flops_all += flops
        secs_all += secs
        table.setdefault(config, {})[layer] = {"done": done, "of": unit, "seconds": round(secs, 2),
                                               "GFLOP/s": round(flops / secs / 1e9, 2) if secs > 0 else None}
    return {"value": flops_all / secs_all / 1e12 if secs_all > 0 else None, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": host_cpu_model(), "seconds": round(secs_all, 2),
            "sample": "seeded query rows of each prefill workload (tiny, dense B=4 S=4096 batch 0, the longest "
                      "THD sequence, the 512 sampled rows of the 131072-token sequence) and whole sequences of "
                      "the 64-sequence decode, full-causal and window-128 layers, each for an equal share of "
                      f"{budget_s:.0f} s; fp64 numpy on the host CPU",
            "per_config": table}


def kv_cache_calls(torch, gx, wl, dev, dq, kc, vc, lens, dsinks, dtable, lengths, d_out, pk, pv):
    """Closures over the decode workload's caches in the other layouts.

    paged_full: the full layer over a pool of 64-row pages holding the same rows in a
    shuffled page order (block table = where each logical page went); ring_window: the
    window layer over 128-slot ring caches (random rows); append_1: one new token per
    sequence appended to the paged pool and to the rings; append_prompt: the dense
    prefill's k and v (B=4 S=4096) appended to a contiguous cache in one call.
    """
    N, Lmax = kc.shape[0], kc.shape[1]
    ps = 64
    npages = N * Lmax // ps
    perm = torch.randperm(npages, generator=torch.Generator().manual_seed(12)).to(dev)
    k_pool = torch.empty((npages, ps, 8, 64), dtype=torch.bfloat16, device=dev)
    v_pool = torch.empty_like(k_pool)
    k_pool[perm] = kc.reshape(npages, ps, 8, 64)
    v_pool[perm] = vc.reshape(npages, ps, 8, 64)
    block_table = perm.to(torch.int32).reshape(N, Lmax // ps).contiguous()
    ring = wl.ring_decode(lengths, 128, seed=45)
    rk, rv = ring.k_cache.to(dev), ring.v_cache.to(dev)
    kn, vn = (t.to(dev) for t in wl.new_tokens(N, 1, 46))
    pws = torch.empty(gx.decode_kv_workspace_size(dq, k_pool, "paged", block_table, 0, Lmax), dtype=torch.uint8,
                      device=dev)
    rws = torch.empty(gx.decode_kv_workspace_size(dq, rk, "ring", None, 128, Lmax), dtype=torch.uint8, device=dev)
    ptable = gx.rope_table(pk.shape[1])
    ck = torch.empty_like(pk)
    cv = torch.empty_like(pv)
    plens = torch.full((pk.shape[0],), pk.shape[1], dtype=torch.int32, device=dev)
    out = torch.empty_like(d_out)

    def append_1():
        gx.kv_append(k_pool, v_pool, kn, vn, lens, kind="paged", block_table=block_table, table=dtable,
                     max_seqlen=Lmax)
        gx.kv_append(rk, rv, kn, vn, lens, kind="ring", table=dtable, max_seqlen=Lmax)

    return {
        "paged_full": lambda: gx.attn_decode_kv(dq, k_pool, v_pool, lens, dsinks, kind="paged",
                                                block_table=block_table, table=dtable, max_seqlen=Lmax, out=out,
                                                workspace=pws),
        "ring_window": lambda: gx.attn_decode_kv(dq, rk, rv, lens, dsinks, kind="ring", window=128, table=dtable,
                                                 max_seqlen=Lmax, out=out, workspace=rws),
        "append_1": append_1,
        "append_prompt": lambda: gx.kv_append(ck, cv, pk, pv, plens, table=ptable),
        "prompt_tokens": pk.shape[0] * pk.shape[1],
    }


def kv_cache_bench(torch, wl, kvc, args, lengths, b_full, b_win, flush):
    timer = Timer(torch)
    names = ("paged_full", "ring_window", "append_1", "append_prompt")
    settle(torch, [kvc[n] for n in names], args.warmup, args.settle_seconds)
    for _ in range(args.steps):
        for n in names:
            if n == "ring_window":
                flush()   # the rings (16.8 MB) would otherwise stay in the last-level cache
            timer.run(n, kvc[n])
    torch.cuda.synchronize()
    ms = {n: timer.mean_ms(n) for n in names}

    # one decode step of a full + window layer pair as a serving loop runs it (append the new
    # tokens to the paged pool and the rings, then both decodes), eager and as a HIP graph
    # replay; K steps back to back between two events
    def step():
        kvc["append_1"]()
        kvc["paged_full"]()
        kvc["ring_window"]()

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    step_ms = {}
    for nm, fn in (("eager", step), ("graph", graph.replay)):
        settle(torch, [fn], args.warmup, args.settle_seconds)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(torch.cuda.current_stream())
        for _ in range(args.steps):
            fn()
        e.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        step_ms[nm] = s.elapsed_time(e) / args.steps
    del graph
    T = kvc["prompt_tokens"]
    b_prompt = T * 8 * 64 * 2 * 4 + 4096 * 64 * 2   # read k, v; write k, v; table rows
    return {
        "workload": "the decode workload's caches as a shuffled pool of 64-row pages (full layer) and as 128-slot "
                    "ring caches (window layer); append: 1 token x 64 sequences into the pool and the rings, and "
                    f"a {T}-token prompt (B=4 S=4096) into a contiguous cache",
        "paged_full_layer": {"ms": round(ms["paged_full"], 4),
                             "GB/s": round(b_full / (ms["paged_full"] * 1e-3) / 1e9, 1),
                             "frac_hbm_peak": round(b_full / (ms["paged_full"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "ring_window_layer": {"ms": round(ms["ring_window"], 4),
                              "GB/s": round(b_win / (ms["ring_window"] * 1e-3) / 1e9, 1),
                              "cache": "a 512 MiB buffer written before each timed call"},
        "append_1_token_ms": round(ms["append_1"], 4),
        "decode_step": {"what": "append 1 token x 64 sequences (pool and rings) + paged full-layer decode + ring "
                                "window-layer decode, K steps back to back",
                        "eager_ms": round(step_ms["eager"], 4), "hip_graph_ms": round(step_ms["graph"], 4)},
        "append_prompt": {"ms": round(ms["append_prompt"], 4), "bytes": b_prompt,
                          "GB/s": round(b_prompt / (ms["append_prompt"] * 1e-3) / 1e9, 1)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle", type=float, default=0.2,
                    help="--profile modes: seconds of matrix-core load before the profiled calls")
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="seconds each timed section runs its own calls before its warm-up and timed calls")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--k-rotation", default="auto", choices=["auto", "fused", "separate"])
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip the THD and 128K-token prefill timings")
    ap.add_argument("--profile", default=None, choices=["step", "prefill-full", "prefill-window", "decode-full", "copy",
                                                        "backward-full", "backward-window", "decode-paged",
                                                        "decode-ring", "kv-append", "proj-rope", "proj",
                                                        "cp-step"])
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): this attention path has no "
              "multi-GPU mode; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    ensure_built()
    import torch
    import attention_yarn_rope_amd as gx
    from attention_yarn_rope_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.profile == "copy":
        # calibration for the HBM counters: a plain 1 GiB device-to-device copy
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {args.steps} x 1 GiB")
        return

    cpu_samples = []   # (config, layer, kind, data) for the oracle baseline at the end
    flush_buf = None
    copy_gbs = fill_gbs = None

    def flush():
        flush_buf.fill_(1)

    if args.profile is None:
        # achievable HBM bandwidth: a plain 1 GiB device-to-device copy (2 GiB moved per call)
        csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        settle(torch, [lambda: cdst.copy_(csrc)], 3, args.settle_seconds)
        timer = Timer(torch)
        for _ in range(10):
            timer.run("copy", lambda: cdst.copy_(csrc))
            timer.run("fill", lambda: cdst.fill_(1))
        torch.cuda.synchronize()
        copy_gbs = 2 * (1 << 30) / (timer.mean_ms("copy") * 1e-3) / 1e9
        fill_gbs = (1 << 30) / (timer.mean_ms("fill") * 1e-3) / 1e9
        del csrc, cdst, timer
        flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        log(f"[bench] device copy {copy_gbs:.0f} GB/s, fill {fill_gbs:.0f} GB/s")

    # ---------------- prefill (the step) ----------------
    log("[bench] generating dense B=4 S=4096 workload")
    inp = wl.dense()
    q, k, v, sinks = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.sinks))
    S = q.shape[1]
    table = torch.empty((S, 64), dtype=torch.bfloat16, device=dev)
    o_full = torch.empty_like(q)
    o_win = torch.empty_like(q)
    ws = torch.empty(max(gx.prefill_workspace_size(q, k), 1), dtype=torch.uint8, device=dev)
    gx.rope_table(S, out=table)

    def call_full():
        gx.attn_prefill(q, k, v, sinks, window=0, table=table, out=o_full, workspace=ws, k_rotation=args.k_rotation)

    def call_win():
        gx.attn_prefill(q, k, v, sinks, window=WINDOW, table=table, out=o_win, workspace=ws,
                        k_rotation=args.k_rotation)

    if args.profile == "step":
        # the timed step's exact call sequence (table, full layer, window layer), for rocprofv3
        settle_clock(torch, dev, args.settle)
        for _ in range(args.steps):
            gx.rope_table(S, out=table)
            call_full()
            call_win()
        torch.cuda.synchronize()
        log(f"step: {args.steps} steps")
        return

    if args.profile in ("prefill-full", "prefill-window"):
        fn = call_full if args.profile == "prefill-full" else call_win
        settle_clock(torch, dev, args.settle)
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        log(f"{args.profile}: {args.steps} launches")
        return

    # ---------------- q/k/v projections with the RoPE in the epilogue ----------------
    def projection_calls():
        pw = wl.projection(q.shape[0] * S, seed=50)
        px = pw.x.to(dev).reshape(q.shape[0], S, -1)
        wts = [t.to(dev) for t in (pw.wq, pw.bq, pw.wk, pw.bk, pw.wv, pw.bv)]
        outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        wcat = torch.cat([wts[0], wts[2], wts[4]]).contiguous()
        bcat = torch.cat([wts[1], wts[3], wts[5]]).contiguous()
        nq, nk = q.shape[2] * 64, k.shape[2] * 64

        def torch_path():
            y = torch.nn.functional.linear(px, wcat, bcat)
            return gx.rope_qk(y[..., :nq].reshape(q.shape), y[..., nq:nq + nk].reshape(k.shape), table)

        return {"fused": lambda: gx.qkv_proj_rope(px, *wts, table=table, out=outs),
                "unrotated": lambda: gx.qkv_proj_rope(px, *wts, out=outs),
                "torch_linear_rope_qk": torch_path,
                "flops": wl.projection_flops(q.shape[0] * S, hidden=px.shape[-1])}

    if args.profile in ("proj-rope", "proj"):
        fn = projection_calls()["fused" if args.profile == "proj-rope" else "unrotated"]
        settle_clock(torch, dev, args.settle)
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        log(f"{args.profile}: {args.steps} calls")
        return

    # ---------------- context-parallel prefill: one GPU's ring step and the merge ----------------
    def cp_calls():
        n, ranks = 16384, 8
        sh = wl.prefill_bshd(1, n, seed=61)
        cq, ck, cv = sh.q.to(dev), sh.k.to(dev), sh.v.to(dev)
        ctab = gx.rope_table(n * ranks)
        o = torch.empty_like(cq)
        lse = torch.empty((n, cq.shape[2]), dtype=torch.float32, device=dev)
        cws = torch.empty(max(gx.prefill_shard_workspace_size(cq, ck), 1), dtype=torch.uint8, device=dev)
        parts_o = torch.randn((ranks, n, cq.shape[2], 64), generator=torch.Generator().manual_seed(62)).to(
            torch.bfloat16).to(dev)
        parts_l = (torch.randn((ranks, n * cq.shape[2]), generator=torch.Generator().manual_seed(63)) * 2).to(dev)
        mo = torch.empty((n, cq.shape[2], 64), dtype=torch.bfloat16, device=dev)
        qo = (ranks - 1) * n
        return {
            "offdiag": lambda: gx.attn_prefill_shard(cq, ck, cv, qo, 0, table=ctab, out=o, lse=lse, workspace=cws),
            "diag": lambda: gx.attn_prefill_shard(cq, ck, cv, qo, qo, table=ctab, out=o, lse=lse, workspace=cws),
            "merge": lambda: gx.attn_merge(parts_o, parts_l, sinks, out=mo),
            "flops_offdiag": 4 * 64 * cq.shape[2] * n * n,
            "flops_diag": wl.prefill_flops([n], 0),
            "bytes_merge": ranks * n * cq.shape[2] * (64 * 2 + 4) + n * cq.shape[2] * 64 * 2,
            "n": n, "ranks": ranks,
        }

    if args.profile == "cp-step":
        fn = cp_calls()["offdiag"]
        settle_clock(torch, dev, args.settle)
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        log(f"cp-step: {args.steps} calls")
        return

    # ---------------- backward of both layers (measured beside the step) ----------------
    def backward_calls():
        """One forward with lse per layer, then closures that run each layer's backward."""
        dout = wl.grad_out(q.shape, 7).to(dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty(q.shape[2], dtype=torch.float32, device=dev))
        bws = torch.empty(max(gx.prefill_backward_workspace_size(q, k), 1), dtype=torch.uint8, device=dev)
        calls = {}
        for name, w in (("full", 0), ("window128", WINDOW)):
            o, lse = gx.attn_prefill_lse(q, k, v, sinks, window=w, table=table)
            calls[name] = (lambda o=o, lse=lse, w=w: gx.attn_prefill_backward(
                q, k, v, sinks, o, dout, lse, window=w, table=table, workspace=bws, grads=grads))
        return calls

    if args.profile in ("backward-full", "backward-window"):
        fn = backward_calls()["full" if args.profile == "backward-full" else "window128"]
        settle_clock(torch, dev, args.settle)
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        log(f"{args.profile}: {args.steps} calls")
        return

    lengths = [S] * q.shape[0]
    flops_full = wl.prefill_flops(lengths, 0)
    flops_win = wl.prefill_flops(lengths, WINDOW)
    bytes_prefill = wl.prefill_bytes(q.shape[0] * S, S)

    if args.profile is None:
        timer = Timer(torch)
        settle(torch, [lambda: gx.rope_table(S, out=table), call_full, call_win], args.warmup, args.settle_seconds)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            timer.run("table", lambda: gx.rope_table(S, out=table))
            timer.run("full", call_full)
            timer.run("window", call_win)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = wall * 1e3 / args.steps
        ms_full, ms_win, ms_table = timer.mean_ms("full"), timer.mean_ms("window"), timer.mean_ms("table")
        log(f"[bench] prefill step {ms_step:.3f} ms (full {ms_full:.3f} ms, window {ms_win:.3f} ms, "
            f"table {ms_table:.4f} ms)")
        del timer

    other_obj = None
    if args.profile is None and not args.no_other_prefill:
        # the same two layers over packed THD sequences (the varlen scheduler) and over one
        # 131072-token sequence (the 128K context); parity cases in the tests, timed here
        other_obj = {}
        ti = wl.thd()
        tq, tk, tv, ts = (t.to(dev) for t in (ti.q, ti.k, ti.v, ti.sinks))
        tcu = ti.cu_seqlens.to(dev)
        ttab = gx.rope_table(ti.max_seqlen)
        tout = torch.empty_like(tq)
        tws = torch.empty(max(gx.prefill_workspace_size(tq, tk, cu_seqlens=tcu, max_seqlen=ti.max_seqlen), 1),
                          dtype=torch.uint8, device=dev)
        thd_calls = {w: (lambda w=w: gx.attn_prefill(tq, tk, tv, ts, window=w, table=ttab, cu_seqlens=tcu,
                                                     max_seqlen=ti.max_seqlen, out=tout, workspace=tws))
                     for w in (0, WINDOW)}
        timer = Timer(torch)
        for w, fn in thd_calls.items():
            settle(torch, [fn], args.warmup, args.settle_seconds)
            for _ in range(args.steps):
                timer.run(w, fn)
            torch.cuda.synchronize()
        other_obj["thd"] = {"workload": f"THD: {len(ti.lengths)} packed sequences, lengths uniform in [128, 8192] "
                                        f"(T = {sum(ti.lengths)}), Hq=64 Hkv=8 D=64, bf16"}
        for w, nm in ((0, "full"), (WINDOW, "window128")):
            ms = timer.mean_ms(w)
            fl = wl.prefill_flops(ti.lengths, w)
            other_obj["thd"][nm] = {"ms": round(ms, 4), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1), "flops": fl}
        del tq, tk, tv, tout, tws, thd_calls, timer
        n_long_seq = max(range(len(ti.lengths)), key=lambda n: ti.lengths[n])
        a, b = int(ti.cu_seqlens[n_long_seq]), int(ti.cu_seqlens[n_long_seq + 1])
        trows = __import__("numpy").random.default_rng(2025).permutation(b - a)
        for w, nm in ((0, "full"), (WINDOW, "window128")):
            cpu_samples.append(("thd_longest_sequence", nm, "rows", (
                ti.q[a:b].double().numpy(), ti.k[a:b].double().numpy(), ti.v[a:b].double().numpy(),
                ti.sinks.double().numpy(), w, trows)))
        del ti
        li = wl.long_context()
        lq, lk, lv, lsk = (t.to(dev) for t in (li.q, li.k, li.v, li.sinks))
        lrows = [int(r) for r in __import__("numpy").random.default_rng(2026).permutation(wl.long_context_rows())]
        for w, nm in ((0, "full"), (WINDOW, "window128")):
            cpu_samples.append(("long_S131072_512_rows", nm, "rows", (
                _RowsF64(li.q[0]), _RowsF64(li.k[0]), _RowsF64(li.v[0]), li.sinks.double().numpy(), w, lrows)))
        del li
        ltab = gx.rope_table(lq.shape[1])
        lout = torch.empty_like(lq)
        lws = torch.empty(max(gx.prefill_workspace_size(lq, lk), 1), dtype=torch.uint8, device=dev)
        timer = Timer(torch)
        n_long = max(min(args.steps, 3), 1)
        for w in (0, WINDOW):
            fn = (lambda w=w: gx.attn_prefill(lq, lk, lv, lsk, window=w, table=ltab, out=lout, workspace=lws))
            # a full-layer call is ~0.13 s of load by itself: two calls settle the clock
            settle(torch, [fn], 2 if w == 0 else args.warmup, 0.0 if w == 0 else args.settle_seconds)
            for _ in range(n_long):
                timer.run(w, fn)
            torch.cuda.synchronize()
        other_obj["long"] = {"workload": f"one sequence of {lq.shape[1]} tokens (B=1), Hq=64 Hkv=8 D=64, bf16",
                             "timed_calls": n_long}
        for w, nm in ((0, "full"), (WINDOW, "window128")):
            ms = timer.mean_ms(w)
            fl = wl.prefill_flops([lq.shape[1]], w)
            other_obj["long"][nm] = {"ms": round(ms, 4), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1), "flops": fl}
        log(f"[bench] THD full {other_obj['thd']['full']['ms']:.3f} ms, window {other_obj['thd']['window128']['ms']:.3f}"
            f" ms; 128K full {other_obj['long']['full']['ms']:.1f} ms, window {other_obj['long']['window128']['ms']:.3f} ms")
        del lq, lk, lv, lout, lws, timer

    projection_obj = None
    if args.profile is None:
        pc = projection_calls()
        timer = Timer(torch)
        names = ("fused", "unrotated", "torch_linear_rope_qk")
        # each call type in its own block of K calls after its warm-up (interleaving the three
        # measured the first one up to 20 % slower than the same kernel run back to back)
        for n in names:
            settle(torch, [pc[n]], args.warmup, args.settle_seconds)
            for _ in range(args.steps):
                timer.run(n, pc[n])
            torch.cuda.synchronize()
        pfl = pc["flops"]
        projection_obj = {
            "workload": f"q/k/v projections of the dense prefill's {q.shape[0] * S} tokens: hidden 2880 -> "
                        "4096 / 512 / 512, Linear with bias, bf16; q and k rotated with the table in the epilogue",
            "flops": pfl,
        }
        for n in names:
            ms = timer.mean_ms(n)
            projection_obj[n] = {"ms": round(ms, 4), "TFLOP/s": round(pfl / (ms * 1e-3) / 1e12, 1),
                                 "frac_mfma_peak": round(pfl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        projection_obj["torch_linear_rope_qk"]["note"] = "context: torch.nn.functional.linear (hipBLASLt) then " \
                                                         "gptoss_rope_qk"
        log(f"[bench] projection fused {projection_obj['fused']['ms']:.3f} ms "
            f"({projection_obj['fused']['TFLOP/s']:.0f} TFLOP/s)")
        del pc, timer

    cp_obj = None
    if args.profile is None:
        cc = cp_calls()
        timer = Timer(torch)
        names = ("offdiag", "diag", "merge")
        settle(torch, [cc[nm] for nm in names], max(args.warmup // 10, 1), args.settle_seconds)
        for _ in range(max(args.steps // 4, 3)):
            for nm in names:
                timer.run(nm, cc[nm])
        torch.cuda.synchronize()
        ms = {nm: timer.mean_ms(nm) for nm in names}
        cp_obj = {
            "workload": f"one ring step of a {cc['n'] * cc['ranks']}-token full-causal prefill over {cc['ranks']} "
                        f"ranks: a {cc['n']}-token query shard (the last rank's) against a {cc['n']}-token key "
                        "shard, q and k rotated at their global positions, no sink; the merge of "
                        f"{cc['ranks']} partial results adds it",
            "offdiag_step": {"ms": round(ms["offdiag"], 4), "flops": cc["flops_offdiag"],
                             "TFLOP/s": round(cc["flops_offdiag"] / (ms["offdiag"] * 1e-3) / 1e12, 1),
                             "frac_mfma_peak": round(cc["flops_offdiag"] / (ms["offdiag"] * 1e-3) / 1e12 /
                                                     PEAK_BF16_TFLOPS, 4)},
            "diag_step": {"ms": round(ms["diag"], 4), "flops": cc["flops_diag"],
                          "TFLOP/s": round(cc["flops_diag"] / (ms["diag"] * 1e-3) / 1e12, 1)},
            "merge": {"ms": round(ms["merge"], 4), "bytes": cc["bytes_merge"],
                      "GB/s": round(cc["bytes_merge"] / (ms["merge"] * 1e-3) / 1e9, 1)},
        }
        log(f"[bench] context-parallel step {ms['offdiag']:.3f} ms (diagonal {ms['diag']:.3f} ms), "
            f"merge {ms['merge']:.3f} ms")
        del cc, timer

    backward_obj = None
    if args.profile is None and not args.no_backward:
        calls = backward_calls()
        timer = Timer(torch)
        settle(torch, list(calls.values()), args.warmup, args.settle_seconds)
        for _ in range(args.steps):
            for name, fn in calls.items():
                timer.run(name, fn)
        torch.cuda.synchronize()
        backward_obj = {
            "workload": "backward of the same two layers (dq, dk, dv, dsinks; dO ~ N(0,1) bf16), "
                        "q and k rotated inside the call",
            "flop_count": "10 * D * Hq per visible (query, key) pair: recomputed S, dP, dV, dQ, dK "
                          "(the kernels execute 14: S and dP are formed in both the dq and the dk/dv kernel)",
        }
        for name, fl in (("full", flops_full), ("window128", flops_win)):
            ms = timer.mean_ms(name)
            bfl = fl * 5 // 2
            backward_obj[name] = {"ms": round(ms, 4), "TFLOP/s": round(bfl / (ms * 1e-3) / 1e12, 2), "flops": bfl,
                                  "frac_mfma_peak": round(bfl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] backward full {backward_obj['full']['ms']:.3f} ms "
            f"({backward_obj['full']['TFLOP/s']:.0f} TFLOP/s), window {backward_obj['window128']['ms']:.3f} ms")
        del calls, timer

    # ---------------- decode ----------------
    decode_obj = None
    if not args.no_decode or args.profile in ("decode-full", "decode-paged", "decode-ring", "kv-append"):
        log("[bench] generating decode workload: 64 sequences, lengths uniform in [1024, 32768]")
        dinp = wl.decode64()
        dq = dinp.q.to(dev)
        kc = dinp.k_cache.to(dev)
        vc = dinp.v_cache.to(dev)
        lens = dinp.cache_seqlens.to(dev)
        dsinks = dinp.sinks.to(dev)
        for w, nm in ((0, "full"), (WINDOW, "window128")):
            cpu_samples.append(("decode_64seq", nm, "decode", (dinp.q, dinp.k_cache, dinp.v_cache, dinp.lengths,
                                                               dinp.sinks.double().numpy(), w)))
        dtable = gx.rope_table(kc.shape[1])
        d_out = torch.empty_like(dq)
        dws = torch.empty(gx.decode_workspace_size(dq.shape[0], 64, kc.shape[1]), dtype=torch.uint8, device=dev)

        def dec(w):
            return lambda: gx.attn_decode(dq, kc, vc, lens, dsinks, window=w, table=dtable, out=d_out,
                                          workspace=dws)

        if args.profile == "decode-full":
            settle_clock(torch, dev, args.settle)
            for _ in range(args.steps):
                dec(0)()
            torch.cuda.synchronize()
            log(f"decode-full: {args.steps} launches")
            return
        kvc = kv_cache_calls(torch, gx, wl, dev, dq, kc, vc, lens, dsinks, dtable, dinp.lengths, d_out, k, v)
        if args.profile in ("decode-paged", "decode-ring", "kv-append"):
            fn = kvc[{"decode-paged": "paged_full", "decode-ring": "ring_window", "kv-append": "append_1"}[args.profile]]
            settle_clock(torch, dev, args.settle)
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            log(f"{args.profile}: {args.steps} launches")
            return
        timer = Timer(torch)
        settle(torch, [dec(0), dec(WINDOW)], args.warmup, args.settle_seconds)
        for _ in range(args.steps):
            timer.run("dfull", dec(0))
            flush()   # the window layer's 17.8 MB of rows would otherwise be served from the last-level cache
            timer.run("dwin", dec(WINDOW))
        torch.cuda.synchronize()
        ms_df, ms_dw = timer.mean_ms("dfull"), timer.mean_ms("dwin")
        b_full = wl.decode_bytes(dinp.lengths, 0)
        b_win = wl.decode_bytes(dinp.lengths, WINDOW)
        gbs = b_full / (ms_df * 1e-3) / 1e9
        decode_obj = {
            "workload": "decode: 64 sequences x 1 token, cache lengths uniform in [1024, 32768] "
                        f"(sum {sum(dinp.lengths)}), Hq=64 Hkv=8 D=64, bf16 cache",
            "value": round(gbs, 1), "unit": "GB/s", "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "ms_full_layer": round(ms_df, 4), "ms_window_layer": round(ms_dw, 4),
            "bytes_full_layer": b_full, "bytes_window_layer": b_win,
            "window_layer_GBps": round(b_win / (ms_dw * 1e-3) / 1e9, 1),
            "window_layer_cache": "a 512 MiB buffer written before each timed call",
            "frac_of_copy": round(gbs / copy_gbs, 4) if copy_gbs else None,
            "traffic": counters_traffic("decode_full_64seq", "decode"),
        }
        log(f"[bench] decode full {ms_df:.3f} ms = {gbs:.0f} GB/s; window {ms_dw:.4f} ms")
        decode_obj["kv_cache"] = kv_cache_bench(torch, wl, kvc, args, dinp.lengths, b_full, b_win, flush)
        del kc, vc, kvc

    tflops = (flops_full + flops_win) / (ms_step * 1e-3) / 1e12
    achieved = flops_full / (ms_full * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "dense BSHD prefill B=4 S=4096 Hq=64 Hkv=8 D=64: YaRN table + full-causal layer + "
                        "window-128 layer, q and k rotated inside each attention call",
            "global_batch": q.shape[0], "seq_len": S, "parallelism": "none (1 GPU)",
            "k_rotation": args.k_rotation,
        },
        "roofline": {
            "kernel": "prefill full-causal layer (gptoss_attn_prefill, window=0)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": counters_traffic("prefill_full_dense_B4_S4096", "prefill"),
            "flops_per_launch": flops_full,
            "ms_per_launch": round(ms_full, 4),
        },
        "layers": {
            "full": {"ms": round(ms_full, 4), "TFLOP/s": round(achieved, 2), "flops": flops_full},
            "window128": {"ms": round(ms_win, 4), "TFLOP/s": round(flops_win / (ms_win * 1e-3) / 1e12, 2),
                          "GB/s": round(bytes_prefill / (ms_win * 1e-3) / 1e9, 1),
                          "frac_hbm_peak": round(bytes_prefill / (ms_win * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "frac_of_copy": round(bytes_prefill / (ms_win * 1e-3) / 1e9 / copy_gbs, 4),
                          "flops": flops_win, "bytes": bytes_prefill,
                          "traffic": counters_traffic("prefill_window128_dense_B4_S4096", "window")},
            "table_ms": round(ms_table, 5),
        },
        "device": {"name": torch.cuda.get_device_name(dev),
                   "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
                   "copy_GBps": round(copy_gbs, 1), "copy_frac_hbm_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
                   "copy": "1 GiB device-to-device copy (torch copy_), 2 GiB moved per call, HIP events",
                   "fill_GBps": round(fill_gbs, 1), "fill": "1 GiB written by torch fill_ (write only)",
                   "clock_settle_s": args.settle_seconds,
                   "clock_settle": "each timed section first runs its own calls for clock_settle_s seconds and "
                                   "then `warmup` rounds, all untimed"},
        "prefill_thd_and_long": other_obj,
        "backward": backward_obj,
        "projection": projection_obj,
        "context_parallel": cp_obj,
        "decode": decode_obj,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline, ~{args.cpu_seconds:.0f} s")
        ti0 = wl.tiny()
        dq0, dk0, dv0 = (inp.q[0].double().numpy(), inp.k[0].double().numpy(), inp.v[0].double().numpy())
        drows = __import__("numpy").random.default_rng(2024).permutation(S)
        head = []
        for w, nm in ((0, "full"), (WINDOW, "window128")):
            head.append(("tiny_S256", nm, "rows", (ti0.q[0].double().numpy(), ti0.k[0].double().numpy(),
                                                   ti0.v[0].double().numpy(), ti0.sinks.double().numpy(), w,
                                                   list(range(256)))))
            head.append(("dense_B4_S4096_batch0", nm, "rows", (dq0, dk0, dv0, inp.sinks.double().numpy(), w,
                                                               drows)))
        result["cpu_baseline"] = cpu_baseline(head + cpu_samples, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
