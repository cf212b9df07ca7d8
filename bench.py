"""Benchmark of the MFA decode-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--pools P]

A step is one decode-attention call (block-table walk, K/V tile loads,
QK^T and PV on MFMA, online softmax, split combine) over one batch of
synthetic input already resident in HBM.  Default workload: 64 slots x 4096
keys, 64 query heads sharing one 256-wide K/V head, bf16, paged 64-token
blocks in a shuffled pool.  The K/V pool is replicated P times and the steps
rotate through the copies so that the 256 MB Infinity Cache cannot serve a
repeat of the previous step.  Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn query tokens/s + achieved HBM GB/s (% peak), MFA 4K ctx, batch 64"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
PAGE = 64


def log(msg):
    print(msg, file=sys.stderr, flush=True)


WORKLOADS = {
    2: "MFA decode: B=64, every context 4096, 64 q heads / 1 KV head, d=256, bf16 q/K/V, "
       "paged 64-token blocks, shuffled pool",
    3: "MFA decode: B=128 ragged (prefill U[1024,8192] + Geo(1/1024) decode index), bf16, paged",
    4: "MFA decode from the hidden state: B=256, low-rank query path (x [256, 7168] -> 2048 -> "
       "RMSNorm -> 64 x 256, bf16 weights) into attention over context 4096, FP8 E4M3 K/V with "
       "per-head scales, paged",
    5: "GQA 64/4/192 decode: B=32, context 32768, dense global layer, bf16, paged",
    6: "GQA 64/4/192 decode: B=32, context 32768, 512-token sliding window, bf16, paged",
}


def make_case(config, fp8=False):
    """Host-drawn inputs for configs 2-4; the Step-5 layer (5: global, 6: local
    window) is drawn on the device (its 1.6 GB pool takes minutes on the host),
    with an E4M3 cache (per-group scales) when fp8 is set."""
    from workloads import config_case
    if config in (2, 3, 4):
        return config_case(config, nan_tail=False)
    if config in (5, 6):
        from workloads.device_gen import make_device_case
        return make_device_case(5, batch=32, ctx_lens=[32768] * 32, hq=64, hkv=4, d=192,
                                window=512 if config == 6 else 0, nan_tail=False,
                                kv_format="e4m3" if fp8 else "bf16", name=f"c{config}")
    raise SystemExit(f"unknown --config {config}")


def cpu_baseline(case, budget_s, single_thread_s=0.0, qi=None):
    """The oracle as it stands, on the host cores: it evaluates the slots of
    the same workload one after another (cycling through the batch) until
    about budget_s seconds have passed; one slot evaluation is one query
    token's decode step (with qi, the query inputs of config 4, the oracle's
    query path first, its exact query then feeding the attention).  A
    second, shorter run limits the BLAS pool to one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import decode_attention, query_proj
    kw = case.oracle_kwargs()
    q = case.q
    if qi is not None:
        q = np.zeros((case.batch, case.hq, case.d))
        kw["q_format"] = "f64"

    def run(seconds):
        done = 0
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) < seconds:
            b = done % case.batch
            if qi is not None:
                q[b] = query_proj(qi.x[b:b + 1], qi.w_down, qi.w_up, fmt="bf16", eps=qi.eps,
                                  num_heads=case.hq, head_dim=case.d)[0]
            decode_attention(q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                             slots=[b], **kw)
            done += 1
        return done, time.perf_counter() - t0

    done, el = run(budget_s)
    info = threadpool_info()
    blas = [i for i in info if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    res = {"value": done / el, "unit": "query tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{done} slot evaluations ({done / case.batch:.1f} passes over the "
                     f"{case.batch} slots of the same workload), fp64 numpy oracle, {el:.1f} s",
           "host_cpu_count": os.cpu_count(),
           "blas": [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '')}"
                    f"{', ' + i['architecture'] if i.get('architecture') else ''})" for i in blas]}
    if single_thread_s > 0:
        with threadpool_limits(limits=1, user_api="blas"):
            done1, el1 = run(single_thread_s)
        res["single_thread"] = {"value": done1 / el1, "unit": "query tokens/s", "cores": 1,
                                "sample": f"{done1} slot evaluations, {el1:.1f} s"}
    return res


# Sources whose change invalidates the committed counter summary.
TRAFFIC_SOURCES = ["decode_mqa.hip", "decode_gqa.hip", "combine.hip", "device_common.h",
                   "kernel_params.h", "host_plan.cpp"]


def source_digest():
    import hashlib
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_mfa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Committed rocprofv3 counter summaries, by --config.
COUNTER_SUMMARIES = {2: "mqa_decode_b64_l4096_bf16_counters.txt",
                     4: "mqa_decode_b256_l4096_fp8_counters.txt"}


def committed_counters(config):
    """(HBM bytes per call, MFMA utilisation of the attention kernel) from the
    committed rocprofv3 counter summary of this workload; (None, None) when
    there is none or the kernels changed since it was taken."""
    name = COUNTER_SUMMARIES.get(config)
    path = os.path.join(ROOT, "profiles", name) if name else ""
    if not name or not os.path.exists(path):
        return None, None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_digest") != source_digest():
        return None, None
    try:
        return float(fields["traffic_bytes_per_call"]), float(fields["mfma_util"])
    except (KeyError, ValueError):
        return None, None


def stream_read_rate(nbytes, steps, warmup, stream):
    """Time mfa_stream_read over nbytes (rounded down to whole 16-byte loads):
    the read rate a kernel with no other work reaches on this GPU."""
    import torch
    import decode_attention_mfa_amd as mfa
    n = (int(nbytes) // 16) * 4
    bufs = [torch.full((n,), i + 1, dtype=torch.int32, device="cuda") for i in range(4)]
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.int32, device="cuda")
    for i in range(max(warmup, 4)):
        mfa.mfa_stream_read(bufs[i % 4], sink, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        mfa.mfa_stream_read(bufs[i % 4], sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del bufs
    return {"achieved": n * 4 / us * 1e-3, "unit": "GB/s", "us": us, "bytes": n * 4,
            "frac_of_peak": n * 4 / us * 1e-3 / HBM_PEAK_GBPS,
            "timed": "mfa_stream_read (16-byte non-temporal loads, one workgroup per compute "
                     "unit) over the call's algorithmic bytes, K back-to-back launches under "
                     "one event pair"}


def copy_calibration(steps):
    """A plain device-to-device copy of a known size (1 GiB per dispatch), run
    under rocprofv3 --pmc to scale the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": n, "dispatches": steps}), flush=True)


def sparse_step(steps, warmup, batch=32, ctx=32768):
    """Time the Step-5 sparse global attention decode step on the global
    layer's shape (B requests of ctx tokens, 64 q heads / 4 KV groups / 192,
    bf16, paged): indexer scores + top-512 selection, then attention over the
    selected blocks and the current block.  The block summaries are built
    once beforehand (a decode step adds at most one per request) and timed
    on their own."""
    import torch
    import decode_attention_mfa_amd as mfa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pages = ctx // PAGE
    n_blocks = batch * pages
    gen = torch.Generator(device=dev)
    gen.manual_seed(909)
    k = torch.randn((n_blocks, 4, PAGE, 192), generator=gen, device=dev, dtype=torch.bfloat16)
    v = torch.randn((n_blocks, 4, PAGE // 8, 192, 8), generator=gen, device=dev, dtype=torch.bfloat16)
    table = torch.from_numpy(np.random.default_rng(910).permutation(n_blocks).astype(np.int32)
                             .reshape(batch, pages)).to(dev)
    lens = torch.full((batch,), ctx, dtype=torch.int32, device=dev)
    q = torch.randn((batch, 64, 192), generator=gen, device=dev, dtype=torch.bfloat16)
    q_idx = torch.randn((batch, 4, 4, 256), generator=gen, device=dev, dtype=torch.bfloat16)
    w = torch.randn((batch, 4, 4), generator=gen, device=dev) * 0.5
    k_idx = torch.randn((batch, ctx, 256), generator=gen, device=dev, dtype=torch.bfloat16)
    z = torch.randn((batch, ctx, 256), generator=gen, device=dev, dtype=torch.bfloat16)
    summ = torch.zeros((batch, pages * 8, 256), dtype=torch.uint8, device=dev)
    sel = torch.empty((batch, 4, 512), dtype=torch.int32, device=dev)
    nsel = torch.empty((batch, 4), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    scale = 1.0 / np.sqrt(192)

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    t_sum = timed(lambda: mfa.mfa_sparse_summarize(k_idx, z, lens, summ, block_table=table), 5)
    t_sel = timed(lambda: mfa.mfa_sparse_select(q_idx, w, summ, lens, sel, nsel,
                                                block_table=table), steps)
    t_att = timed(lambda: mfa.mfa_sparse_attention(q, k, v, table, lens, sel, nsel, out, scale),
                  steps)

    def step():
        mfa.mfa_sparse_select(q_idx, w, summ, lens, sel, nsel, block_table=table)
        mfa.mfa_sparse_attention(q, k, v, table, lens, sel, nsel, out, scale)
    t_step = timed(step, steps)
    cand = (ctx - 1) // 8
    tokens = 512 * 8 + (ctx - 1) % 8 + 1                       # |J| per (request, group)
    att_bytes = batch * (4 * tokens * 192 * 2 * 2 + 64 * 192 * 2 * 2)
    sel_bytes = batch * (cand * 256 + 16 * 256 * 2 + 16 * 4 + 4 * 512 * 4)
    nbytes = att_bytes + sel_bytes
    print(json.dumps({
        "metric": "Step-5 sparse global attention decode step (select + attention)",
        "value": batch / t_step, "unit": "query tokens/s", "ms_per_step": t_step * 1e3,
        "config": {"workload": f"Step-5 global sparse layer: B={batch}, context {ctx}, 64 q heads / "
                               "4 KV groups / d=192 bf16, indexer 4x4x256, 8-token blocks, top-512",
                   "batch": batch, "ctx": ctx},
        "select_us": t_sel * 1e6, "attention_us": t_att * 1e6,
        "summaries_all_blocks_us": t_sum * 1e6,
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "achieved": nbytes / t_step / 1e9, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": nbytes / t_step / 1e9 / HBM_PEAK_GBPS,
                     "traffic": None},
        "dense_kv_bytes_per_step": batch * 4 * ctx * 192 * 2 * 2}), flush=True)


def latency_model(steps, warmup):
    """Fit the attention-FFN ratio page's attention latency model
    t_A = alpha_A * T + beta_A to this library on one GPU: MFA decode calls
    (64 heads, one 256-wide K/V head, paged) over uniform batches, B slots of
    L keys each, T = B * L cached tokens; bf16 and FP8 caches.  Each call
    reads blocks no other call of the sweep point reads (the pool is cycled
    through), so the timings are HBM timings, not cache hits."""
    import torch
    import decode_attention_mfa_amd as mfa
    from decode_attention_mfa_amd import accounting
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_blocks = 32768                                   # 2M tokens, 1 GiB per bf16 pool
    gen = torch.Generator(device=dev)
    gen.manual_seed(707)
    kb = torch.randn((n_blocks, 1, PAGE, 256), generator=gen, device=dev, dtype=torch.bfloat16)
    vb = torch.randn((n_blocks, 1, 256, PAGE), generator=gen, device=dev, dtype=torch.bfloat16)
    pools = {"bf16": (kb, vb, None),
             "e4m3": (kb.to(torch.float8_e4m3fn), vb.to(torch.float8_e4m3fn),
                      torch.ones(1, dtype=torch.float32, device=dev))}
    perm = torch.from_numpy(np.random.default_rng(708).permutation(n_blocks).astype(np.int32)).to(dev)
    fits = {}
    for fmt, (k, v, sc) in pools.items():
        pts = []
        for B in (16, 32, 64, 128, 256):
            for L in (1024, 2048, 4096, 8192):
                nb = L // PAGE
                need = B * nb
                sets = max(1, n_blocks // need)
                tables = [perm[j * need:(j + 1) * need].view(B, nb) for j in range(sets)]
                lens = torch.full((B,), L, dtype=torch.int32, device=dev)
                q = torch.randn((B, 64, 256), generator=gen, device=dev, dtype=torch.bfloat16)
                out = torch.empty_like(q)

                def call(i):
                    mfa.mfa_decode_attention(q, k, v, tables[i % sets], lens, out, 1.0 / 16,
                                             k_scale=sc, v_scale=sc)
                for i in range(warmup):
                    call(i)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(steps):
                    call(warmup + i)
                e1.record()
                torch.cuda.synchronize()
                pts.append((B, L, B * L, e0.elapsed_time(e1) * 1e-3 / steps))
                log(f"latency model {fmt}: B={B} L={L} {pts[-1][3] * 1e6:.1f} us")
        alpha, beta, r2 = accounting.fit_latency_model([x[2] for x in pts], [x[3] for x in pts])
        kv_bytes = 2 * 256 * accounting.DTYPE_BYTES[fmt]
        fits[fmt] = {"alpha_A_ns_per_token": alpha * 1e9, "beta_A_us": beta * 1e6, "r2": r2,
                     "kv_bytes_per_token": kv_bytes,
                     "bandwidth_of_alpha_GBps": kv_bytes / alpha / 1e9,
                     "points_B_L_us": [[b, l, round(t * 1e6, 2)] for b, l, _, t in pts]}
    print(json.dumps({"latency_model": "t_A = alpha_A * T + beta_A (T = sum of context lengths)",
                      "workload": "MFA decode, 64 q heads / 1 KV head, d=256, paged, uniform "
                                  "lengths, B in {16..256}, L in {1K..8K}",
                      "steps_per_point": steps, "fits": fits}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--pools", type=int, default=4)
    ap.add_argument("--prewarm", type=float, default=0.3,
                    help="seconds of untimed steps before the warmup steps (GPU clock ramp)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--fp8", action="store_true",
                    help="configs 5 and 6 with an E4M3 cache (one fp32 scale per KV group)")
    ap.add_argument("--v-layout", choices=["channel", "subblock8"], default="channel",
                    help="V pool layout of the per-group configs (5, 6): channel-major, or "
                         "the 8-token sub-blocks the sparse global attention reads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph instead of launching it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--with-append", action="store_true",
                    help="each step appends one token per slot (mfa_kv_append, length "
                         "advanced on the device) before the attention; lengths start "
                         "steps+warmup below the workload's and grow to it")
    ap.add_argument("--mtp", type=int, default=1,
                    help="query tokens per slot (multi-token decode, causal among them; the "
                         "contexts count them); dense one-KV-head configs only")
    ap.add_argument("--latency-model", action="store_true",
                    help="fit t_A = alpha_A * T + beta_A over a sweep of batch sizes and "
                         "context lengths (bf16 and FP8 caches) and print the fits")
    ap.add_argument("--sparse", action="store_true",
                    help="time the Step-5 sparse global attention decode step (B=32, 32K "
                         "context) and print its own line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the decode path shards by slot with no cross-GPU traffic, so run one "
              "process per GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.sparse:
        sparse_step(min(args.steps, 50), min(args.warmup, 5))
        return
    if args.latency_model:
        latency_model(min(args.steps, 30), min(args.warmup, 5))
        return

    import torch
    import decode_attention_mfa_amd as mfa
    from decode_attention_mfa_amd import accounting
    from workloads.torch_io import to_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: building config {args.config} inputs")
    if args.fp8 and args.config not in (5, 6):
        raise SystemExit("--fp8 selects the E4M3 cache of configs 5 and 6 (config 4 is E4M3 already)")
    case = make_case(args.config, fp8=args.fp8)
    if hasattr(case, "host_slots"):   # drawn on the device
        t = {"q": case.q, "k": case.k, "v": case.v, "table": case.table, "lens": case.lens,
             "k_scale": case.k_scale, "v_scale": case.v_scale,
             "out": torch.empty((case.batch, case.hq, case.d), dtype=torch.bfloat16, device=dev)}
        cpu_case = case.host_slots([0, 1])
    else:
        t = to_device(case, device=dev)
        cpu_case = case
    qpath = None
    if t["q"] is None:
        # Config 4: the step starts from the hidden state.  The low-rank query
        # path (x [B, 7168] -> W_qdown -> RMSNorm -> W_qup -> 64 x 256) writes
        # the bf16 queries the FP8-cache attention then reads.
        from workloads import config_query_inputs
        qi = config_query_inputs(4, batch=case.batch)

        def dev_bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
                torch.bfloat16).to(dev)
        qpath = {"x": dev_bf16(qi.x), "wd": dev_bf16(qi.w_down.T), "wu": dev_bf16(qi.w_up.T),
                 "eps": qi.eps, "hidden": qi.x.shape[1], "rank": qi.w_down.shape[1]}
        t["q"] = torch.empty((case.batch, case.hq, case.d), dtype=torch.bfloat16, device=dev)

    def query_path():
        mfa.mfa_query_proj(qpath["x"], qpath["wd"], qpath["wu"], t["q"].view(case.batch, -1),
                           num_heads=case.hq, eps=qpath["eps"])
    if args.v_layout != "channel":
        if case.hkv == 1 or args.mtp != 1:
            raise SystemExit("--v-layout subblock8 is read by the per-group configs (5, 6)")
        nb_, hkv_, d_, page_ = t["v"].shape
        t["v"] = t["v"].view(nb_, hkv_, d_, page_ // 8, 8).permute(0, 1, 3, 2, 4).contiguous()
    pools = [(t["k"], t["v"])]
    for _ in range(max(0, args.pools - 1)):
        pools.append((t["k"].clone(), t["v"].clone()))
    out = t["out"]
    window = case.window
    tq = args.mtp
    if tq != 1:
        if case.hkv != 1 or window or args.with_append or tq < 1:
            raise SystemExit("--mtp takes a dense one-KV-head config (2, 3 or 4), without "
                             "--with-append")
        from workloads import make_mtp_queries
        qm = make_mtp_queries(606, batch=case.batch, tq=tq, hq=case.hq, d=case.d)
        t["q"] = torch.from_numpy(qm.view(np.int16)).view(torch.bfloat16).to(dev)
        out = torch.empty((case.batch, tq, case.hq, case.d), dtype=torch.bfloat16, device=dev)
    n_calls = max(args.warmup, len(pools)) + args.steps
    if args.with_append:
        # A decode loop: the device-side lengths start n_calls below the
        # workload's and grow by one per step; the new tokens are fixed.
        if args.graph:
            raise SystemExit("--with-append times eager launches (graph warm-up replays would "
                             "advance the lengths past the accounted ones)")
        if window or np.min(case.ctx_lens) < n_calls:
            raise SystemExit("--with-append needs a dense config with contexts >= steps + warmup")
        t["lens"] = torch.from_numpy((case.ctx_lens - n_calls).astype(np.int32)).to(dev)
        rng_new = np.random.default_rng(505)
        from workloads import bf16_round_bits
        new_kv = [torch.from_numpy(bf16_round_bits(rng_new.standard_normal(
            (case.batch, case.hkv, case.d), dtype=np.float32)).view(np.int16)).view(
            torch.bfloat16).to(dev) for _ in range(2)]

    def call(i):
        k, v = pools[i % len(pools)]
        if qpath is not None:
            query_path()
        if args.with_append:
            mfa.mfa_kv_append(new_kv[0], new_kv[1], k, v, t["table"], t["lens"],
                              k_scale=t["k_scale"], v_scale=t["v_scale"])
        if tq != 1:
            mfa.mfa_decode_attention_mtp(t["q"], k, v, t["table"], t["lens"], out, case.scale,
                                         k_scale=t["k_scale"], v_scale=t["v_scale"],
                                         num_splits=args.num_splits)
        elif case.hkv == 1 and window == 0:
            mfa.mfa_decode_attention(t["q"], k, v, t["table"], t["lens"], out, case.scale,
                                     k_scale=t["k_scale"], v_scale=t["v_scale"],
                                     num_splits=args.num_splits)
        else:
            mfa.mfa_decode_attention_gqa(t["q"], k, v, t["table"], t["lens"], out, case.scale,
                                         window=window, k_scale=t["k_scale"],
                                         v_scale=t["v_scale"], num_splits=args.num_splits,
                                         v_layout=args.v_layout)

    # Untimed pre-warm: the GPU raises its clocks over a few hundred
    # microseconds of load, so the same step is run for args.prewarm seconds
    # before the warmup steps; the timed steps then see steady-state clocks
    # (a handful of warmup steps alone left the first timed steps 10-20 %
    # slower than the rest).
    log(f"bench: pre-warm {args.prewarm:.2f} s")
    t_end = time.perf_counter() + args.prewarm
    i = 0
    while time.perf_counter() < t_end:
        call(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"bench: warmup {args.warmup}")
    for i in range(max(args.warmup, len(pools))):
        call(i)
    torch.cuda.synchronize()
    step = call
    if args.graph:
        # The same launches replayed from captured graphs (one per pool copy).
        graphs = []
        for i in range(len(pools)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()

        def step(i):
            graphs[i % len(graphs)].replay()
    # One HIP event pair brackets the K timed steps on the launch stream (an
    # event pair around every call would add its own marker packets, several
    # microseconds each, between the kernels it measures).
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = wall * 1e3 / args.steps
    call_ms = start.elapsed_time(end) / args.steps

    # Per-call distribution (the survey's protocol): a HIP event pair around
    # every step of a second pass.  The markers add their own packets between
    # the kernels, so these figures sit a few microseconds above the
    # back-to-back mean; they are reported for the spread, not as the rate.
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        pairs[i][0].record(stream)
        step(i)
        pairs[i][1].record(stream)
    torch.cuda.synchronize()
    per_call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])

    # The attention kernel alone (the roofline's kernel): K back-to-back
    # launches of the call's first phase (attention without the merge) under
    # one event pair on the launch stream, rotating through the pool copies
    # like the steps.  No marker sits between the launches, so the mean is
    # the kernel's own duration plus the dispatch gap, as rocprofv3 sees it.
    kernel_ms = None
    if tq == 1 and case.hkv == 1 and window == 0 and not args.graph and not args.with_append:
        kw = dict(k_scale=t["k_scale"], v_scale=t["v_scale"], num_splits=args.num_splits)

        def attention_only(i):
            k, v = pools[i % len(pools)]
            mfa.mfa_decode_attention_phase(t["q"], k, v, t["table"], t["lens"], out, case.scale, 1,
                                           **kw)
        for i in range(max(args.warmup, len(pools))):
            attention_only(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            attention_only(i)
        e1.record(stream)
        torch.cuda.synchronize()
        kernel_ms = e0.elapsed_time(e1) / args.steps

    # The query path alone (config 4): K back-to-back calls under one event
    # pair, against its own roofline max(bytes / HBM peak, FLOPs / bf16 MFMA
    # peak) ("Step-3 is Large yet Affordable", section 4: the cost model's
    # max form).
    qpath_res = None
    if qpath is not None:
        for _ in range(args.warmup):
            query_path()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            query_path()
        e1.record(stream)
        torch.cuda.synchronize()
        qp_us = e0.elapsed_time(e1) * 1e3 / args.steps
        qp_bytes, qp_flops = accounting.query_proj_work(case.batch, hidden=qpath["hidden"],
                                                        rank=qpath["rank"], heads=case.hq,
                                                        head_dim=case.d)
        floor_us = max(qp_bytes / (HBM_PEAK_GBPS * 1e3), qp_flops / (MFMA_BF16_PEAK_TFLOPS * 1e6))
        qpath_res = {"us": qp_us, "bytes": qp_bytes, "flops": qp_flops, "floor_us": floor_us,
                     "frac_of_floor": floor_us / qp_us,
                     "achieved_GBps": qp_bytes / qp_us * 1e-3,
                     "achieved_TFLOPs": qp_flops / qp_us * 1e-6,
                     "timed": "one HIP event pair around K back-to-back query-path calls"}
        # Context only: the vendor BLAS (torch.matmul -> hipBLASLt) on the same
        # two products and layouts, timed the same way.
        r_ctx = torch.ones(case.batch, qpath["rank"], dtype=torch.bfloat16, device="cuda")
        lib_us = {}
        for name, fn in (("down", lambda: torch.matmul(qpath["x"], qpath["wd"].t())),
                         ("up", lambda: torch.matmul(r_ctx, qpath["wu"].t()))):
            for _ in range(args.warmup):
                fn()
            cur = torch.cuda.current_stream()
            e0.record(cur)
            for _ in range(args.steps):
                fn()
            e1.record(cur)
            torch.cuda.synchronize()
            lib_us[name] = e0.elapsed_time(e1) * 1e3 / args.steps
        qpath_res["vendor_blas_gemm_us"] = lib_us

    fmt_kv = case.kv_format
    append_bytes = 0
    if args.with_append:
        # Lengths the timed steps' attention saw (after their appends), and
        # the append's own bytes: new K/V read, cache rows written, lengths.
        first = case.ctx_lens - n_calls + max(args.warmup, len(pools)) + 1
        nbytes = float(np.mean([accounting.decode_call_bytes(
            first + i, hq=case.hq, hkv=case.hkv, d=case.d, q_fmt="bf16", kv_fmt=fmt_kv,
            out_fmt=case.out_format, window=window) for i in range(args.steps)]))
        elem = {"bf16": 2, "e4m3": 1, "f32": 4}[fmt_kv]
        append_bytes = case.batch * (2 * case.hkv * case.d * (2 + elem) + 8)
        nbytes += append_bytes
    else:
        # Multi-token: each sequence's K/V once, and Tq rows of q and out.
        nbytes = accounting.decode_call_bytes(case.ctx_lens, hq=case.hq * tq, hkv=case.hkv,
                                              d=case.d, q_fmt="bf16", kv_fmt=fmt_kv,
                                              out_fmt=case.out_format, window=window)
    flops = sum(accounting.decode_call_flops(np.maximum(case.ctx_lens - (tq - 1 - j), 0),
                                             hq=case.hq, d=case.d, window=window)
                for j in range(tq))
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    kernel_achieved = nbytes / (kernel_ms * 1e-3) / 1e9 if kernel_ms else None
    # Split count of the query slots (a pair of tokens per slot for even Tq).
    slots = case.batch * (tq // 2 if tq % 2 == 0 else tq)
    desc = mfa.decode_desc(t["q"][:slots] if tq == 1 else t["q"].view(-1, case.hq, case.d)[:slots],
                           t["k"], t["table"], out.view(-1, case.hq, case.d)[:slots],
                           args.num_splits)
    splits = mfa.mfa_decode_plan_splits(desc, window,
                                        torch.cuda.get_device_properties(dev).multi_processor_count)

    # The read rate of a kernel that only streams, measured in the same run:
    # the library's plain streaming-read kernel over the call's algorithmic
    # byte count (the attention's, for config 4), K back-to-back launches
    # under one event pair, rotating over four buffers like the pool copies.
    # A practical reference below the published peak, not a bound: the
    # per-group kernel matches it on the 32K global layer.
    stream_ref = stream_read_rate(nbytes, args.steps, args.warmup, stream)

    counters = committed_counters(args.config) if not args.with_append else (None, None)
    if qpath is not None:
        nbytes += qpath_res["bytes"]
        flops += qpath_res["flops"]
        achieved = nbytes / (call_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": case.batch * tq / (ms_per_step * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "e4m3": "fp8_e4m3 storage, bf16 MFMA", "f32": "f32"}[fmt_kv],
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "batch": case.batch,
                   "ctx_len_mean": float(np.mean(case.ctx_lens) - (
                       (n_calls - max(args.warmup, len(pools)) - 1 - (args.steps - 1) / 2)
                       if args.with_append else 0.0)), "q_heads": case.hq,
                   "kv_heads": case.hkv, "head_dim": case.d, "kv_dtype": fmt_kv,
                   "page": 64, "window": window, "splits": splits, "kv_pool_copies": len(pools),
                   "launch": "hip graph replay" if args.graph else "eager",
                   "prewarm_s": args.prewarm,
                   "append": bool(args.with_append), "query_tokens_per_slot": tq,
                   "v_layout": args.v_layout},
        "hbm_gbps": achieved,
        "hbm_frac_of_peak": achieved / HBM_PEAK_GBPS,
        "call_us_mean": call_ms * 1e3,
        "call_us_percentiles": {
            "p10": float(np.percentile(per_call_us, 10)), "p50": float(np.median(per_call_us)),
            "p90": float(np.percentile(per_call_us, 90)),
            "timed": "a HIP event pair around each step of a second pass (markers between "
                     "the steps add their own time)"},
        "algorithmic_bytes_per_call": nbytes,
        "append_bytes_per_call": append_bytes,
        "flops_per_call": flops,
        "roofline": {"bound": "hbm", "achieved": kernel_achieved or achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": (kernel_achieved or achieved) / HBM_PEAK_GBPS,
                     "kernel_us": kernel_ms * 1e3 if kernel_ms else None,
                     "step_achieved": achieved, "step_frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counters[0] if tq == 1 else None,
                     "mfma_util": counters[1] if tq == 1 else None,
                     "counters": (f"profiles/{COUNTER_SUMMARIES[args.config]}"
                                  if tq == 1 and counters[0] is not None else None),
                     "timed": ("the attention kernel: one HIP event pair on the launch stream "
                               "around K back-to-back launches of the call's attention phase "
                               "(no merge, no marker between launches); step_*: one event pair "
                               "around the K timed steps (attention + merge)") if kernel_ms else (
                              "one HIP event pair around the timed steps on the launch "
                              "stream, divided by the step count (attention kernel + split "
                              "merge kernel per step" + (", after the KV append)" if
                                                        args.with_append else ")"))},
    }
    res["roofline"]["stream_read"] = dict(
        stream_ref, kernel_frac=(kernel_achieved / stream_ref["achieved"]) if kernel_achieved else None,
        step_frac=achieved / stream_ref["achieved"] if qpath is None else None)
    if qpath_res is not None:
        res["query_path"] = qpath_res
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample of the same workload")
        res["cpu_baseline"] = cpu_baseline(cpu_case, args.cpu_seconds,
                                           single_thread_s=args.cpu_seconds / 2,
                                           qi=qi if qpath is not None else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
