"""Benchmark: one MLA decode step (one layer) at the DeepSeek-V2 shape on one MI355X.

A step is absorb_q -> rope (append) -> decode_attn -> combine -> absorb_out over one batch of
synthetic inputs resident in HBM. Prints ONE JSON line with whole-step throughput (tokens/s),
the latent-cache read bandwidth of the attention kernels, the roofline record of the dominant
kernel (decode_attn) timed with HIP events on its launch stream, and the CPU oracle timed on a
bounded sample of the same workload.

Default workload: batch 64, every sequence 4096 tokens (contiguous bf16 latent cache
[64, 4096, 576]), n_h=128, d_h=128, d_c=512, d_c'=1536, d_h^R=64, d=5120; hidden states N(0,1),
weights N(0, 0.006). The cache is replicated `--rotate` times and the steps cycle through the
copies so that successive steps do not find the cache in the 256 MB last-level (MALL) cache.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
# HBM bytes per launch of the decode kernel (k_decode_v3 / k_decode_fp8) from rocprofv3 FETCH_SIZE
# (KiB, x2.0) + WRITE_SIZE (KiB, x1.0), both scaled by a plain copy of known size; recorded in
# profiles/decode_attn_config2_hbm_counters.md and profiles/decode_attn_config4_hbm_counters.md for
# the kernels as they stand. Workloads without a recorded measurement report null.
DECODE_TRAFFIC_BYTES = {
    "2": 153666 * 1024 * 2 + 38145 * 1024,
    "4": 297090 * 1024 * 2 + 38144 * 1024,
    "4f8": 150874 * 1024 * 2 + 36864 * 1024,
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="2", help="workload key (0, 1, 2, 3, 4, 4f8, 4f6)")
    ap.add_argument("--splits", type=int, default=0,
                    help="decode ranges (0 = the library's default: one per CU at the V2 shape, two otherwise)")
    ap.add_argument("--rotate", type=int, default=2, help="cache copies cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--graph", action="store_true", help="replay each step as a HIP graph")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the decode_attn sub-records of the other DeepSeek-V2 workloads (configs 3, 4, 4f8, 4f6)")
    ap.add_argument("--prefill", type=int, default=0, metavar="C",
                    help="chunked-prefill mode: C new tokens per sequence after 2048 stored rows, B=16 "
                         "(a separate JSON line; the default run is the decode step)")
    ap.add_argument("--unfused", action="store_true",
                    help="run mla_combine + mla_absorb_out instead of the fused mla_combine_absorb_out")
    ap.add_argument("--naive", action="store_true",
                    help="with --prefill: the naive execution form (keys and values expanded per head)")
    ap.add_argument("--prefix", type=int, default=2048, help="with --prefill: stored rows per sequence")
    ap.add_argument("--precombined", action="store_true",
                    help="the pre-combined absorption variant: W~^Q and W~^O built once, then one product each "
                         "in place of the two-step projections (a separate JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (reference for the HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of known size: each launch reads and writes 256 MiB."""
    import torch
    n = 64 << 20  # float32 elements
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                                           "launches": 5}}), flush=True)


def stream_read_ceiling(mla, nbytes=1 << 30, reps=10):
    """HBM read ceiling measured on this GPU: mla_stream_read (a plain read-only streaming kernel)
    over a buffer four times the last-level cache, timed with HIP events on its launch stream."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(mla.STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    for _ in range(2):
        mla.stream_read(src, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mla.stream_read(src, sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del src
    torch.cuda.empty_cache()
    return nbytes / t / 1e9


def build_cache(mla, case):
    import torch
    cfg, dims = case.cfg, case.dims
    if cfg.layout == "contiguous":
        cache = mla.LatentCache.contiguous(case.B, case.t_cap, dims.row, cfg.cdtype)
    else:
        cache = mla.LatentCache.paged(case.num_pages, cfg.page_size, dims.row, cfg.cdtype, case.block_table)
    if cfg.cdtype not in ("fp8_e4m3", "fp6_e2m3"):
        cache.rows.copy_(case.rows)
    else:
        n_rows = (case.seq_lens - 1).to(torch.int32).contiguous()
        mla.cache_store(mla.Dims.of(dims), cache, n_rows, case.t_cap, case.rows32.contiguous(), case.t_cap)
    return cache


def cpu_baseline(case, budget_s):
    """The oracle as it stands, on whole sequences of this workload until the budget is spent."""
    import numpy as np
    from oracle import OracleDims, decode_step_explicit
    W = {k: v.double().cpu().numpy() for k, v in case.weights.items()}
    od = OracleDims.of(case.dims)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    t0 = time.perf_counter()
    done = 0
    for b in range(case.B):
        pre = case.prefix_rows(b)
        if case.cfg.cdtype == "fp8_e4m3":
            from oracle import e4m3_decode, quantize_rows_e4m3
            codes, sc = quantize_rows_e4m3(pre.float().cpu().numpy())
            pre64 = e4m3_decode(codes) * sc.astype(np.float64)[:, None]
        elif case.cfg.cdtype == "fp6_e2m3":
            from oracle import e2m3_decode, quantize_rows_e2m3
            codes, sc = quantize_rows_e2m3(pre.float().cpu().numpy())
            pre64 = e2m3_decode(codes) * sc.astype(np.float64)[:, None]
        else:
            pre64 = pre.double().cpu().numpy()
        decode_step_explicit(W, case.h[b].double().cpu().numpy(), pre64, od, case.cfg.cdtype)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    T = int(case.seq_lens[0])
    return {"value": done / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {case.B} sequences (T={T} each, full decode step incl. all heads), "
                      f"{dt:.1f} s, numpy float64 explicit K/V reconstruction",
            "cpu_model": _cpu_model(), "blas": _blas_name()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_name():
    try:
        import numpy as np
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:  # numpy without the build-info dictionary
        return None


def decode_subrecord(mla, key, splits):
    """Another DeepSeek-V2 workload, timed the way the main line is: whole decode steps (absorb_q,
    rope, decode_attn, then the fused combine + output call) with HIP events around each call on its
    launch stream. Reports the step and the decode_attn call; the latent-cache bytes over the
    decode_attn call as a fraction of the HBM peak."""
    import numpy as np
    import torch
    from synth import get_config, make_case
    cfg = get_config(key)
    case = make_case(cfg, device="cuda")
    # two copies (cycled) unless one alone outgrows the 256 MB MALL many times over (config 3: 2.5 GB)
    caches = [build_cache(mla, case) for _ in range(1 if key == "3" else 2)]
    step = mla.DecodeStep(cfg.dims, case.B, splits, fused="auto")
    d, W, h, seq_lens = step.dims, case.weights, case.h, case.seq_lens
    sigma_T = int(seq_lens.sum())
    row_bytes = mla.row_bytes(cfg.cdtype, cfg.dims.row) + (4 if cfg.cdtype in ("fp8_e4m3", "fp6_e2m3") else 0)

    def one(c, e):
        e[0].record()
        mla.absorb_q(d, h, W, step.ws_q, step.q_lat, step.q_pe, step.kv_new)
        mla.rope(d, seq_lens, step.q_pe, step.kv_new, c)
        e[1].record()
        mla.decode_attn(d, step.q_lat, step.q_pe, c, seq_lens, splits, step.ws_d)
        e[2].record()
        if step.fused:
            mla.combine_absorb_out(d, splits, step.ws_d, W["W_uv"], W["W_o"], step.ws_o, step.u, step.lse)
        else:
            mla.combine(d, splits, seq_lens, step.ws_d, step.o_lat, step.lse)
            mla.absorb_out(d, step.o_lat, W["W_uv"], W["W_o"], step.ws_o, step.u)
        e[3].record()

    warm, n = 20, 20
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(warm + n)]
    for i, e in enumerate(evs):
        one(caches[i % len(caches)], e)
    torch.cuda.synchronize()
    t = [float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs[warm:]])) * 1e-3 for k in range(3)]
    t_step = float(np.mean([e[0].elapsed_time(e[3]) for e in evs[warm:]])) * 1e-3
    cache_bytes = sigma_T * row_bytes
    out = {"workload": f"config {cfg.key}: {cfg.title}", "sum_context_tokens": sigma_T,
           "step_us": t_step * 1e6, "tokens_per_s": case.B / t_step,
           "absorb_q_rope_us": t[0] * 1e6, "decode_attn_us": t[1] * 1e6, "combine_absorb_out_us": t[2] * 1e6,
           "output_call": "mla_combine_absorb_out" if step.fused else "mla_combine + mla_absorb_out",
           "achieved_gbps": cache_bytes / t[1] / 1e9, "frac": cache_bytes / t[1] / 1e9 / HBM_PEAK_GBPS,
           "traffic": DECODE_TRAFFIC_BYTES.get(key), "bytes_per_launch": cache_bytes,
           "per_unit": f"{row_bytes} B per cached token x {sigma_T} tokens"}
    del caches, case, step
    torch.cuda.empty_cache()
    return out


def prefill_bench(args):
    """Chunked prefill of C tokens per sequence (B=16, 2048 stored rows each by default, bf16 V2
    shape, paged). Absorbed form: mla_prefill_tables + the five decode calls over B*C causal
    pseudo-sequences, the dominant call (decode_attn) priced against the dense bf16 MFMA peak.
    Naive form (--naive): tables, absorb_q_naive + rope, prefill_naive_attn (gather, K/V expansion,
    attention), output_proj; the attention call priced likewise. Throughput in chunk tokens/s."""
    import numpy as np
    import torch

    import mla_latent_kv_25_amd as mla
    from synth import get_config, make_prefill_case

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mla.lib()
    C, B, P0 = args.prefill, 16, args.prefix
    cfg = get_config("3")
    case = make_prefill_case(cfg, [P0] * B, C, device="cuda")
    dims = case.dims
    cache = build_cache(mla, case)
    pf = mla.PrefillStep(dims, B, C, int(case.block_table.shape[1]), args.splits, naive=args.naive,
                         max_ctx=P0 + C if args.naive else None)
    W = case.weights

    def one_naive(ev=None):
        if ev is not None:
            ev[0].record()
        mla.prefill_tables(cache, B, C, case.p0, pf.seq_lens, pf.block_table)
        view = mla.LatentCache(cache.rows, cache.dtype, cache.t_cap, cache.scales, pf.block_table, cache.page_size)
        st, d = pf.step, pf.dims
        mla.absorb_q_naive(d, case.h_chunk.view(B * C, -1), W, st.ws_q, pf.q_c, st.q_pe, st.kv_new)
        mla.rope(d, pf.seq_lens, st.q_pe, st.kv_new, view)
        if ev is not None:
            ev[1].record()
        mla.prefill_naive_attn(d, B, C, pf.q_c, st.q_pe, cache, case.p0, pf.max_ctx, W["W_uk"], W["W_uv"], pf.ws_n,
                               pf.o)
        if ev is not None:
            ev[2].record()
        mla.output_proj(d, pf.o, W["W_o"], pf.ws_p, st.u)
        if ev is not None:
            ev[3].record()

    def one(ev=None):
        if ev is not None:
            ev[0].record()
        mla.prefill_tables(cache, B, C, case.p0, pf.seq_lens, pf.block_table)
        view = mla.LatentCache(cache.rows, cache.dtype, cache.t_cap, cache.scales, pf.block_table, cache.page_size)
        st, d = pf.step, pf.dims
        mla.absorb_q(d, case.h_chunk.view(B * C, -1), W, st.ws_q, st.q_lat, st.q_pe, st.kv_new)
        mla.rope(d, pf.seq_lens, st.q_pe, st.kv_new, view)
        if ev is not None:
            ev[1].record()
        mla.decode_attn(d, st.q_lat, st.q_pe, view, pf.seq_lens, args.splits, st.ws_d)
        if ev is not None:
            ev[2].record()
        if st.fused and W["W_uv"].dtype == torch.bfloat16:
            mla.combine_absorb_out(d, args.splits, st.ws_d, W["W_uv"], W["W_o"], st.ws_o, st.u, st.lse)
        else:
            mla.combine(d, args.splits, pf.seq_lens, st.ws_d, st.o_lat, st.lse)
            mla.absorb_out(d, st.o_lat, W["W_uv"], W["W_o"], st.ws_o, st.u)
        if ev is not None:
            ev[3].record()

    if args.naive:
        one = one_naive  # noqa: F811
    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        one()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        one(evs[i])
    torch.cuda.synchronize()
    st = [float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs])) * 1e-3 for k in range(3)]
    pairs = B * (C * P0 + C * (C + 1) // 2)                     # (query, key) pairs of the chunk
    if args.naive:
        rows = B * (P0 + C)                                      # context rows expanded to K^C and V
        flops = pairs * 2 * dims.n_h * (dims.d_h + dims.d_r + dims.d_h) + rows * 4 * dims.n_h * dims.d_h * dims.d_c
        per_unit = (f"81,920 flop per (query, key) pair x {pairs} pairs + 33,554,432 flop per expanded row x "
                    f"{rows} rows")
        kern = "prefill_naive_attn"
        names = ("tables+absorb_q_naive+rope", "prefill_naive_attn", "output_proj")
    else:
        flops = pairs * 2 * dims.n_h * (dims.row + dims.d_c)     # 278,528 flop per pair at V2
        per_unit = f"278,528 flop per (query, key) pair x {pairs} pairs"
        kern = "decode_attn"
        names = ("tables+absorb_q+rope", "decode_attn", "combine+absorb_out")
    achieved = flops / st[1] / 1e12
    out = {
        "metric": "MLA chunked-prefill tokens/s (chunk tokens), 1 MI355X",
        "value": B * C / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random-init weights of the DeepSeek-V2 attention shape)",
        "config": {"workload": f"chunked prefill ({'naive' if args.naive else 'absorbed'} form): B={B} sequences "
                               f"x {P0} stored rows, chunk C={C}, bf16 paged cache (64-row pages), DeepSeek-V2 "
                               f"shape", "batch": B, "chunk": C, "prefix": P0, "pseudo_sequences": B * C,
                   "form": "naive" if args.naive else "absorbed"},
        "kernels_us": {names[0]: st[0] * 1e6, names[1]: st[1] * 1e6, names[2]: st[2] * 1e6, "step": ms * 1e3},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None, "kernel": kern,
                     "flops_per_launch": flops, "per_unit": per_unit},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; across GPUs the path would shard "
                                   "decode over sequences and token ranges (one log-sum-exp all-gather per "
                                   "sequence before the combine), which is not built"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.prefill:
        prefill_bench(args)
        return
    import numpy as np
    import torch

    import mla_latent_kv_25_amd as mla
    from synth import get_config, make_case

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mla.lib()  # fails loudly when libmla.so is missing
    cfg = get_config(args.config)
    dims = cfg.dims
    case = make_case(cfg, device="cuda")
    B = case.B
    caches = [build_cache(mla, case) for _ in range(max(1, args.rotate))]
    # the fused combine + W^UV call where it has kernels (DeepSeek-V2 head shape, bf16 weights)
    fused = (not args.unfused and not args.precombined and dims.d_h == 128 and dims.d_c == 512 and dims.d_r == 64
             and case.weights["W_uv"].dtype == torch.bfloat16 and mla.fused_output_suits(B, args.splits))
    if args.precombined:
        step = mla.PrecombinedStep(dims, B, args.splits, case.weights)
    else:
        step = mla.DecodeStep(dims, B, args.splits, fused=fused)
    torch.cuda.synchronize()
    W, h, seq_lens = case.weights, case.h, case.seq_lens
    d = step.dims
    sigma_T = int(seq_lens.sum())
    row_bytes = mla.row_bytes(cfg.cdtype, dims.row) + (4 if cfg.cdtype in ("fp8_e4m3", "fp6_e2m3") else 0)
    cache_bytes = sigma_T * row_bytes
    flops_attn = sigma_T * 2 * dims.n_h * (dims.row + dims.d_c)
    wsz = {k: v.numel() * v.element_size() for k, v in case.weights.items()}
    wq_bytes = sum(wsz[k] for k in ("W_dq", "W_uq", "W_qr", "W_dkv", "W_kr", "W_uk"))
    wo_bytes = wsz["W_uv"] + wsz["W_o"]
    if args.precombined:
        wq_bytes += step.Wq_pre.numel() * step.Wq_pre.element_size() - wsz["W_uq"] - wsz["W_uk"]
        wo_bytes = step.Wo_pre.numel() * step.Wo_pre.element_size()

    def one_step(cache, ev=None):
        if ev is not None:
            ev[0].record()
        if args.precombined:
            mla.absorb_q_pre(d, h, W, step.Wq_pre, step.ws_q, step.q_lat, step.q_pe, step.kv_new)
        else:
            mla.absorb_q(d, h, W, step.ws_q, step.q_lat, step.q_pe, step.kv_new)
        if ev is not None:
            ev[1].record()
        mla.rope(d, seq_lens, step.q_pe, step.kv_new, cache)
        if ev is not None:
            ev[2].record()
        mla.decode_attn(d, step.q_lat, step.q_pe, cache, seq_lens, args.splits, step.ws_d)
        if ev is not None:
            ev[3].record()
        if fused:
            mla.combine_absorb_out(d, args.splits, step.ws_d, W["W_uv"], W["W_o"], step.ws_o, step.u, step.lse)
            if ev is not None:
                ev[4].record()
                ev[5].record()
            return
        mla.combine(d, args.splits, seq_lens, step.ws_d, step.o_lat, step.lse)
        if ev is not None:
            ev[4].record()
        if args.precombined:
            mla.absorb_out_pre(d, step.o_lat, step.Wo_pre, step.ws_op, step.u)
        else:
            mla.absorb_out(d, step.o_lat, W["W_uv"], W["W_o"], step.ws_o, step.u)
        if ev is not None:
            ev[5].record()

    graphs = None
    if args.graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in caches:
                one_step(c)
        torch.cuda.current_stream().wait_stream(s)
        for c in caches:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_step(c)
            graphs.append(g)

    for i in range(args.warmup):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            one_step(caches[i % len(caches)])
    torch.cuda.synchronize()

    # timed region: K whole steps
    t_start = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            one_step(caches[i % len(caches)])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = e0.elapsed_time(e1) / args.steps

    # decode_attn / combine launch durations, measured with events on the launch stream over the
    # same number of eager steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        one_step(caches[i % len(caches)], evs[i])
    torch.cuda.synchronize()
    stage = [float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs])) * 1e-3 for k in range(5)]
    t_dec, t_comb = stage[2], stage[3]
    # the latent-cache rate counts decode_attn + mla_combine; when the step merges the pieces inside
    # mla_combine_absorb_out, mla_combine is timed as its own call on the same pieces
    t_merge = t_comb
    if fused:
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            mla.decode_attn(d, step.q_lat, step.q_pe, caches[i % len(caches)], seq_lens, args.splits, step.ws_d)
            cev[i][0].record()
            mla.combine(d, args.splits, seq_lens, step.ws_d, step.o_lat, step.lse)
            cev[i][1].record()
        torch.cuda.synchronize()
        t_merge = float(np.mean([e[0].elapsed_time(e[1]) for e in cev])) * 1e-3

    tok_s = B / (ms_step * 1e-3)
    achieved = cache_bytes / t_dec / 1e9
    out = {
        "metric": "MLA decode latent-cache GB/s (% HBM peak) + decode tokens/s, 1 MI355X",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.cdtype == "bf16" else cfg.cdtype,
        "data": "synthetic (seeded; random-init weights of the "
                + ("DeepSeek-V2 attention shape)" if dims.n_h == 128 else "running-model shape)"),
        "config": {"workload": f"config {cfg.key}: {cfg.title}", "batch": B, "seq_len": int(seq_lens.max()),
                   "sum_context_tokens": sigma_T, "cache_dtype": cfg.cdtype, "layout": cfg.layout,
                   "n_h": dims.n_h, "d_c": dims.d_c, "d_r": dims.d_r, "d": dims.d,
                   "decode_splits": args.splits or ("one per CU" if dims.n_h == 128 else "two per CU"), "cache_copies_cycled": len(caches),
                   "hip_graph": bool(graphs),
                   "absorption": "pre-combined" if args.precombined else "two-step",
                   "combine": "fused with W^UV (mla_combine_absorb_out)" if fused else "separate call"},
        # latent-cache bytes over decode_attn + mla_combine (the combine timed as its own call when the
        # step uses the fused output call); decode_attn alone in decode_attn_gbps
        "latent_cache_gbps": cache_bytes / (t_dec + t_merge) / 1e9,
        "latent_cache_pct_hbm_peak": 100.0 * cache_bytes / (t_dec + t_merge) / 1e9 / HBM_PEAK_GBPS,
        "decode_attn_gbps": cache_bytes / t_dec / 1e9,
        "combine_us": t_merge * 1e6,
        "kernels_us": ({"absorb_q": stage[0] * 1e6, "rope_append": stage[1] * 1e6, "decode_attn": t_dec * 1e6,
                        "combine_absorb_out": t_comb * 1e6, "step": ms_step * 1e3} if fused else
                       {"absorb_q": stage[0] * 1e6, "rope_append": stage[1] * 1e6, "decode_attn": t_dec * 1e6,
                        "combine": t_comb * 1e6, "absorb_out": stage[4] * 1e6, "step": ms_step * 1e3}),
        "weights_gbps": {"absorb_q": wq_bytes / stage[0] / 1e9,
                         "absorb_out": wo_bytes / (t_comb if fused else stage[4]) / 1e9},
        "weight_bytes": {"absorb_q": wq_bytes, "absorb_out": wo_bytes},
        "attn_mfma_tflops": flops_attn / t_dec / 1e12,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": DECODE_TRAFFIC_BYTES.get(cfg.key),
                     "kernel": "decode_attn", "bytes_per_launch": cache_bytes,
                     "per_unit": f"{row_bytes} B per cached token x {sigma_T} tokens"},
        "wall_s": wall,
    }
    ceiling = stream_read_ceiling(mla)
    out["stream_read_ceiling_gbps"] = ceiling
    out["latent_cache_pct_stream_ceiling"] = 100.0 * out["latent_cache_gbps"] / ceiling
    out["decode_attn_pct_stream_ceiling"] = 100.0 * out["decode_attn_gbps"] / ceiling
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    if cfg.key == "2" and not args.no_other_workloads and not args.precombined:
        del caches
        torch.cuda.empty_cache()
        out["other_workloads"] = {k: decode_subrecord(mla, k, args.splits) for k in ("3", "4", "4f8", "4f6")}
        for rec in out["other_workloads"].values():
            rec["pct_stream_ceiling"] = 100.0 * rec["achieved_gbps"] / ceiling
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
