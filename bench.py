"""Benchmark of the hyper-connection residual mix on one MI355X.

One step = the hyper-connection work of one DeepSeek-V4.1 block at prefill size
(B=1, T=4096, 4 streams of d=5120, bf16 streams, fp32 mix parameters), with random
bf16 stand-ins for the attention and FFN outputs:
  1. hc_fused_step  attention boundary: coefficients from x, collapse with pi
  2. hc_fused_step  FFN boundary: x1 = expand(attention output), coefficients from
                    x1, collapse with attention's pre
  3. hc_post        x2 = expand(FFN output)
Inputs are resident in HBM before timing; three independent input sets are cycled
so that no step re-reads the previous step's data from the 256 MB last-level cache.

Prints one JSON line (see the keys below). --gpus N > 1 is refused: this build runs
on one GPU.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

KERNEL_SOURCES = ("hyper_connection_residual_mixes_amd/csrc/hc_kernels.hip",
                  "hyper_connection_residual_mixes_amd/csrc/hc_internal.h")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "ffn_boundary_counters_prefill_T4096.md")
ENTRY_KERNELS = {   # at the benchmark's 4096 tokens the sweeps run in 128-token groups
    "attn_fused": "bf16_sweep2_kernel<no expand, collapse> + finalize_kernel",
    "ffn_fused": "bf16_sweep2_kernel<expand, collapse> + finalize_kernel",
    "ffn_post": "post_kernel",
}

METRIC = "tokens/s and achieved HBM TB/s (% of peak), fused HC mix, d=5120, 4 streams"
PEAK_HBM_GBS = 8000.0


def algorithmic_bytes(n: int, d: int, es: int = 2, hc: int = 4):
    """Bytes each entry point must move (read + write), counted once each.
    Coefficients are fp32: pre/post 4*hc B, comb 4*hc^2 B per token (16, 16, 64 at
    hc = 4); hc_fn M*hc*d*4 B plus base (4M B) and scale (12 B) once per call,
    M = (2+hc)hc mix numbers."""
    M = (2 + hc) * hc
    coef = 4 * M                                                 # pre + post + comb
    w = M * hc * d * 4 + 4 * M + 12
    k1 = n * (hc * d * es + 4 * hc + d * es + coef) + w          # x, pi -> y, pre/post/comb
    k2 = n * (hc * d * es + d * es + coef + hc * d * es + d * es + coef) + w   # + f, post/comb/pi -> x1, y
    k3 = n * (d * es + hc * d * es + 4 * (hc + hc * hc) + hc * d * es)         # f, x1, post/comb -> x2
    return dict(attn_fused=k1, ffn_fused=k2, ffn_post=k3, block=k1 + k2 + k3)


def kernel_source_digest() -> str:
    """sha256 over the HIP sources; a stored counter record is valid only for the
    kernels it was taken on."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(entry: str):
    """HBM bytes per launch of ``entry`` from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a plain copy
    of known size), or None when the kernels changed since the counters were taken."""
    try:
        text = open(TRAFFIC_RECORD).read()
    except OSError:
        return None
    m = re.search(r"^traffic-record: (\{.*\})$", text, flags=re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("bytes_per_launch", {}).get(entry)


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _ceilings_lib():
    import ctypes
    path = os.path.join(ROOT, "bench_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing (run __graft_entry__.build())")
    L = ctypes.CDLL(path)
    L.bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                             ctypes.c_void_p]
    L.bench_copy.restype = ctypes.c_int
    L.bench_stream_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.bench_stream_mix.restype = ctypes.c_int
    L.bench_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.bench_empty.restype = ctypes.c_int
    L.bench_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.bench_mfma_bf16.restype = ctypes.c_int
    return L


def _median_seconds(run, stream, reps):
    import statistics
    import torch
    for _ in range(3):
        run()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    return statistics.median(times)


def copy_ceiling(dev, nbytes: int = 1 << 30, reps: int = 10):
    """The plain-copy reference (bench_ceilings.hip, a copy of 16-byte elements) on
    `nbytes` in + `nbytes` out, with cached and with non-temporal stores, one element
    per lane and grid-stride at three grid sizes; HIP events on the launch stream,
    median of `reps` after 3 warm-up copies. Returns (best GB/s, all figures)."""
    import torch
    L = _ceilings_lib()
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    stream = torch.cuda.current_stream(dev)
    figures = {}
    for nt in (0, 1):
        for wgs in (0, 1024, 2048, 4096):
            def run():
                rc = L.bench_copy(src.data_ptr(), dst.data_ptr(), nbytes, nt, wgs, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"bench_copy failed ({rc})")
            figures[f"{'nontemporal' if nt else 'cached'}_{wgs or 'one_shot'}wg"] = 2 * nbytes / _median_seconds(run, stream,
                                                                                                   reps) / 1e9
    del src, dst
    return max(figures.values()), figures


STREAM_MIXES = (("read_4", 4, 0), ("attention_flow_4r_1w", 4, 1), ("ffn_flow_5r_5w", 5, 5),
                ("expand_flow_5r_4w", 5, 4))


def stream_mix_ceilings(dev, rows: int = 4096, row_bytes: int = 5120 * 2, reps: int = 10):
    """Plain streaming with the block's read/write mixes (bench_ceilings.hip: rows of
    4096 tokens, each holding its planes of one 5120-channel bf16 stream back to back,
    as the streams are laid out), cached and non-temporal stores, one element per
    lane and grid-stride at 512 and 1024 workgroups. Three sets rotate so that no call finds its inputs in the 256 MB
    last-level cache. Returns (best GB/s per mix, all figures)."""
    import torch
    L = _ceilings_lib()
    stream = torch.cuda.current_stream(dev)
    set_bytes = rows * 5 * row_bytes
    src = torch.empty(3 * set_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(3 * set_bytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    best, figures = {}, {}
    for name, nr, nw in STREAM_MIXES:
        for nt in (0, 1):
            if nw == 0 and nt:
                continue
            key = f"{name}{'_nontemporal' if nt else ''}"
            for wgs in (0, 512, 1024):
                k = [0]

                def run():
                    s = k[0] % 3
                    k[0] += 1
                    rc = L.bench_stream_mix(src.data_ptr() + s * set_bytes, dst.data_ptr() + s * set_bytes, rows,
                                            row_bytes, nr, nw, nt, wgs, stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"bench_stream_mix failed ({rc})")
                gbs = (nr + nw) * rows * row_bytes / _median_seconds(run, stream, reps) / 1e9
                figures[f"{key}_{wgs or 'one_shot'}wg"] = gbs
                best[key] = max(best.get(key, 0.0), gbs)
    del src, dst
    return best, figures


def mfma_ceiling(dev, iters: int = 2000, reps: int = 5):
    """Sustained rate of v_mfma_f32_16x16x32_bf16 (bench_ceilings.hip: eight
    independent accumulators per wave, no memory traffic), in TFLOP/s, at 1024,
    2048 and 4096 workgroups of 4 waves; median of `reps`. Returns (best, all figures)."""
    import torch
    L = _ceilings_lib()
    stream = torch.cuda.current_stream(dev)
    figures = {}
    for wgs in (1024, 2048, 4096):
        out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)

        def run():
            rc = L.bench_mfma_bf16(out.data_ptr(), out.numel() * 4, wgs, iters, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"bench_mfma_bf16 failed ({rc})")
        flops = wgs * 4 * iters * 8 * 16384
        figures[f"{wgs}wg"] = flops / _median_seconds(run, stream, reps) / 1e12
        del out
    return max(figures.values()), figures


def cpu_baseline(sets_cpu):
    """The C oracle (fp64, one thread) on the whole block for each input set."""
    import oracle

    n_tok, dt = 0, 0.0
    for x, prev, attn, ffn, fa, ff in sets_cpu:
        pi, _, _ = oracle.hc_split_sinkhorn(*prev)   # collapse weights of the previous call
        t0 = time.perf_counter()
        oracle.block(x, pi, attn, ffn, fa, ff)
        dt += time.perf_counter() - t0
        n_tok += x.shape[0]
    d = sets_cpu[0][0].shape[-1]
    return dict(value=n_tok / dt, unit="tokens/s", cores=1, kind="oracle", cpu_model=cpu_model(),
                sample=f"the full block (attention + FFN boundary) on {len(sets_cpu)} input sets of "
                       f"{sets_cpu[0][0].shape[0]} tokens, d={d}: {n_tok} tokens, "
                       f"single-threaded C oracle in fp64, {dt:.1f} s")


def cpu_baseline_threads(sets_cpu, max_threads: int = 16):
    """The same oracle run on the same input sets, with the tokens cut into one
    contiguous chunk per host core (threads; the oracle's C calls release the GIL).
    Every token of the block is independent, so the chunks need no exchange."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    cores = max(1, min(max_threads, len(os.sched_getaffinity(0))))
    n_tok, dt = 0, 0.0
    with ThreadPoolExecutor(max_workers=cores) as pool:
        for x, prev, attn, ffn, fa, ff in sets_cpu:
            pi, _, _ = oracle.hc_split_sinkhorn(*prev)
            n = x.shape[0]
            cuts = [n * i // cores for i in range(cores + 1)]
            t0 = time.perf_counter()
            list(pool.map(lambda i: oracle.block(x[cuts[i]:cuts[i + 1]], pi[cuts[i]:cuts[i + 1]], attn, ffn,
                                                 fa[cuts[i]:cuts[i + 1]], ff[cuts[i]:cuts[i + 1]]), range(cores)))
            dt += time.perf_counter() - t0
            n_tok += n
    return dict(value=n_tok / dt, unit="tokens/s", cores=cores, kind="oracle", cpu_model=cpu_model(),
                sample=f"the same {n_tok} tokens as cpu_baseline, one contiguous token chunk per thread "
                       f"({cores} threads), {dt:.1f} s")


def decode_latency(dev, reps: int = 300):
    """One decode block (64 tokens x 4 streams x 5120 bf16; attention boundary, FFN
    boundary, FFN expand) called eagerly and replayed from a HIP graph of the same
    three entry points, which takes the host-side launch path out. Every graph
    replay is checked against the eager outputs. Returns the figures per block."""
    import torch
    import hc_inputs
    import hyper_connection_residual_mixes_amd as hc
    w = hc_inputs.DECODE
    n, d = w.n, w.d
    sets = []
    for s in range(3):
        inp = hc_inputs.decode(seed=s, device=dev)
        pi, _, _ = hc.hc_split_sinkhorn(*inp["prev"])
        out = dict(yA=torch.empty(n, d, dtype=w.dtype, device=dev), yF=torch.empty(n, d, dtype=w.dtype, device=dev),
                   x1=torch.empty(n, 4, d, dtype=w.dtype, device=dev),
                   x2=torch.empty(n, 4, d, dtype=w.dtype, device=dev),
                   cA=tuple(torch.empty(sh, device=dev) for sh in ((n, 4), (n, 4), (n, 4, 4))),
                   cF=tuple(torch.empty(sh, device=dev) for sh in ((n, 4), (n, 4), (n, 4, 4))))
        sets.append((inp, pi, out))
    ws = torch.empty(hc.workspace_size(n, 4, d), dtype=torch.uint8, device=dev)

    def step(i):
        inp, pi, o = sets[i % 3]
        a = hc.hc_fused_step(inp["x"], *inp["attn"], pre_mix=pi, y=o["yA"], out=o["cA"], workspace=ws)
        f = hc.hc_fused_step(inp["x"], *inp["ffn"], pre_mix=a["pre"], f_prev=inp["f_attn"], post_prev=a["post"],
                             comb_prev=a["comb"], streams_out=o["x1"], y=o["yF"], out=o["cF"], workspace=ws)
        hc.hc_post(inp["f_ffn"], f["streams"], f["post"], f["comb"], out=o["x2"])

    def outputs():
        return [t for _, _, o in sets for t in (o["yA"], o["yF"], o["x1"], o["x2"], *o["cA"], *o["cF"])]

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for i in range(30):
            step(i)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(reps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_wall = (time.perf_counter() - t0) / reps
    eager_gpu = e0.elapsed_time(e1) * 1e-3 / reps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(3):
            step(i)
    for _ in range(3):                       # replays, with eager work between them
        for t in outputs():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(ref, outputs())):
            raise RuntimeError("decode block: a graph replay differs from the eager result")
        step(0)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps // 3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_wall = (time.perf_counter() - t0) / (reps // 3 * 3)
    # The launch floor of the same chain: five dependent empty kernels with the block's
    # launch shapes (sweep, finalize, sweep, finalize, expand), replayed from a graph.
    L = _ceilings_lib()
    shapes = ((80, 512), (16, 256), (80, 512), (16, 256), (160, 256))
    ge = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ge):
        for _ in range(3):
            for wgs, threads in shapes:
                if L.bench_empty(wgs, threads, torch.cuda.current_stream(dev).cuda_stream) != 0:
                    raise RuntimeError("bench_empty failed")
    for _ in range(20):
        ge.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps // 3):
        ge.replay()
    torch.cuda.synchronize()
    floor = (time.perf_counter() - t0) / (reps // 3 * 3)
    block_bytes = algorithmic_bytes(n, d)["block"]
    return {"workload": f"decode block, {n} tokens x 4 streams x {d} bf16 (attention + FFN boundaries)",
            "us_per_block_eager": eager_wall * 1e6, "us_per_block_eager_gpu": eager_gpu * 1e6,
            "us_per_block_graph": graph_wall * 1e6, "tokens_per_s_graph": n / graph_wall,
            "launch_floor_us_per_block_graph": floor * 1e6,
            "algorithmic_bytes": block_bytes, "achieved_gb_s_graph": block_bytes / graph_wall / 1e9}


def generic_hc_blocks(dev, steps: int = 20, warmup: int = 100):
    """The prefill block (4096 tokens x hc streams x 5120 bf16) at stream counts
    other than four, which run one kernel per step; timed with HIP events around
    `steps` blocks after `warmup` blocks, the steady state (after 20 warm-up blocks
    the hc = 8 block still measured 470-473 us, after 100 462-466 us)."""
    import torch
    import hc_inputs
    import hyper_connection_residual_mixes_amd as hc
    out = {}
    for hc_ in (2, 8):
        w = hc_inputs.Workload(f"prefill_hc{hc_}", 1, 4096, 5120, torch.bfloat16, hc=hc_)
        inp = hc_inputs.block_inputs(w, seed=0, device=dev, outlier_frac=0.01)
        n, d = w.n, w.d
        pi, _, _ = hc.hc_split_sinkhorn(*inp["prev"], hc_mult=hc_)
        ws = torch.empty(hc.workspace_size(n, hc_, d), dtype=torch.uint8, device=dev)
        x1 = torch.empty_like(inp["x"])
        x2 = torch.empty_like(inp["x"])

        def step():
            hc.block(inp["x"], pi, inp["attn"], inp["ffn"], inp["f_attn"], inp["f_ffn"], x1_out=x1, x2_out=x2,
                     workspace=ws)

        for _ in range(warmup):
            step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / steps
        ab = algorithmic_bytes(n, d, hc=hc_)["block"]
        out[f"hc{hc_}"] = {"workload": f"prefill block, {n} tokens x {hc_} streams x {d} bf16",
                           "us_per_block": sec * 1e6, "tokens_per_s": n / sec, "algorithmic_bytes": ab,
                           "effective_gb_s": ab / sec / 1e9, "frac": ab / sec / 1e9 / PEAK_HBM_GBS}
        del inp, x1, x2, ws
    return out


def long_prefill_steady(dev, steps: int = 8):
    """The long-prefill workload's steady state (2 x 32768 tokens, 4 streams x 5120 bf16):
    the per-sublayer boundary with expand, coefficients and collapse
    (hc_fused_step), chained step after step on double-buffered streams, with two
    parameter sets and two sublayer outputs alternating. A step's working set
    (~7 GB) is far beyond the caches, so this is the HBM-bound rate."""
    import torch
    import hc_inputs
    import hyper_connection_residual_mixes_amd as hc
    w = hc_inputs.LONG_PREFILL
    n, d = w.n, w.d
    g = hc_inputs.generator(7, dev)
    params = [hc_inputs.mix_params(g, 4, d, "uniform", dev) for _ in range(2)]
    cur = hc_inputs.streams(g, n, 4, d, w.dtype, device=dev)
    nxt = torch.empty_like(cur)
    fs = [hc_inputs.sublayer_output(g, n, d, w.dtype, dev) for _ in range(2)]
    y = torch.empty(n, d, dtype=w.dtype, device=dev)
    ws = torch.empty(hc.workspace_size(n, 4, d), dtype=torch.uint8, device=dev)
    pi = torch.full((n, 4), 0.25, device=dev)
    first = hc.hc_fused_step(cur, *params[0], pre_mix=pi, y=y, workspace=ws)
    coef = (first["pre"], first["post"], first["comb"])
    outs = [tuple(torch.empty(sh, device=dev) for sh in ((n, 4), (n, 4), (n, 4, 4))) for _ in range(2)]

    def step(i):
        nonlocal cur, nxt, coef
        r = hc.hc_fused_step(cur, *params[i % 2], pre_mix=coef[0], f_prev=fs[i % 2], post_prev=coef[1],
                             comb_prev=coef[2], streams_out=nxt, y=y, out=outs[i % 2], workspace=ws)
        coef = (r["pre"], r["post"], r["comb"])
        cur, nxt = nxt, cur

    for i in range(2):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / steps
    ab = algorithmic_bytes(n, d)["ffn_fused"]
    res = {"workload": f"long-prefill steady state: hc_fused_step with expand + collapse, {n} tokens x 4 x {d} bf16",
           "us_per_sublayer": sec * 1e6, "tokens_per_s_per_sublayer": n / sec,
           "us_all_80_sublayers": 80 * sec * 1e6, "algorithmic_bytes": ab,
           "effective_gb_s": ab / sec / 1e9, "frac": ab / sec / 1e9 / PEAK_HBM_GBS}
    del cur, nxt, fs, y, ws, params, outs
    return res


def split_stress(dev, steps: int = 20):
    """The split stage alone (hc_split_sinkhorn) on the stress set: 1,048,576 rows of 24
    logits (~N(0, 3), 5% with one comb logit +40), 20 rounds. 96 B in and 96 B out
    per row."""
    import torch
    import hc_inputs
    import hyper_connection_residual_mixes_amd as hc
    st = hc_inputs.stress(seed=0, device=dev)
    m, s, b = st["mixes"], st["scale"], st["base"]
    n = m.shape[0]
    out = (torch.empty(n, 4, device=dev), torch.empty(n, 4, device=dev), torch.empty(n, 4, 4, device=dev))
    for _ in range(3):
        hc.hc_split_sinkhorn(m, s, b, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        hc.hc_split_sinkhorn(m, s, b, out=out)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / steps
    ab = n * (96 + 96) + 96 + 12
    return {"workload": f"split + Sinkhorn only, {n} rows x 24 logits, 20 rounds",
            "us": sec * 1e6, "rows_per_s": n / sec, "algorithmic_bytes": ab,
            "achieved_gb_s": ab / sec / 1e9, "frac": ab / sec / 1e9 / PEAK_HBM_GBS}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The block time settles only after ~130 back-to-back steps (~27 ms of load: 216 us per
    # step over the first 40 after a short warm-up, 201.5 us from then on), so the default
    # warm-up runs 200 steps.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--sets", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the per-token work shards across GPUs without communication)", file=sys.stderr)
        sys.exit(2)

    import torch

    import hc_inputs
    import hyper_connection_residual_mixes_amd as hc

    dev = torch.device("cuda:0")
    w = hc_inputs.PREFILL
    n, d = w.n, w.d
    print(f"bench: preparing {args.sets} input sets of {w.name}", file=sys.stderr, flush=True)
    sets = []
    for s in range(args.sets):
        inp = hc_inputs.prefill(seed=s, device=dev)
        pi, _, _ = hc.hc_split_sinkhorn(*inp["prev"])
        out = dict(yA=torch.empty(n, d, dtype=w.dtype, device=dev),
                   yF=torch.empty(n, d, dtype=w.dtype, device=dev),
                   x1=torch.empty(n, 4, d, dtype=w.dtype, device=dev),
                   x2=torch.empty(n, 4, d, dtype=w.dtype, device=dev),
                   cA=tuple(torch.empty(sh, device=dev) for sh in ((n, 4), (n, 4), (n, 4, 4))),
                   cF=tuple(torch.empty(sh, device=dev) for sh in ((n, 4), (n, 4), (n, 4, 4))))
        sets.append((inp, pi, out))
    ws = torch.empty(hc.workspace_size(n, 4, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        inp, pi, o = sets[i % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        a = hc.hc_fused_step(inp["x"], *inp["attn"], pre_mix=pi, y=o["yA"], out=o["cA"], workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        f = hc.hc_fused_step(inp["x"], *inp["ffn"], pre_mix=a["pre"], f_prev=inp["f_attn"],
                             post_prev=a["post"], comb_prev=a["comb"], streams_out=o["x1"],
                             y=o["yF"], out=o["cF"], workspace=ws)
        if ev is not None:
            ev[2].record(stream)
        hc.hc_post(inp["f_ffn"], f["streams"], f["post"], f["comb"], out=o["x2"])
        if ev is not None:
            ev[3].record(stream)

    # The plain-copy ceiling first (the reference the block's rates are read
    # against); its ~40 ms of copies also take the GPU out of its idle clocks
    # before the block's own warm-up.
    copy_gbs, copy_figures, mix_best, mix_figures, mfma_tf, mfma_figures = None, None, None, None, None, None
    if not args.no_copy_ceiling:
        print("bench: plain-copy and MFMA ceilings", file=sys.stderr, flush=True)
        copy_gbs, copy_figures = copy_ceiling(dev)
        mix_best, mix_figures = stream_mix_ceilings(dev)
        mfma_tf, mfma_figures = mfma_ceiling(dev)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # K timed steps bracketed by device synchronisation: the throughput. A timed event
    # serialises the stream where it is recorded, so these steps record none.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same K steps again with HIP events on the launch stream around each entry
    # point: the per-entry-point durations for the roofline
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    per = {k: 1e-3 * sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
           for j, k in enumerate(("attn_fused", "ffn_fused", "ffn_post"))}

    ab = algorithmic_bytes(n, d)
    ms = 1e3 * wall / args.steps
    tok_s = n * args.steps / wall
    eff_gbs = ab["block"] / (wall / args.steps) / 1e9
    dom = "ffn_fused"
    ach = ab[dom] / per[dom] / 1e9

    # next row: RMSNorm + MXFP8 cast of the attention boundary's collapsed input
    # (cast only, the GEMM-ready operand), timed with HIP events on its own
    gain = torch.rand(d, generator=torch.Generator(device=dev).manual_seed(5), device=dev) + 0.5
    qbuf = torch.empty(n, d, dtype=torch.uint8, device=dev)
    sbuf = torch.empty(n, d // 32, dtype=torch.uint8, device=dev)
    for i in range(3):
        hc.rmsnorm_mxfp8(sets[i % len(sets)][2]["yA"], gain, want_norm=False, q=qbuf, scale=sbuf)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        hc.rmsnorm_mxfp8(sets[i % len(sets)][2]["yA"], gain, want_norm=False, q=qbuf, scale=sbuf)
    e1.record(stream)
    torch.cuda.synchronize()
    norm_us = e0.elapsed_time(e1) * 1e3 / args.steps
    norm_bytes = n * (2 * d + d + d // 32) + 4 * d     # y in, codes + scales out, gain once
    next_rows = {"rmsnorm_mxfp8": {
        "workload": f"RMSNorm (gain) + MXFP8 cast of the collapsed input, {n} x {d} bf16 -> E4M3 + UE8M0",
        "kernel": "rmsnorm_mxfp8_kernel", "us": norm_us, "algorithmic_bytes": norm_bytes,
        "achieved_gb_s": norm_bytes / norm_us / 1e3, "frac": norm_bytes / norm_us / 1e3 / PEAK_HBM_GBS,
        "traffic": stored_traffic("rmsnorm_mxfp8")}}

    result = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "prefill block, B=1 T=4096, 4 streams x d=5120, bf16 streams, "
                               "attention + FFN boundaries", "batch": 1, "seq_len": 4096,
                   "d": d, "hc": 4, "stream_dtype": "bf16", "input_sets": args.sets},
        "hbm_effective_gb_s": eff_gbs, "hbm_effective_pct_of_peak": 100 * eff_gbs / PEAK_HBM_GBS,
        "copy_ceiling_gb_s": copy_gbs, "copy_figures_gb_s": copy_figures,
        "stream_mix_ceilings_gb_s": mix_best, "stream_mix_figures_gb_s": mix_figures,
        "mfma_bf16_16x16x32_ceiling_tflop_s": mfma_tf, "mfma_figures_tflop_s": mfma_figures,
        "entry_point_us": {k: v * 1e6 for k, v in per.items()},
        "algorithmic_bytes": ab,
        "roofline": {"kernel": f"hc_fused_step, FFN boundary ({ENTRY_KERNELS[dom]})",
                     "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS, "traffic": stored_traffic(dom)},
        "entry_point_roofline": {k: {"kernels": ENTRY_KERNELS[k], "achieved_gb_s": ab[k] / per[k] / 1e9,
                                     "frac": ab[k] / per[k] / 1e9 / PEAK_HBM_GBS,
                                     "traffic": stored_traffic(k)} for k in per},
    }
    next_rows["decode"] = decode_latency(dev)
    next_rows["generic_hc"] = generic_hc_blocks(dev)
    next_rows["long_prefill"] = long_prefill_steady(dev)
    next_rows["split_stress"] = split_stress(dev)
    result["next_rows"] = next_rows
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on every input set", file=sys.stderr, flush=True)
        cpu = lambda t: t.cpu() if isinstance(t, torch.Tensor) else tuple(u.cpu() for u in t)
        sets_cpu = [(cpu(inp["x"]), cpu(inp["prev"]), cpu(inp["attn"]), cpu(inp["ffn"]), cpu(inp["f_attn"]),
                     cpu(inp["f_ffn"])) for inp, _, _ in sets]
        result["cpu_baseline"] = cpu_baseline(sets_cpu)
        result["cpu_baseline_threads"] = cpu_baseline_threads(sets_cpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
