"""Benchmark: sparse MLA fp8 decode on one MI355X.

Workload (the headline decode batch): 64 decode tokens, one per request, contexts
U{4096..8192}, h_q = 64, top-k = 2048 distinct positions per token, fp8_ds_mla
paged cache (656-byte rows, block size 64, shuffled block table), bf16 q. One
step = the whole hot path over the batch (index conversion, gather + dequant,
QK^T, softmax, PV, split merge), inputs already resident in HBM: one
smla_decode_fp8 call (the attention kernel, then the merge kernel). A second
pass issues the same call in its two stages (the attention kernel with the
merge deferred, then the merge only: together bit-identical to the call), with
a HIP event between them, to time each kernel; the roofline object is the
attention kernel's.

Cold-cache timing: before every timed step a 1 GiB buffer is read (outside the
timed events) so neither L2 nor the 256 MB MALL holds the 95 MB working set; a
read leaves no dirty lines behind for the timed call to write back. Each step is
bracketed by HIP events on the stream the library launches on. Warm-cache
throughput (back-to-back calls) is reported beside it.

The same run also times every other workload of the target, one call per step
over the whole batch, cold, HIP events around the call (the `configs` key): the
tiny batch (bf16 and fp8 caches), the bf16 prefill batch (4 x 4096 tokens, h_q
128), the speculative-decode batch at h_q 16 with top-k 512, 1024 and 2048, and
the long mixed batch (32 decode + 2 x 2048 prefill tokens, h_q 128, contexts to
131072), each with its own binding roofline.

Prints ONE JSON line. `python bench.py --gpus N --steps K --warmup W`;
`--only NAME` times one workload alone (for profiler runs).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-MLA fp8 decode query-tokens/s & TFLOP/s (h_q=64, topk=2048), % roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6        # MI355X dense bf16 MFMA, published
CSRC = os.path.join(ROOT, "sparse_mla_attention_indices_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_fp8_decode_c2.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_work(w):
    """Bytes the path must move at minimum and the flops it must do.

    Bytes: unique cache rows read (every valid (request, position) once), q, o,
    lse, the logical indices, the block-table rows of the requests used, and
    req_id. Split partials, converted indices and line over-fetch are costs of an
    implementation, not of the method. Flops: 2 * h_q * (576 + 512) per valid slot.
    """
    idx = w.topk_indices
    valid = idx >= 0
    n_valid = int(valid.sum())
    pairs = np.unique((w.req_id_per_token[:, None].astype(np.int64) << 32 | idx.astype(np.int64))[valid])
    row_bytes = {"fp8": 656, "nvfp4": 352, "bf16": 1152}[w.cache_format]
    T, H, K = w.num_tokens, w.h_q, w.topk
    reqs = np.unique(w.req_id_per_token)
    by = {
        "cache_rows": int(pairs.size) * row_bytes,
        "q": T * H * 576 * 2,
        "out": T * H * 512 * 2,
        "lse": T * H * 4,
        "indices": T * K * 4,
        "block_table_rows": int(reqs.size) * w.max_blocks_per_req * 4,
        "req_id": T * 4,
    }
    flops = 2 * H * (576 + 512) * n_valid
    return sum(by.values()), flops, by, n_valid


def cache_writer_bench(torch, smla, dev, stream, flush, sink, steps: int):
    """The cache writer (smla_concat_and_cache_mla, fp8_ds_mla) on a prefill-sized
    batch of 16384 tokens into a 1.3 GB pool, with two slot patterns: random slots,
    and paged slots (256 blocks taken in shuffled order, each filled by 64
    consecutive tokens, as a prefill request's block table assigns them). Also the
    decode batch size (64 tokens, random slots). Cold cache. Algorithmic bytes
    per token: 1024 latent + 128 RoPE + 8 slot read, 656 written."""
    res = {}
    g = torch.Generator(device="cpu").manual_seed(21)
    NB = 32768
    cache = torch.zeros((NB, 64, 656), dtype=torch.uint8, device=dev)
    for T, name in ((16384, "tokens_16384"), (16384, "tokens_16384_paged"), (64, "tokens_64")):
        lat = (torch.randn(T, 512, generator=g) * 2).to(torch.bfloat16).to(dev)
        rope = torch.randn(T, 64, generator=g).to(torch.bfloat16).to(dev)
        if name.endswith("paged"):
            blocks = torch.randperm(NB, generator=g)[:T // 64].to(torch.int64)
            slots = (blocks[:, None] * 64 + torch.arange(64)).reshape(-1).to(dev)
        else:
            slots = torch.randperm(NB * 64, generator=g)[:T].to(torch.int64).to(dev)
        for _ in range(3):
            smla.smla_concat_and_cache_mla(lat, rope, cache, slots, stream=stream)
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            torch.amax(flush, 0, out=sink)
            e0[i].record(stream)
            smla.smla_concat_and_cache_mla(lat, rope, cache, slots, stream=stream)
            e1[i].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in zip(e0, e1)]))
        nbytes = T * (1024 + 128 + 8 + 656)
        res[name] = {"ms": ms, "tokens_per_s": T / (ms * 1e-3), "algorithmic_bytes": nbytes,
                              "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
                              "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del cache
    return res


def upconvert_bench(torch, smla, W, dev, stream, flush, sink, steps: int):
    """The separate-prefill mode's gather-and-upconvert (smla_gather_upconvert_fp8)
    over config 5's two prefill contexts (131072 and 65536 positions, 196608 rows,
    one launch), cold cache. Algorithmic bytes per row: 656 read + 1152 written;
    plus one 4-byte block-table entry per 64 rows."""
    lens = np.array([131072, 65536], dtype=np.int32)
    bt, nb = W.allocate_block_table(np.random.default_rng(70), lens)
    g = torch.Generator(device="cpu").manual_seed(70)
    # contents do not change the work: random bytes, scales forced finite and small
    cache = torch.randint(0, 256, (nb, 64, 656), dtype=torch.uint8, generator=g)
    cache[:, :, 512:528] = torch.tensor([0, 0, 128, 60] * 4, dtype=torch.uint8)     # 1/64 as float32
    cache = cache.to(dev)
    rows = int(lens.sum())
    ws = torch.empty((rows, 576), dtype=torch.bfloat16, device=dev)
    bt_d = torch.from_numpy(bt).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    starts_d = torch.tensor([0, int(lens[0])], dtype=torch.int32, device=dev)
    for _ in range(3):
        smla.smla_gather_upconvert_fp8(cache, bt_d, lens_d, starts_d, int(lens.max()), ws, stream=stream)
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        torch.amax(flush, 0, out=sink)
        e0[i].record(stream)
        smla.smla_gather_upconvert_fp8(cache, bt_d, lens_d, starts_d, int(lens.max()), ws, stream=stream)
        e1[i].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in zip(e0, e1)]))
    nbytes = rows * (656 + 1152) + (rows // 64) * 4
    del cache, ws
    return {"kernel": "upconvert_kernel", "rows": rows, "ms": ms, "algorithmic_bytes": nbytes,
            "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "workload": "config 5 prefill contexts: 131072 + 65536 positions, shuffled blocks"}


def nvfp4_prefill_bench(torch, smla, W, dev, stream, flush, sink, steps: int, seed: int):
    """Config 5's prefill part (2 x 2048 query tokens, h_q 128, top-k 2048,
    contexts 131072 and 65536) over an nvfp4_ds_mla cache, both ways the library
    offers, cold cache, HIP events around each call: native decode
    (smla_decode_nvfp4: one 16-head workgroup per head block, each gathering the
    token's rows) and the staged separate-prefill mode
    (smla_forward_nvfp4_separate_prefill: the workspace index conversion, the
    exact upconvert of both contexts into one bf16 workspace, then the 128-head
    bf16 kernel over it; its host plan is built once, outside the events)."""
    w = W.config5_prefill(seed, "nvfp4")
    q, cache, bt, req, idx = upload(torch, w, dev)
    T, H, K = w.num_tokens, w.h_q, w.topk
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(smla.smla_workspace_size(T, H, K), 1), dtype=torch.uint8, device=dev)
    counts = np.bincount(w.req_id_per_token, minlength=w.num_reqs)
    qsl = np.concatenate([[0], np.cumsum(counts)])
    rows = int(w.ctx_lens.sum())
    plan = smla.smla_build_separate_prefill_plan(qsl, w.ctx_lens, 0, rows, dev)
    bf16_ws = torch.empty((plan.workspace_rows, 576), dtype=torch.bfloat16, device=dev)
    slots = torch.empty_like(idx)

    def native():
        smla.smla_decode_nvfp4(q, cache, bt, req, idx, w.sm_scale, out=out, lse=lse, workspace=ws, stream=stream)

    def staged():
        smla.smla_forward_nvfp4_separate_prefill(q, cache, bt, req, idx, w.sm_scale, plan, out=out, lse=lse,
                                                 bf16_workspace=bf16_ws, slots=slots, stream=stream)

    res = {"workload": w.name + ": 2 x 2048 query tokens, h_q 128, top-k 2048, contexts 131072 + 65536",
           "num_tokens": T}
    for name, fn in (("native_decode", native), ("staged_prefill", staged)):
        for _ in range(2):
            torch.amax(flush, 0, out=sink)
            fn()
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            torch.amax(flush, 0, out=sink)
            e0[i].record(stream)
            fn()
            e1[i].record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in zip(e0, e1)]))
        r = {"ms_median": ms}
        r.update(roofline_of(w, ms))
        res[name] = r
    del q, cache, bt, req, idx, out, lse, ws, bf16_ws, slots
    torch.cuda.empty_cache()
    return res


def kernels_of_plan(cache_format: str, h_q: int, splits: int):
    """Names of the kernels one call launches, from the split plan (the same rule the
    library's launcher applies: one workgroup covers all h_q heads of a token, except
    fp8 with h_q = 128, which takes two 64-head workgroups, and nvfp4, which takes
    one 16-head workgroup per 16 heads)."""
    fmt = cache_format
    if fmt == "nvfp4":
        names = ["attn_kernel<nvfp4, 1>"]
    elif h_q == 128 and fmt == "bf16":
        names = ["attn128_kernel"]
    elif fmt == "fp8" and h_q >= 64:
        names = ["attn_pc_kernel"]
    else:
        names = [f"attn_kernel<{fmt}, {h_q // 16}>"]
    if splits > 1:
        names.append(f"merge_kernel<{splits}>")
    return names


def upload(torch, w, dev):
    """A workload's arrays as device tensors (q, cache, block table, request ids, indices)."""
    q = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if w.cache_format == "bf16":
        cache = torch.from_numpy(w.cache.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        cache = torch.from_numpy(w.cache).to(dev)
    return (q, cache, torch.from_numpy(w.block_table).to(dev), torch.from_numpy(w.req_id_per_token).to(dev),
            torch.from_numpy(w.topk_indices).to(dev))


def roofline_of(w, ms: float):
    """Throughput and the binding roofline (lower of bf16 MFMA peak and HBM peak x
    arithmetic intensity) of one call over workload w taking ms milliseconds."""
    bytes_alg, flops, by, n_valid = algorithmic_work(w)
    ai = flops / bytes_alg
    roof_tflops = min(BF16_PEAK_TFLOPS, HBM_PEAK_GBS * 1e9 * ai / 1e12)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"query_tokens_per_s": w.num_tokens / (ms * 1e-3), "tflops": tflops,
            "binding_roofline": {"bound": "hbm" if roof_tflops < BF16_PEAK_TFLOPS else "mfma",
                                 "arith_intensity_flop_per_byte": ai, "tflops": roof_tflops},
            "pct_of_binding_roofline": 100.0 * tflops / roof_tflops,
            "algorithmic_GBps": bytes_alg / (ms * 1e-3) / 1e9,
            "algorithmic_bytes": bytes_alg, "flops": flops, "valid_slots": n_valid}


def config_bench(torch, smla, w, dev, stream, flush, sink, steps: int, warmup: int = 2):
    """One workload through its entry point (smla_prefill_bf16 for a bf16 cache,
    smla_decode_fp8 for fp8_ds_mla, smla_decode_nvfp4 for nvfp4_ds_mla), one call
    per step over the whole batch, cold
    cache (the 1 GiB read before each step, outside the events), HIP events on the
    library's stream around each call."""
    q, cache, bt, req, idx = upload(torch, w, dev)
    T, H, K = w.num_tokens, w.h_q, w.topk
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(smla.smla_workspace_size(T, H, K), 1), dtype=torch.uint8, device=dev)
    entry = {"bf16": "smla_prefill_bf16", "fp8": "smla_decode_fp8", "nvfp4": "smla_decode_nvfp4"}[w.cache_format]
    fn = getattr(smla, entry)
    props = torch.cuda.get_device_properties(dev)
    splits, _ = smla.smla_plan(T, H, K, props.multi_processor_count)

    def call():
        fn(q, cache, bt, req, idx, w.sm_scale, out=out, lse=lse, workspace=ws, stream=stream)

    for _ in range(warmup):
        torch.amax(flush, 0, out=sink)
        call()
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        torch.amax(flush, 0, out=sink)
        e0[i].record(stream)
        call()
        e1[i].record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in zip(e0, e1)])
    ms = float(np.median(t))
    rec = {"workload": w.name, "num_tokens": T, "h_q": H, "topk": K,
           "cache": {"bf16": "bf16", "fp8": "fp8_ds_mla", "nvfp4": "nvfp4_ds_mla"}[w.cache_format],
           "entry_point": entry,
           "kernels": kernels_of_plan(w.cache_format, H, splits), "num_splits": splits,
           "steps": steps, "ms_median": ms, "ms_p10": float(np.percentile(t, 10)),
           "ms_p90": float(np.percentile(t, 90))}
    rec.update(roofline_of(w, ms))
    del q, cache, bt, req, idx, out, lse, ws
    torch.cuda.empty_cache()
    return rec


# The other workloads of the target, each timed in the default run beside the
# headline batch: name -> (generator, timed steps).
def other_configs(W, seed: int):
    def c4():
        return W.config4_sweep(seed)

    def c4_nvfp4():
        return W.config4_sweep(seed, "nvfp4")
    return [("c1_tiny_bf16", lambda: [W.config1(seed)], 20),
            ("c1_tiny_fp8", lambda: [W.config1_fp8(seed)], 20),
            ("c3_bf16_prefill", lambda: [W.config3(seed)], 5),
            ("c4_spec_decode", c4, 20),
            ("c4_spec_decode_nvfp4", c4_nvfp4, 20),
            ("c5_long_mixed", lambda: [W.config5(seed)], 5)]


def cpu_identity():
    """Host CPU model and core counts, as the host reports them."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "os_cpu_count": os.cpu_count()}


def cpu_baseline(w, target_s: float = 10.0):
    """The oracle as it stands, on this host's cores: whole passes over the batch's
    tokens (in a fixed shuffled order) until about target_s of CPU work is done."""
    import oracle
    threads = oracle.num_threads()
    order = np.random.default_rng(0).permutation(w.num_tokens)
    n = max(1, min(w.num_tokens, threads))
    done, t_total, passes = 0, 0.0, 0
    while t_total < target_s and passes < 100:
        for s in range(0, w.num_tokens, n):
            tok = order[s:s + n]
            t0 = time.perf_counter()
            oracle.attention(oracle.FP8_CACHE, w.q, w.cache, w.block_table, w.req_id_per_token,
                             w.topk_indices, w.sm_scale, tokens=tok)
            t_total += time.perf_counter() - t0
            done += len(tok)
            if t_total >= target_s:
                break
        passes += 1
    rec = {"value": done / t_total, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} token evaluations ({passes} pass(es) over the batch's {w.num_tokens} "
                     f"tokens, all {w.h_q} heads, top-k {w.topk}), float64 C + OpenMP, "
                     f"{t_total:.1f} s"}
    rec.update(cpu_identity())
    return rec


def traffic_from_profile():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    ap.add_argument("--only", default=None,
                    help="time one workload alone and print its record (for profiler runs): "
                         "c2 (the headline batch, no side measurements), c1_tiny_bf16, c1_tiny_fp8, "
                         "c3_bf16_prefill, c4_spec_decode (top-k 512, 1024, 2048), c4_spec_decode_nvfp4 "
                         "(the same over an nvfp4_ds_mla cache), c5_long_mixed")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (the headline line only)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_mla_attention_indices_amd import smla
    from sparse_mla_attention_indices_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calib:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": src.numel(), "launches": 5}), flush=True)
        return

    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)     # 1 GiB, read to evict caches
    sink = torch.empty((), dtype=torch.int32, device=dev)
    if args.only is not None and args.only != "c2":
        gens = {name: (gen, steps) for name, gen, steps in other_configs(W, args.seed)}
        if args.only not in gens:
            print(f"unknown workload {args.only!r}; choose c2 or one of {sorted(gens)}", file=sys.stderr)
            sys.exit(2)
        gen, steps = gens[args.only]
        for w in gen():
            print(f"[bench] {w.name}", file=sys.stderr, flush=True)
            print(json.dumps(config_bench(torch, smla, w, dev, stream, flush, sink, min(steps, args.steps),
                                          args.warmup)), flush=True)
        return

    w = W.config2(args.seed)
    q, cache, bt, req, idx = upload(torch, w, dev)
    out = torch.empty((w.num_tokens, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.num_tokens, w.h_q), dtype=torch.float32, device=dev)
    ws_bytes = smla.smla_workspace_size(w.num_tokens, w.h_q, w.topk)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    props = torch.cuda.get_device_properties(dev)
    splits, _ = smla.smla_plan(w.num_tokens, w.h_q, w.topk, props.multi_processor_count)

    def step():
        smla.smla_decode_fp8(q, cache, bt, req, idx, w.sm_scale, out=out, lse=lse, workspace=ws,
                             stream=stream)

    def attention():
        smla.smla_decode_fp8(q, cache, bt, req, idx, w.sm_scale, out=out, lse=lse, workspace=ws,
                             stream=stream, stage="attention")

    def merge():
        smla.smla_decode_fp8(q, cache, bt, req, idx, w.sm_scale, out=out, lse=lse, workspace=ws,
                             stream=stream, stage="merge")

    for i in range(args.warmup):
        torch.amax(flush, 0, out=sink)
        step()
    torch.cuda.synchronize()

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    starts, ends = events(args.steps), events(args.steps)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        torch.amax(flush, 0, out=sink)
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    cold_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    # per-kernel times: the call in its two stages, with an event between
    a0, a1, m1 = events(args.steps), events(args.steps), events(args.steps)
    for i in range(args.steps):
        torch.amax(flush, 0, out=sink)
        a0[i].record(stream)
        attention()
        a1[i].record(stream)
        merge()
        m1[i].record(stream)
    torch.cuda.synchronize()
    attn_ms = np.array([s.elapsed_time(e) for s, e in zip(a0, a1)])
    merge_ms = np.array([s.elapsed_time(e) for s, e in zip(a1, m1)])

    # warm cache: back-to-back calls, working set resident in MALL
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        step()
    w0.record(stream)
    for _ in range(args.steps):
        step()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps

    bytes_alg, flops, by, n_valid = algorithmic_work(w)
    ms = float(cold_ms.mean())
    tok_s = w.num_tokens / (ms * 1e-3)
    tflops = flops / (ms * 1e-3) / 1e12
    ai = flops / bytes_alg
    roof_tflops = min(BF16_PEAK_TFLOPS, HBM_PEAK_GBS * 1e9 * ai / 1e12)
    roof_tok_s = w.num_tokens * roof_tflops * 1e12 / flops
    # the dominant kernel: attention reads every input byte of the method; the
    # merge kernel writes the output (and re-reads the split partials)
    attn_bytes = bytes_alg - by["out"] - by["lse"]
    attn_avg_ms = float(attn_ms.mean())
    achieved_gbs = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    traffic = traffic_from_profile()

    rec = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8/bf16",
        "data": "synthetic",
        "config": {
            "workload": "fp8_ds_mla sparse MLA decode: 64 tokens (1 per request), ctx U{4096..8192}, "
                        "h_q 64, top-k 2048 distinct, block 64, shuffled block table, cold cache",
            "num_tokens": w.num_tokens, "h_q": w.h_q, "topk": w.topk, "cache": "fp8_ds_mla",
            "num_splits": splits, "seed": args.seed,
        },
        "tflops": tflops,
        "pct_of_binding_roofline": 100.0 * tok_s / roof_tok_s,
        "binding_roofline": {"bound": "hbm" if roof_tflops < BF16_PEAK_TFLOPS else "mfma",
                             "arith_intensity_flop_per_byte": ai, "tflops": roof_tflops,
                             "query_tokens_per_s": roof_tok_s},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "attn_pc_kernel", "algorithmic_bytes_per_launch": attn_bytes,
                     "avg_launch_ms": attn_avg_ms},
        "kernels_ms_cold": {"attn_pc_kernel": attn_avg_ms, "merge_kernel": float(merge_ms.mean())},
        "whole_step_hbm_frac": bytes_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": bytes_alg,
        "algorithmic_bytes_breakdown": by,
        "flops_per_step": flops,
        "valid_slots": n_valid,
        "ms_per_step_median": float(np.median(cold_ms)),
        "ms_per_step_p10": float(np.percentile(cold_ms, 10)),
        "ms_per_step_p90": float(np.percentile(cold_ms, 90)),
        "warm_cache": {"ms_per_step": warm_ms, "query_tokens_per_s": w.num_tokens / (warm_ms * 1e-3)},
        "timed_region_wall_s_incl_flushes": t_wall,
        "timing": ("HIP events on the library's stream around each step (attention kernel, then merge "
                   "kernel) and between the two kernels"),
        "kernel_source_hash": kernel_source_hash(),
        "device": props.name,
    }
    if args.only == "c2":
        print(json.dumps(rec), flush=True)
        return
    del q, cache, bt, req, idx, out, lse, ws
    torch.cuda.empty_cache()
    if not args.no_configs:
        rec["configs"] = {}
        for name, gen, steps in other_configs(W, args.seed):
            for wc in gen():
                print(f"[bench] {wc.name}", file=sys.stderr, flush=True)
                rec["configs"][wc.name] = config_bench(torch, smla, wc, dev, stream, flush, sink,
                                                       min(steps, args.steps))
        rec["configs"][w.name] = {"workload": w.name, "kernels": kernels_of_plan("fp8", w.h_q, splits),
                                  "num_splits": splits, "ms_median": rec["ms_per_step_median"],
                                  "note": "the headline batch: see the top-level fields"}
        rec["configs"][w.name].update(roofline_of(w, rec["ms_per_step_median"]))
    rec["cache_writer"] = cache_writer_bench(torch, smla, dev, stream, flush, sink, min(args.steps, 20))
    rec["separate_prefill_upconvert"] = upconvert_bench(torch, smla, W, dev, stream, flush, sink,
                                                        min(args.steps, 20))
    if not args.no_configs:
        rec["nvfp4_prefill"] = nvfp4_prefill_bench(torch, smla, W, dev, stream, flush, sink, min(args.steps, 5),
                                                   args.seed)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
