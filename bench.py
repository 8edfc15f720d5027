#!/usr/bin/env python3
"""Benchmark of one TPLA decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload dsv3_32k]

A step is the whole decode hot path over one batch, with every input already
resident in HBM: rotate the absorbed query and the new token's latent and
append the new row to the shard caches (tpla_rotate_append: one launch for
what tpla_hadamard_latent and tpla_append_kv do separately), decode the shard
(tpla_decode_shard: split-K attention and log-sum-exp merge) and combine the
shard outputs: every shard's merge writes its latent columns of the combined
output (the placement tpla_combine_shards performs for outputs held apart).
`--up-project D_V` adds each shard's value up-projection (tpla_up_project,
random bf16 weights) with the shards' terms summed; `--latent-norm` adds the
RMS norm of the new latent to the append.
The default workload is the DeepSeek-V3-shaped shard at 32K context
(B=16, H=128, d_c=512 split TP=2 -> d_s=256, d_r=64, paged blocks of 64 with
a permuted block table); `--workload ragged_tp2` runs both shards of the
ragged TP=2 step in turn.  `--workload mla_tp2_32k` is the comparison TPLA
is measured against: plain MLA under TP=2, one device's 64 of the 128 heads
over the whole 512-wide latent (no rotation: the step appends the new row
with tpla_append_kv and decodes); `--workload mla_tp4_32k` is the same for
Kimi-K2 under TP=4 (16 of its 64 heads per device).

Steps are replayed from HIP graphs (one holding several steps, cache replicas
in turn, plus one per replica for a remainder).  Replicas rotate
so that the caches read by consecutive steps together exceed the 256 MB
Infinity Cache (the next layer's cache would evict it in a real model).
The untimed warm-up replays the same graphs for at least W steps and at
least 0.1 s, since the GPU needs some 15-20 ms of sustained load after idle
to reach its steady clock (`warmup_steps_run` reports how many it ran).

Prints one JSON line.  `value` is the latent-cache bytes the step streams
(sum_b L_b * (d_s + d_r) * 2 per shard) divided by the step time, in GB/s.
`roofline` gives the decode kernel alone, timed with HIP events in a loop of
back-to-back launches on its own stream right after the timed steps;
`cpu_baseline` times the fp64 oracle on the host over a bounded sample.

`--mode prefill` (or `--workload mla_prefill_4k`) measures the MLA-form
prefill instead: tpla_mla_prefill over B=2 prompts of 4096 tokens with 64
heads, plus the hand-off of the prompt rows into two TPLA shard caches
(tpla_rotate_append); `value` is the attention's algorithmic TFLOP/s over
the whole step and `roofline` the attention kernel against the dense bf16
matrix-core peak.

`--mode copy` runs a plain 1 GiB device copy (for calibrating rocprofv3
FETCH_SIZE/WRITE_SIZE counters); `--mode decode` runs only decode launches.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TPLA decode: latent-cache GB/s (% HBM peak) and decode tokens/s at 32K ctx"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, vendor figure
MALL_BYTES = 256 * 2 ** 20      # Infinity Cache
WARM_SECONDS = 0.1              # minimum untimed warm-up of sustained work


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3_32k",
                    choices=["dsv3_32k", "kimi_k2_32k", "ragged_tp2", "dsv3_4k", "mla_tp2_32k",
                             "mla_tp4_32k", "mla_prefill_4k"])
    ap.add_argument("--mode", default="step", choices=["step", "decode", "copy", "prefill"])
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas (0 = auto)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--up-project", type=int, default=0, metavar="D_V",
                    help="add each shard's value up-projection to the step (random bf16 "
                         "weights, D_V output columns per head; the shards' terms are summed)")
    ap.add_argument("--latent-norm", default="none", choices=["none", "global", "slice"],
                    help="RMS norm of the rotated new latent inside rotate/append (slice = "
                         "each shard's columns on their own)")
    ap.add_argument("--decode-launches", type=int, default=40)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle's host timing (0 disables it)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_latent_decode_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("decode_") or name in ("tpla_api.hip", "merge_combine.hip",
                                                  "tpla_internal.h", "unit_map.h", "merge_item.h"):
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def stored_counters(workload: str):
    """Figures per decode launch from committed rocprofv3 counter runs
    (profiles/decode_<workload>_traffic.json), if they were taken on the
    current kernel sources: (record, None), else (None, reason)."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None, f"no counter record for {workload}"
    rec = json.load(open(path))
    if rec.get("kernel_sha") != kernel_source_hash():
        return None, (f"counters were taken on kernel sources {rec.get('kernel_sha')}, these are "
                      f"{kernel_source_hash()}")
    return rec, None


def copy_probe(torch, steps, n=1 << 30):
    """A plain device copy of n bytes (read n, write n), timed with events:
    the HBM rate a streaming kernel can reach on this GPU, in GB/s."""
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del src, dst
    return {"bytes_read_per_copy": n, "bytes_written_per_copy": n, "ms_per_copy": ms,
            "copy_GBps": 2 * n / ms / 1e6}


def run_copy(torch, steps):
    print(json.dumps({"mode": "copy", **copy_probe(torch, steps)}), flush=True)


def host_cpu():
    """(CPU model, cores this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def timed_reps(fn, reps=3):
    """One untimed warm-up run, then the median of `reps` timed runs (s)."""
    fn()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def cpu_baseline(case, seconds: float):
    """The fp64 oracle over whole sequences of the same workload, on the host:
    one warm-up and three timed runs over a sample of sequences (median), with
    the BLAS thread pool as it is and again limited to one thread."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    model, cores = host_cpu()
    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cfg = case.cfg
    d_s, tp = cfg.d_s, cfg.tp
    shards = list(range(tp)) if cfg.name == "ragged_tp2" else [0]
    rotate = tp > 1             # plain MLA (one shard) has no rotation
    bs = cfg.block_size
    f64 = oracle.bf16_bits_to_f64
    starts = np.concatenate([[0], np.cumsum(case.seq_lens - 1)])

    def caches_of(b):
        """Sequence b's paged cache per shard with its history rows (set-up)."""
        n = int(case.seq_lens[b]) - 1
        rows = slice(int(starts[b]), int(starts[b]) + n)
        out = []
        for g in shards:
            cache = np.zeros((case.num_blocks, bs, d_s + cfg.d_r), np.uint16)
            oracle.paged_append(cache, case.block_table, bs, case.hist_seq[rows],
                                case.hist_pos[rows], case.hist_latent[rows, g * d_s:(g + 1) * d_s],
                                case.hist_rope[rows])
            out.append(cache)
        return out

    def step_seq(b, caches):
        """The step for sequence b: rotate, append the new row, attention per
        shard, combine (the appended row is rewritten identically each run)."""
        q = f64(case.q_latent[b])
        new = f64(case.new_latent[b])[None]
        if rotate:
            q = oracle.fwht(q)
            new = oracle.fwht(new)
        new = oracle.f32_to_bf16_bits(new.astype(np.float32))
        outs = []
        for g, cache in zip(shards, caches):
            oracle.paged_append(cache, case.block_table, bs, np.array([b]), case.new_pos[b:b + 1],
                                new[:, g * d_s:(g + 1) * d_s], case.new_rope[b:b + 1])
            o, _ = oracle.tpla_decode_paged(
                oracle.shard_slice(q, g, tp)[None], f64(case.q_rope[b])[None], cache,
                case.block_table[b:b + 1], case.seq_lens[b:b + 1], bs, d_s, cfg.scale)
            outs.append(o)
        oracle.combine_shards(outs)

    def seq_bytes(seqs):
        return sum(int(case.seq_lens[b]) for b in seqs) * (d_s + cfg.d_r) * 2 * len(shards)

    # sample: as many sequences as fit a quarter of the budget per (warm-up +
    # 3 runs) of the pool as it is; the one-thread runs take a quarter more
    order = list(range(cfg.batch))
    caches = {0: caches_of(0)}
    t0 = time.perf_counter()
    step_seq(0, caches[0])
    per_seq = max(time.perf_counter() - t0, 1e-6)
    n_multi = int(max(1, min(cfg.batch, seconds / 4 / 4 / per_seq)))
    seqs = order[:n_multi]
    for b in seqs:
        if b not in caches:
            caches[b] = caches_of(b)
    med = timed_reps(lambda: [step_seq(b, caches[b]) for b in seqs])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        step_seq(0, caches[0])
        per_seq1 = max(time.perf_counter() - t0, 1e-6)
        n_one = int(max(1, min(n_multi, seconds / 4 / 4 / per_seq1)))
        seqs1 = order[:n_one]
        med1 = timed_reps(lambda: [step_seq(b, caches[b]) for b in seqs1])
    what = (f"whole step per sequence: {'rotate, ' if rotate else ''}append, paged gather + fp64 "
            f"attention per shard, combine")
    return {"value": seq_bytes(seqs) / med / 1e9, "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{len(seqs)} of {cfg.batch} sequences of the same workload ({what}); "
                      f"median of 3 runs after 1 warm-up, {med:.2f} s each; tokens/s "
                      f"{len(seqs) / med:.3g}",
            "cpu_model": model, "host_cores": cores, "blas_threads": int(blas_threads),
            "single_thread": {"value": seq_bytes(seqs1) / med1 / 1e9, "unit": "GB/s", "cores": 1,
                              "sample": f"{len(seqs1)} sequences, median of 3 runs after 1 "
                                        f"warm-up, {med1:.2f} s each"}}


PREFILL_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix cores, vendor figure


def prefill_flops(lens, heads: int, d_c: int, d_r: int) -> int:
    """Algorithmic FLOPs of causal MLA attention: position t of every head
    scores t+1 keys over d_c + d_r and sums t+1 values over d_c."""
    return sum(heads * (int(L) * (int(L) + 1) // 2) * 2 * (2 * d_c + d_r) for L in lens)


def cpu_prefill_baseline(pc, seconds: float):
    """The fp64 oracle on a bounded sample: prefixes of the first prompt,
    doubled in length until the time budget is spent."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:           # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    model, cores = host_cpu()
    f64 = oracle.bf16_bits_to_f64
    d_c = pc.cfg.d_c
    n, done, elapsed, dt = 64, 0, 0.0, 0.0
    # the next prefix costs about 4x the last one: stop before it would
    # overrun the budget by half
    while elapsed + 4 * dt < 1.5 * seconds and n <= int(pc.seq_lens[0]):
        kv = f64(pc.kv[0, :n])
        ql, qr = f64(pc.q_latent[0, :n]), f64(pc.q_rope[0, :n])
        t0 = time.perf_counter()
        oracle.mla_prefill(ql, qr, kv[:, :d_c], kv[:, d_c:], pc.cfg.scale)
        dt = time.perf_counter() - t0
        elapsed += dt
        done += prefill_flops([n], pc.cfg.heads, d_c, pc.cfg.d_r)
        last = n
        n *= 2
    return {"value": done / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"prefixes of 64..{last} tokens of the first prompt (all {pc.cfg.heads} heads), "
                      f"{elapsed:.1f} s on the host",
            "cpu_model": model, "host_cores": cores}


def run_prefill(args, torch):
    import numpy as np
    from tensor_latent_decode_amd import tpla
    from tensor_latent_decode_amd.inputs import PREFILL_CONFIGS, make_prefill_case

    t_setup = time.perf_counter()
    pc = make_prefill_case(PREFILL_CONFIGS["mla_prefill_4k"])
    cfg = pc.cfg
    B, S, H, d_c, d_r = cfg.batch, cfg.max_len, cfg.heads, cfg.d_c, cfg.d_r

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    q, qr, kv = dev(pc.q_latent), dev(pc.q_rope), dev(pc.kv)
    lens = torch.from_numpy(pc.seq_lens).cuda()
    out = torch.empty((B, S, H, d_c), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    # the hand-off: prompt rows rotated, sliced and appended to two shard caches
    tp, d_s, bs = 2, d_c // 2, 64
    nb = (S + bs - 1) // bs
    bt = torch.arange(B * nb, dtype=torch.int32, device="cuda").view(B, nb)
    caches = [torch.empty((B * nb, bs, d_s + d_r), dtype=torch.bfloat16, device="cuda")
              for _ in range(tp)]
    rows = kv.reshape(B * S, d_c + d_r)
    seq = torch.arange(B, dtype=torch.int32, device="cuda").repeat_interleave(S)
    pos = torch.arange(S, dtype=torch.int32, device="cuda").repeat(B)
    stream = torch.cuda.Stream()

    def attention():
        tpla.mla_prefill(q, qr, kv, lens, cfg.scale, out=out, lse=lse)

    def step():
        attention()
        tpla.rotate_append(None, None, rows[:, :d_c], rows[:, d_c:], seq, pos, caches, bt)

    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
        setup_s = time.perf_counter() - t_setup
        t_w = time.perf_counter()
        n_w = 0
        while n_w < max(args.warmup, 2) or time.perf_counter() - t_w < WARM_SECONDS:
            step()
            n_w += 1
            if n_w % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        steps = max(1, args.steps // 10)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / steps
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(steps):
            attention()
        a1.record(stream)
        torch.cuda.synchronize()
        ms_att = a0.elapsed_time(a1) / steps
    flops = prefill_flops(pc.seq_lens, H, d_c, d_r)
    result = {
        "metric": "MLA-form prefill: attention TFLOP/s (bf16 matrix cores) at 4K prompts",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_w,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "heads": H, "d_c": d_c, "d_r": d_r,
                   "prompt_len": S, "global_batch": B, "seq_len": S, "out_dtype": "bf16",
                   "handoff_shards": tp},
        "prompt_tokens_per_s": round(B * S / (ms_step * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(flops / (ms_att * 1e-3) / 1e12, 1),
                     "peak": PREFILL_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (ms_att * 1e-3) / 1e12 / PREFILL_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "tpla_mla_prefill",
                     "ms_per_launch": round(ms_att, 4), "algorithmic_flops_per_launch": flops},
        "setup_s": round(setup_s, 1),
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_prefill_baseline(pc, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): TPLA shards would sit on separate GPUs joined by an RCCL "
              "collective, which this benchmark does not run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from tensor_latent_decode_amd import tpla
    from tensor_latent_decode_amd.inputs import CONFIGS, make_case

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.mode == "copy":
        run_copy(torch, max(args.steps, 1))
        return
    if args.mode == "prefill" or args.workload == "mla_prefill_4k":
        run_prefill(args, torch)
        return

    t_setup = time.perf_counter()
    case = make_case(CONFIGS[args.workload])
    cfg = case.cfg
    B, H, d_c, d_s, d_r, tp = cfg.batch, cfg.heads, cfg.d_c, cfg.d_s, cfg.d_r, cfg.tp
    shards = list(range(tp)) if args.workload == "ragged_tp2" else [0]
    rotate = tp > 1             # plain MLA (one shard) has no rotation
    if not rotate and args.latent_norm != "none":
        print("--latent-norm applies to the rotated TPLA workloads only", file=sys.stderr)
        sys.exit(2)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bt, lens = dev(case.block_table), dev(case.seq_lens)
    q_raw, q_rope = dev(case.q_latent), dev(case.q_rope)
    new_raw, new_rope = dev(case.new_latent), dev(case.new_rope)
    new_seq = torch.arange(B, dtype=torch.int32, device="cuda")
    new_pos = dev(case.new_pos)
    cache_bytes = int(case.num_blocks) * cfg.block_size * (d_s + d_r) * 2
    step_cache_bytes = cache_bytes * len(shards)
    replicas = args.replicas or max(2, -(-3 * MALL_BYTES // step_cache_bytes))
    hist_lat, hist_rope = dev(case.hist_latent), dev(case.hist_rope)
    hist_seq, hist_pos = dev(case.hist_seq), dev(case.hist_pos)
    caches = []
    for _ in range(replicas):
        per = []
        for g in shards:
            c = torch.empty((case.num_blocks, cfg.block_size, d_s + d_r), dtype=torch.bfloat16,
                            device="cuda")
            tpla.append_kv(c, bt, hist_seq, hist_pos, hist_lat[:, g * d_s:(g + 1) * d_s], hist_rope)
            per.append(c)
        caches.append(per)
    del hist_lat, hist_rope, hist_seq, hist_pos
    maxlen = int(case.seq_lens.max())
    q_rot = torch.empty((B, H, d_c), dtype=torch.bfloat16, device="cuda") if rotate else q_raw
    # the combine: shard i's merge writes its latent columns of the combined
    # output directly (placement of disjoint slices; tpla_combine_shards does
    # the same for outputs held in separate buffers)
    combined = torch.empty((B, H, len(shards) * d_s), dtype=torch.float32, device="cuda")
    outs = [combined[:, :, i * d_s:(i + 1) * d_s] for i in range(len(shards))]
    lses = [torch.empty((B, H), dtype=torch.float32, device="cuda") for _ in shards]
    args0 = tpla.make_decode_args(q_rot[:, :, :d_s], q_rope, caches[0][0], bt, lens, cfg.scale,
                                  maxlen, outs[0], lses[0], args.num_splits)
    # split count from the host's copy of the lengths (a serving loop has them)
    splits = args.num_splits or tpla.decode_suggest_splits(args0, case.seq_lens)
    args0.num_splits = splits
    workspace = tpla.decode_workspace(args0)
    torch.cuda.synchronize()

    def decode(r, i, g):
        tpla.decode_shard(q_rot[:, :, g * d_s:(g + 1) * d_s], q_rope, caches[r][i], bt, lens,
                          cfg.scale, maxlen, out=outs[i], lse=lses[i], num_splits=splits,
                          workspace=workspace)

    # optional value up-projection: each shard's latent columns of every
    # head's W_UV (synthetic, seeded), the shards' terms summed into y
    w_up, y_up = [], None
    if args.up_project:
        gen = torch.Generator(device="cpu").manual_seed(7)
        for _ in shards:
            w_up.append((torch.randn((H, args.up_project, d_s), generator=gen) / 16)
                        .to(torch.bfloat16).cuda())
        y_up = torch.empty((B, H, args.up_project), dtype=torch.float32, device="cuda")

    def step(r):
        if rotate:
            tpla.rotate_append(q_raw, q_rot, new_raw, new_rope, new_seq, new_pos, caches[r], bt,
                               first_shard=shards[0], latent_norm=args.latent_norm)
        else:
            tpla.append_kv(caches[r][0], bt, new_seq, new_pos, new_raw, new_rope)
        for i, g in enumerate(shards):
            decode(r, i, g)
        for i in range(len(w_up)):
            tpla.up_project(outs[i], w_up[i], out=y_up, accumulate=i > 0)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for r in range(replicas):          # eager warm-up of every replica
            step(r)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graphs = []
    for r in range(replicas):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            step(r)
        graphs.append(gr)
    # one graph holding several steps, replicas in turn (a model's whole decode
    # step, all layers, would be one graph; a replay costs a fixed host and
    # queue overhead that a one-layer graph would otherwise carry alone)
    per_cycle = replicas * max(1, -(-8 // replicas))
    cycle = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cycle, stream=stream):
        for k in range(per_cycle):
            step(k % replicas)
    # graph of back-to-back decode launches (replicas rotating) for kernel timing
    dec_graph = torch.cuda.CUDAGraph()
    n_dec = max(args.decode_launches, replicas)
    with torch.cuda.graph(dec_graph, stream=stream):
        for k in range(n_dec):
            decode(k % replicas, 0, shards[0])
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    warm_steps = 0
    if args.mode == "step" or args.mode == "decode":
        # Untimed warm-up on the timed loop's own graphs: at least W steps and
        # at least WARM_SECONDS of back-to-back work.  From idle the GPU takes
        # some 15-20 ms of sustained load to reach its steady clock (the first
        # ~100 steps run 10-30% slower), which a steady decode loop never sees.
        for r in range(replicas):
            graphs[r].replay()
        warm_steps = replicas
        t_w = time.perf_counter()
        n_rep = 0
        while warm_steps < args.warmup or time.perf_counter() - t_w < WARM_SECONDS:
            cycle.replay()
            warm_steps += per_cycle
            n_rep += 1
            if n_rep % 4 == 0:      # keep the host clock tied to finished work
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    if args.mode == "decode":
        # profiling aid: decode launches only
        for _ in range(max(1, args.steps // n_dec)):
            dec_graph.replay()
        torch.cuda.synchronize()
        print(json.dumps({"mode": "decode", "launches": n_dec * max(1, args.steps // n_dec)}))
        return

    torch.cuda.synchronize()
    full, rest = divmod(args.steps, per_cycle)
    # one event between consecutive replays: per-window step times
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(full + 1)]
    ev0.record()
    marks[0].record()
    for k in range(full):
        cycle.replay()
        marks[k + 1].record()
    for k in range(rest):
        graphs[k % replicas].replay()
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    windows = sorted(marks[k].elapsed_time(marks[k + 1]) / per_cycle for k in range(full))

    def pct(q):
        return windows[min(len(windows) - 1, int(q * len(windows)))] if windows else ms_step

    # decode kernel alone: back-to-back launches on the same stream
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    dec_graph.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        d0.record(stream)
        reps = 3
        for _ in range(reps):
            dec_graph.replay()
        d1.record(stream)
    torch.cuda.synchronize()
    ms_dec = d0.elapsed_time(d1) / (reps * n_dec)

    del graphs, cycle, dec_graph
    probe = copy_probe(torch, 10)

    lens_sum = int(np.sum(case.seq_lens.astype(np.int64)))
    bytes_per_shard = lens_sum * (d_s + d_r) * 2
    step_bytes = bytes_per_shard * len(shards)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = bytes_per_shard / (ms_dec * 1e-3) / 1e9
    counters, why_not = stored_counters(args.workload)
    traffic = counters.get("hbm_bytes_per_launch") if counters else None
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_windows": {"windows": len(windows), "steps_per_window": per_cycle,
                                "median": round(pct(0.5), 5), "p10": round(pct(0.1), 5),
                                "p90": round(pct(0.9), 5)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "heads": H, "d_c": d_c, "tp": tp,
                   "shards_run": len(shards), "d_s": d_s, "d_r": d_r,
                   "context": (list(cfg.ctx) if isinstance(cfg.ctx, tuple) else cfg.ctx),
                   "tokens_attended": lens_sum, "block_size": cfg.block_size,
                   "cache_replicas": replicas, "global_batch": B, "num_splits": splits,
                   "latent_norm": args.latent_norm, "up_project_d_v": args.up_project,
                   "seq_len": maxlen},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "copy_probe_GBps": round(probe["copy_GBps"], 1),
        "pct_of_copy_probe": round(100.0 * value / probe["copy_GBps"], 2),
        "decode_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_source": (counters.get("source") if counters else why_not),
                     "mfma_busy_pct": counters.get("mfma_busy_pct") if counters else None,
                     "pct_of_copy_probe": round(100.0 * achieved / probe["copy_GBps"], 2),
                     "kernel": "tpla_decode_shard (split-K attention + LSE merge)",
                     "ms_per_launch": round(ms_dec, 5),
                     "algorithmic_bytes_per_launch": bytes_per_shard},
        "setup_s": round(setup_s, 1),
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
