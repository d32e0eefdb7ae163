"""Benchmark: MLA decode throughput on one MI355X, in KV-token·heads/s.

One step = one pass of the whole decode hot path (plan, attended-set and paged
gather, QK^T, mask, online softmax, PV, finalize, split-KV merge) over one
batch of synthetic, seeded inputs that are already resident in HBM.  The
default workload is the DSA/SFA sparse decode: B=32, Q=1, h_q=128, S=32768,
top_k=2048 (3 sequences keep 1500 entries), paged block_size 64, bf16.

Cache effects: each timed step reads a different one of `--rotate` index sets
(or cache copies for dense workloads), so the rows a step touches are not left
in the 256 MiB Infinity Cache by the previous step.

Prints one JSON line.  `--gpus N` with N > 1 exits: this build measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix, TFLOP/s
METRIC = "sparse/dense MLA decode KV-token·heads/s at 1 GPU; % of HBM/MFMA roofline"
KERNEL_SOURCES = [os.path.join(ROOT, "latent_decode_attention_amd", "csrc", f)
                  for f in ("mla_kernels.hip", "mla_api.cpp", "mla_internal.h", "mla_fastdiv.h")]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_work(w, indices_list=None):
    """Bytes and flops the method must move/compute for one step.

    bytes = latent rows attended (each once per sequence) x 1152 (int8 cache: 576 + a
            4-byte row factor) + q + O + lse
            + index lists + block-table entries of the blocks touched
            (+ the fp32 shard partials written and read, under DCP).
    flops = sum_{b,q} |A(b,q)| * h_q * 2 * (576 + 512).
    """
    B, Q, H = w.B, w.Q, w.h_q
    rows_bytes = 0
    bt_bytes = 0
    kv_heads = 0
    for b in range(B):
        S = int(w.seq_lens[b])
        if w.indices is None:
            need = set(range(S))                                  # every position, causal union
            per_q = [max(0, S - Q + qi + 1) for qi in range(Q)]
        else:
            lst = indices_list[b] if indices_list is not None else w.indices.reshape(-1)[
                b * w.index_stride_b: b * w.index_stride_b + w.top_k]
            lst = np.asarray(lst)
            need = set(int(i) for i in lst if 0 <= i <= S - 1)
            per_q = [int(np.count_nonzero((lst >= 0) & (lst <= S - Q + qi))) for qi in range(Q)]
        rows_bytes += len(need) * (1152 if w.kv8 is None else 576 + 4)
        bt_bytes += len({p // w.block_size for p in need}) * 4
        kv_heads += sum(per_q) * H
    q_bytes = B * Q * H * 576 * 2
    o_bytes = B * Q * H * 512 * 2
    lse_bytes = B * Q * H * 4
    idx_bytes = 0 if w.indices is None else B * (1 if w.index_stride_q == 0 else Q) * w.top_k * 4
    extra = 0
    if w.num_shards > 1:  # the formulation emits fp32 shard partials, written then read by the merge
        o_bytes = B * Q * H * 512 * 2
        extra = 2 * w.num_shards * B * Q * H * (512 + 1) * 4
    total = rows_bytes + q_bytes + o_bytes + lse_bytes + idx_bytes + bt_bytes + extra
    flops = kv_heads * 2 * (576 + 512)
    return dict(bytes=total, flops=flops, kv_token_heads=kv_heads, rows_bytes=rows_bytes)


def stored_traffic(workload_name: str):
    """HBM bytes per call (every kernel the call launches) from the committed
    rocprofv3 counter summary, if the kernel sources have not changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload_name)
    if not ent or ent.get("kernel_hash") != kernel_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Parity bars (the contract): lse within 1e-3; O within 1e-2, for bf16 outputs
# where |O_ref| < 4 (1 bf16 ulp of O_ref beyond, where rounding alone exceeds 1e-2).
def _o_bar(o_ref, bf16_out):
    if not bf16_out:
        return np.full_like(o_ref, 1e-2)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(o_ref), 1e-30))) - 7)
    return np.where(np.abs(o_ref) < 4.0, 1e-2, ulp)


def cpu_baseline(w, target_s: float, gpu_out=None, seed: int = 0):
    """Time the fp64 oracle on a bounded sample of output rows of the same workload.

    gpu_out = (O [rows, 512] float64, lse [rows], bf16_out) of the GPU path on
    the workload's own inputs: the rows the oracle computes on its first pass
    over the workload are compared with them (max |dO|, max |dlse|, max |O_ref|)."""
    import oracle
    g = np.random.default_rng(seed)
    rows_all = g.permutation(w.rows)
    n = 16
    spent = 0.0
    done_rows = 0
    done_work = 0
    err = dict(max_abs_dO=0.0, max_abs_dlse=0.0, max_abs_O_ref=0.0, rows_compared=0, within_bars=True)
    # Rows are taken in a seeded random order; a workload smaller than the time
    # budget is run again from the start, so the rate is measured over >= target_s.
    passes = 0
    while spent < target_s:
        start = done_rows % w.rows
        sel = rows_all[start:start + n]
        if start + len(sel) >= w.rows:
            passes += 1
        t0 = time.perf_counter()
        if w.indices is not None:
            ro, rl = oracle.sparse(w, rows=sel)
        else:
            ro, rl = oracle.dense(w, rows=sel)
        spent += time.perf_counter() - t0
        if gpu_out is not None and done_rows < w.rows:
            go, gl, bf16_out = gpu_out
            d_o = np.abs(go[sel] - ro)
            both_inf = np.isneginf(gl[sel]) & np.isneginf(rl)
            d_l = np.where(both_inf, 0.0, np.abs(gl[sel] - rl))
            err["max_abs_dO"] = max(err["max_abs_dO"], float(d_o.max()))
            err["max_abs_dlse"] = max(err["max_abs_dlse"], float(np.nanmax(d_l)))
            err["max_abs_O_ref"] = max(err["max_abs_O_ref"], float(np.abs(ro).max()))
            err["rows_compared"] += len(sel)
            err["within_bars"] &= bool(np.all(d_o <= _o_bar(ro, bf16_out)) and np.all(d_l <= 1e-3))
        for r in sel:
            b = int(r) // (w.Q * w.h_q)
            qi = (int(r) // w.h_q) % w.Q
            S = int(w.seq_lens[b])
            if w.indices is None:
                done_work += max(0, S - w.Q + qi + 1)
            else:
                lst = w.indices.reshape(-1)[b * w.index_stride_b + qi * w.index_stride_q:][:w.top_k]
                done_work += int(np.count_nonzero((lst >= 0) & (lst <= S - w.Q + qi)))
        done_rows += len(sel)
        n = min(n * 2, 4096)
    rec = dict(value=done_work / spent, unit="KV-token·heads/s", cores=oracle.num_threads(),
               kind="oracle", cpu_model=cpu_model(),
               sample=(f"{done_rows} output rows (b,q,head) of {w.name} ({w.rows} rows in all, "
                       f"{passes} full passes), fp64, {spent:.1f} s"))
    if gpu_out is not None:
        rec["parity"] = err
    return rec


def measure_copy_gbs(torch, dev, mib: int = 1024, reps: int = 10) -> float:
    """Device-to-device copy rate (bytes read + written per second) of a plain
    torch copy of `mib` MiB: the bandwidth a streaming kernel reaches on this machine."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / (ms * 1e-3) / 1e9


def run_kv_write(args, torch, md, W, dev):
    """Latent KV-cache write: T = 32768 prefill tokens per call (8 sequences of
    4096, each filling 64-slot blocks drawn at random) into a 262144-slot cache
    (302 MB), cycling through 8 input sets (302 MB of new rows) so the Infinity
    Cache cannot serve them.  Bytes = each stored row read and written once
    (2 x 1152 B) + the 4-byte slot of every token."""
    T, num_slots, sets = 32768, 262144, 8
    xs = [W.make_kv_write_inputs(T, num_slots, seed=2000 + r) for r in range(sets)]
    rows = [torch.from_numpy(x.rows.view(np.int16)).to(dev).view(torch.bfloat16) for x in xs]
    slots = [torch.from_numpy(x.slots).to(dev) for x in xs]
    kv = torch.zeros((num_slots, 576), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        r = i % sets
        md.mla_kv_write(rows[r], slots[r], kv, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    stored = float(np.mean([((x.slots >= 0) & (x.slots < num_slots)).sum() for x in xs]))
    nbytes = stored * 2 * 1152 + T * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": "latent KV-cache write (slot_mapping scatter) rows stored/s at 1 GPU; % of HBM roofline",
        "value": stored / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"kv_write_t{T}_slots{num_slots}", "T": T, "num_slots": num_slots,
                   "stored_rows_mean": stored, "rotating_input_sets": sets},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": stored_traffic(f"kv_write_t{T}_slots{num_slots}"),
                     "kernel": "kv_write_kernel",
                     "launch_ms": ms, "algorithmic_bytes": nbytes},
    }
    print(f"[bench] kv_write {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s algorithmic = {gbs / HBM_PEAK_GBS:.3f} "
          f"of HBM peak", file=sys.stderr, flush=True)
    rec["cpu_baseline"] = None
    if args.cpu_seconds > 0:
        from oracle import cache_ops
        kv_host = np.zeros((num_slots, 576), dtype=np.uint16)
        t0, done, n = time.perf_counter(), 0, 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            x = xs[n % sets]
            kv_host = cache_ops.kv_write(kv_host, x.rows, x.slots)
            done += int(((x.slots >= 0) & (x.slots < num_slots)).sum())
            n += 1
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": done / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} full calls ({done} rows stored) of the same workload, "
                                         f"numpy, {dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def run_topk(args, torch, md, W, dev):
    """Indexer top-k selection at the headline sparse shape: B = 32 rows of S =
    32768 fp32 scores (--topk-batch changes B), top 2048 each.  Each call reads
    a different one of the score sets (about 300 MB in all, each a rolled copy
    of one seeded set) so the Infinity Cache cannot serve them.  Bytes = every
    score once (4 B) + the selected positions (4 B each) + seq_lens."""
    B, S, k = args.topk_batch, 32768, 2048
    sets = max(2, (300 << 20) // (B * S * 4))
    x = W.make_topk_scores(B, 1, [S] * B, k, seed=1009)
    base = torch.from_numpy(x.scores).to(dev)
    scores = [torch.roll(base, shifts=977 * r, dims=2).contiguous() for r in range(sets)]
    seq = torch.from_numpy(x.seq_lens).to(dev)
    out = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        md.mla_topk_select(scores[i % sets], seq, k, out=out, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    ranked = B * S
    nbytes = ranked * 4 + B * k * 4 + B * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = f"topk_b{B}_s{S}_k{k}"
    rec = {
        "metric": "indexer top-k selection, scores ranked/s at 1 GPU; % of HBM roofline",
        "value": ranked / (ms * 1e-3), "unit": "scores/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "B": B, "Q": 1, "seq_len": S, "top_k": k, "rotating_input_sets": sets},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": stored_traffic(name), "kernel": "topk_kernel",
                     "launch_ms": ms, "algorithmic_bytes": nbytes},
    }
    print(f"[bench] topk {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s algorithmic = {gbs / HBM_PEAK_GBS:.3f} "
          f"of HBM peak", file=sys.stderr, flush=True)
    rec["cpu_baseline"] = None
    if args.cpu_seconds > 0:
        from oracle import topk
        t0, rows = time.perf_counter(), 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            b = rows % B
            topk.select_row(x.scores[b, 0], k)
            rows += 1
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": rows * S / dt, "unit": "scores/s", "cores": 1, "kind": "oracle",
                               "sample": f"{rows} rows of {S} scores of the same workload, numpy, {dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # 200 untimed calls: the shader clock ramps up over the first ~100 calls
    # after idle (the first 10-call chunks run ~10 % slower), so a short
    # warm-up times the ramp rather than the steady state.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=3, help="workload preset (1..7); 3 = sparse S=32k")
    ap.add_argument("--rotate", type=int, default=8, help="distinct input sets cycled through")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget (0 = skip)")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--topk-batch", type=int, default=32, help="rows of the top-k workload (--op topk)")
    ap.add_argument("--top-k", type=int, default=0,
                    help="list length for a sparse preset (0 = the preset's own; a per-tile cost is the "
                         "difference of two lengths)")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "int8"],
                    help="latent cache element type: bf16, or int8 codes with one fp32 factor per row")
    ap.add_argument("--group-rows", type=int, default=0, choices=[0, 64, 128],
                    help="work-group shape (query rows per work-group); 0 = the planner's choice")
    ap.add_argument("--op", default="decode", choices=["decode", "kv_write", "topk"],
                    help="decode: the attention call (default); kv_write: the latent-cache write "
                         "through slot_mapping (32768 prefill tokens into a 262144-slot cache); "
                         "topk: the indexer's top-2048 selection over 32768 scores per row")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB 5 times (the known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the split-KV path runs "
              "its shards on one device and no multi-GPU run is part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from latent_decode_attention_amd import mla_decode as md
    from latent_decode_attention_amd import workloads as W
    from latent_decode_attention_amd.device import bf16_tensor, upload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
        return
    if args.op == "kv_write":
        run_kv_write(args, torch, md, W, dev)
        return
    if args.op == "topk":
        run_topk(args, torch, md, W, dev)
        return
    md.GROUP_ROWS = args.group_rows
    t0 = time.time()
    if args.top_k:
        w = W.PRESETS[args.config]()
        if w.indices is None or w.index_stride_q != 0:
            raise SystemExit("--top-k applies to the sparse presets with one list per sequence")
        w = W.make_workload(f"{w.name}_k{args.top_k}", w.B, w.Q, w.h_q, w.seq_lens, w.block_size,
                            int(w.meta["seed"]), top_k=args.top_k)
    else:
        w = W.PRESETS[args.config]()
    if args.kv == "int8":
        w = W.int8_cache(w)
    d = upload(w, dev)
    print(f"[bench] workload {w.name} ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    stream = torch.cuda.current_stream()

    # Rotating inputs so consecutive steps touch different rows.
    if w.indices is not None:
        idx_host = [w.indices] + [W.rotate_indices(w, 1000 + r) for r in range(args.rotate - 1)]
        idx_dev = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev) for x in idx_host]
        kv_dev = [d.kv]
    else:
        idx_host, idx_dev = None, None
        copies = max(1, min(args.rotate, int((2 << 30) // max(1, d.kv.numel() * d.kv.element_size()))))
        kv_dev = [d.kv] + [d.kv.clone() for _ in range(copies - 1)]

    p0 = md.make_problem(d.q, d.kv, d.block_table, d.seq_lens, w.scale, w.max_seq_len, d.kv_scale)
    plan = md.mla_plan_query(p0, num_shards=w.num_shards, interleave=w.interleave,
                             top_k=w.top_k, index_stride_q=w.index_stride_q,
                             num_cus=torch.cuda.get_device_properties(dev).multi_processor_count)
    splits = plan["splits"]
    ws_bytes = md.mla_workspace_size(p0, w.num_shards, w.interleave, -1, w.top_k, w.index_stride_q)
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    sharded = w.num_shards > 1
    if sharded:
        out = torch.empty((w.num_shards, w.B, w.Q, w.h_q, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((w.num_shards, w.B, w.Q, w.h_q), dtype=torch.float32, device=dev)
        merged = torch.empty((w.B, w.Q, w.h_q, 512), dtype=out_dtype, device=dev)
        mlse = torch.empty((w.B, w.Q, w.h_q), dtype=torch.float32, device=dev)
    else:
        out = torch.empty((w.B, w.Q, w.h_q, 512), dtype=out_dtype, device=dev)
        lse = torch.empty((w.B, w.Q, w.h_q), dtype=torch.float32, device=dev)

    def step(i):
        r = i % len(kv_dev if idx_dev is None else idx_dev)
        if idx_dev is not None:
            md.mla_decode_sparse(d.q, d.kv, d.block_table, d.seq_lens, idx_dev[r], scale=w.scale,
                                 max_seq_len=w.max_seq_len, top_k=w.top_k, index_stride_b=w.index_stride_b,
                                 index_stride_q=w.index_stride_q, num_shards=w.num_shards,
                                 interleave=w.interleave, shard_id=-1, out=out, lse=lse,
                                 workspace=workspace, stream=stream, kv_scale=d.kv_scale)
        else:
            md.mla_decode_dense(d.q, kv_dev[r], d.block_table, d.seq_lens, scale=w.scale,
                                max_seq_len=w.max_seq_len, num_shards=w.num_shards, interleave=w.interleave,
                                shard_id=-1, out=out, lse=lse, workspace=workspace, stream=stream,
                                kv_scale=d.kv_scale)
        if sharded:
            md.mla_merge_lse(out, lse, out=merged, lse_out=mlse, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The timed region: K steps between two synchronizations, with an event
    # between every chunk of steps (events only mark the stream; nothing waits
    # on them inside the region).  The rate is the region's mean; the chunk
    # median is robust to a slow stretch (the clock varies with power draw).
    chunk = max(1, args.steps // 10)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range((args.steps + chunk - 1) // chunk + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(args.steps):
        step(i)
        if (i + 1) % chunk == 0 or i + 1 == args.steps:
            marks[(i + chunk) // chunk].record(stream)
    torch.cuda.synchronize()
    ms_per_step = marks[0].elapsed_time(marks[-1]) / args.steps
    bounds = list(range(0, args.steps, chunk)) + [args.steps]
    chunk_ms = np.array([marks[k].elapsed_time(marks[k + 1]) / (bounds[k + 1] - bounds[k])
                         for k in range(len(marks) - 1)])

    # Per-call times: a second pass of K steps with an event pair around each
    # call (the per-call median the workload description asks for; the pairs
    # themselves add a little to each call).
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(pairs):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    per_step = np.array([e0.elapsed_time(e1) for e0, e1 in pairs])

    # One step is one library call: the decode kernel plus, when the planner
    # splits sequences into partitions (or for DCP shards), the merge kernel.
    # The whole call is the measured unit; profiles/ gives the per-kernel split.
    call_ms = ms_per_step

    # Work per step (averaged over the rotating index sets).
    if idx_host is not None:
        works = []
        for x in idx_host:
            lists = np.asarray(x).reshape(w.B, -1)[:, :w.top_k]
            works.append(algorithmic_work(w, lists))
        work = {k: float(np.mean([x[k] for x in works])) for k in works[0]}
    else:
        work = algorithmic_work(w)
    value = work["kv_token_heads"] / (ms_per_step * 1e-3)
    t_roof_hbm = work["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_roof_mfma = work["flops"] / (MFMA_BF16_PEAK_TFS * 1e12)
    bound = "hbm" if t_roof_hbm >= t_roof_mfma else "mfma"
    achieved_gbs = work["bytes"] / (call_ms * 1e-3) / 1e9
    achieved_tfs = work["flops"] / (call_ms * 1e-3) / 1e12
    traffic = stored_traffic(w.name)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "KV-token·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Q": w.Q, "h_q": w.h_q, "kv_dtype": args.kv,
                   "seq_len": int(w.max_seq_len), "top_k": w.top_k or None,
                   "num_shards": w.num_shards, "block_size": w.block_size,
                   "out_dtype": args.out_dtype, "rotating_input_sets": len(idx_dev or kv_dev),
                   "split_kv_partitions": splits, "grid": plan["grid"]},
        "roofline": {"bound": bound,
                     "achieved": achieved_gbs if bound == "hbm" else achieved_tfs,
                     "peak": HBM_PEAK_GBS if bound == "hbm" else MFMA_BF16_PEAK_TFS,
                     "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                     "frac": (achieved_gbs / HBM_PEAK_GBS) if bound == "hbm" else
                             (achieved_tfs / MFMA_BF16_PEAK_TFS),
                     "traffic": traffic,
                     "kernel": "decode_kernel" + ("+merge_kernel" if splits > 1 or sharded else ""),
                     "launch_ms": call_ms,
                     "mfma_tflops": achieved_tfs,
                     "mfma_frac": achieved_tfs / MFMA_BF16_PEAK_TFS,
                     "algorithmic_bytes": work["bytes"], "algorithmic_flops": work["flops"]},
    }
    rec["timing"] = {"mean_ms": ms_per_step, "chunk_steps": chunk,
                     "chunk_median_ms": float(np.median(chunk_ms)),
                     "chunk_min_ms": float(chunk_ms.min()), "chunk_max_ms": float(chunk_ms.max()),
                     "per_call_median_ms": float(np.median(per_step)),
                     "per_call_min_ms": float(per_step.min()), "per_call_max_ms": float(per_step.max())}
    copy_gbs = measure_copy_gbs(torch, dev)
    rec["roofline"]["copy_gbs"] = copy_gbs
    rec["roofline"]["frac_of_copy"] = achieved_gbs / copy_gbs
    print(f"[bench] {ms_per_step * 1e3:.1f} us/step (chunk median {np.median(chunk_ms) * 1e3:.1f}, per-call median "
          f"{np.median(per_step) * 1e3:.1f}; {splits} partitions "
          f"per unit), {achieved_gbs:.0f} GB/s algorithmic = {achieved_gbs / HBM_PEAK_GBS:.3f} of HBM peak, "
          f"{achieved_gbs / copy_gbs:.3f} of the measured copy rate ({copy_gbs:.0f} GB/s)",
          file=sys.stderr, flush=True)
    if args.cpu_seconds > 0:
        # The GPU result on the workload's own inputs, for the CPU leg's comparison.
        step(0)
        torch.cuda.synchronize()
        o_res, l_res = (merged, mlse) if sharded else (out, lse)
        gpu_out = (o_res.float().cpu().numpy().astype(np.float64).reshape(-1, 512),
                   l_res.float().cpu().numpy().astype(np.float64).reshape(-1), o_res.dtype == torch.bfloat16)
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, gpu_out)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
