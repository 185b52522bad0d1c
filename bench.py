"""Benchmark of one data-parallel rank's ZeRO mixed-precision optimizer step
on one MI355X.

A step is one pass of the whole hot path over the rank's shard:
  zds_grad_accumulate_norm (copy the per-tensor grads into the flat bucket,
  with the overflow/norm pass fused in; --unfused runs zds_grad_accumulate
  and zds_overflow_and_norm instead), zds_adam_step, zds_loss_scaler_update.
  The Stage-2 intake workload sums the peers' slices with
  zds_reduce_peer_slices_norm (the norm fused in the same way) in place of
  the flatten.
Default workload: the Llama-7B-shaped Stage-1 shard at N = 8 (rank 0: 33
table entries, 842,301,440 params), bf16 grads N(0, 2e-3), fp32 master
N(0, 0.02), moments shaped like one prior step, static loss scale 1, clip
1.0, AdamW lr 1e-3 (0.9, 0.999) eps 1e-8 wd 0.01, bf16 params out.

Prints one JSON line. `value` is params updated per second over the timed
steps (inputs resident in HBM); `roofline` is for the dominant kernel
(zds_adam_step, 28 algorithmic bytes per param for 16-bit grads), timed with
HIP events on the stream it runs on; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload on the host.
"""

import argparse
import json
import os
import sys
import time

METRIC = "params updated/sec and achieved HBM GB/s (% of peak) per ZeRO Adam step"
HBM_PEAK_GBS = 8000.0


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b_s1",
                    choices=["llama7b_s1", "llama7b_s1_accum16", "llama7b_whole_1024", "llama65b_s1", "tiny",
                             "llama7b_s2_intake8", "llama7b_s1_offload", "llama7b_s1_checkpoint",
                             "llama7b_s1_onebit8"])
    ap.add_argument("--offload-threads", type=int, default=0,
                    help="host threads for the offloaded optimizer (0: all available)")
    ap.add_argument("--ckpt-dir", default=None,
                    help="directory for the checkpoint workload's shard file (default: a new one under $TMPDIR)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured into a HIP graph and replayed (copy-mode workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="separate overflow/norm pass instead of the one fused into the last "
                         "flatten/accumulate call")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="oracle sample size in params (default: the whole shard, at most 2^30)")
    ap.add_argument("--cpu-repeats", type=int, default=2, help="oracle passes over the sample")
    ap.add_argument("--cpu-procs", type=int, default=None,
                    help="oracle host processes (default: the CPUs of the affinity mask)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run torch's device copy of a known size (1 GiB read + 1 GiB write) "
                         "5 times, to calibrate HBM byte counters")
    return ap.parse_args()


# ------------------------------------------------------------------ workloads

def _workload(name):
    from workloads import llama_7b_tensors, llama_65b_tensors, llama_7b_split_1024, tiny_shard_sizes
    if name == "llama7b_s1":
        return dict(tensors=llama_7b_tensors(), world=8, rank=0, gdt="bf16", pdt="bf16", sigma=2e-3,
                    accum=1, scale=None, prior=True, mode="copy")
    if name == "llama7b_s1_accum16":
        return dict(tensors=llama_7b_tensors(), world=8, rank=0, gdt="fp16", pdt="fp16", sigma=1e-3,
                    accum=16, scale=14, prior=True, mode="accumulate")
    if name == "llama7b_whole_1024":
        return dict(tensors=llama_7b_split_1024(), world=1, rank=0, gdt="fp16", pdt="fp16", sigma=1e-3,
                    accum=1, scale=16, prior=False, mode="copy")
    if name == "llama7b_s2_intake8":
        # Stage 2 at N = 8: the rank sums the 8 peers' bf16 copies of its slice
        # into an fp32 shard gradient, then steps on it (mean over the peers)
        return dict(tensors=llama_7b_tensors(), world=8, rank=0, gdt="bf16", pdt="bf16", sigma=2e-3,
                    accum=8, scale=None, prior=True, mode="intake", peers=8)
    if name == "llama7b_s1_offload":
        # the C2 shard with its fp32 optimizer state in pinned host memory
        return dict(tensors=llama_7b_tensors(), world=8, rank=0, gdt="bf16", pdt="bf16", sigma=2e-3,
                    accum=1, scale=None, prior=True, mode="copy", offload=True)
    if name == "llama7b_s1_checkpoint":
        # save and reload the C2 shard's optimizer state (master, m, v, state)
        return dict(tensors=llama_7b_tensors(), world=8, rank=0, gdt="bf16", pdt="bf16", sigma=2e-3,
                    accum=1, scale=None, prior=True, mode="copy", checkpoint=True)
    if name == "llama7b_s1_onebit8":
        # 1-bit codec on the C2 shard: encode with error feedback, then the
        # decode-sum of 8 peers' messages, chunk 2048
        return dict(tensors=llama_7b_tensors(), world=8, rank=0, gdt="bf16", pdt="bf16", sigma=2e-3,
                    accum=1, scale=None, prior=False, mode="copy", onebit=True, peers=8, chunk=2048)
    if name == "llama65b_s1":
        return dict(tensors=llama_65b_tensors(), world=8, rank=0, gdt="bf16", pdt="bf16", sigma=1e-3,
                    accum=1, scale=None, prior=True, mode="copy")
    return dict(tensors=tiny_shard_sizes(), world=1, rank=0, gdt="fp16", pdt="fp16", sigma=1e-3,
                accum=1, scale=16, prior=False, mode="copy")


def _bytes_per_param(w, fused):
    """Algorithmic HBM bytes per param of each kernel of one step. Fused, the
    norm reads nothing extra: it is formed from the values the last
    flatten/accumulate call (or the intake) stores."""
    g = 2
    if w["mode"] == "intake":
        return dict(accum_total=2 * w["peers"] + 4, norm=0 if fused else 4, adam=30)
    if w["mode"] == "accumulate":
        acc = 6 + 10 * (w["accum"] - 1)      # overwrite once, then accumulate
        return dict(accum_total=acc, norm=0 if fused else 4, adam=30)
    return dict(accum_total=2 * g, norm=0 if fused else g, adam=28)


# ------------------------------------------------------------------ GPU part

def run_gpu(args, w):
    import torch
    from zero_sharded_mixed_tensor_amd import zds
    from zero_sharded_mixed_tensor_amd.step import ShardStep

    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}
    numels = [n for _, n in w["tensors"]]
    _, total = zds.zds_flat_layout(numels, 64)
    lo, hi = zds.zds_shard_range(total, w["world"], w["rank"], 64)
    n = hi - lo
    plan = zds.zds_plan_create(numels, 64, lo, hi)
    ents = plan.entries()
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)

    # per-tensor grads of the tensors this shard touches (whole tensors)
    srcs = [None] * len(numels)
    for t, _, _, _ in ents:
        if w["mode"] != "intake":
            srcs[t] = torch.empty(numels[t], dtype=tdt[w["gdt"]], device=dev)
    scale = 1.0 if w["scale"] is None else 2.0 ** w["scale"]

    def fill_grads(k):
        g = torch.Generator(device=dev)
        g.manual_seed(5000 + k)
        for s in srcs:
            if s is not None:
                s.normal_(0.0, w["sigma"] * scale, generator=g)

    fill_grads(0)
    master = torch.empty(n, dtype=torch.float32, device=dev).normal_(0.0, 0.02, generator=gen)
    if w["prior"]:
        m = torch.empty(n, dtype=torch.float32, device=dev).normal_(0.0, 0.1 * w["sigma"], generator=gen)
        v = torch.empty(n, dtype=torch.float32, device=dev).normal_(0.0, w["sigma"], generator=gen)
        v.mul_(v).mul_(0.001)
        t0, b1p, b2p = 1, float(torch.tensor(0.9, dtype=torch.float32)), float(torch.tensor(0.999, dtype=torch.float32))
    else:
        m = torch.zeros(n, dtype=torch.float32, device=dev)
        v = torch.zeros(n, dtype=torch.float32, device=dev)
        t0, b1p, b2p = 0, 1.0, 1.0
    p16 = master.to(tdt[w["pdt"]])
    if w["mode"] == "intake":
        peers = []
        for k in range(w["peers"]):
            pk = torch.empty(n, dtype=tdt[w["gdt"]], device=dev)
            gk = torch.Generator(device=dev)
            gk.manual_seed(7000 + k)
            peers.append(pk.normal_(0.0, w["sigma"], generator=gk))
        bucket = torch.zeros(n, dtype=torch.float32, device=dev)
    elif w["mode"] == "accumulate":
        bucket = torch.zeros(n, dtype=torch.float32, device=dev)
    else:
        bucket = torch.zeros(n, dtype=tdt[w["gdt"]], device=dev)
    cfg = (zds.scaler_config(dynamic=False, static_scale=1.0) if w["scale"] is None
           else zds.scaler_config(initial_scale_power=w["scale"], window=1000, hysteresis=1))
    st = ShardStep(n, zds.hparams(), cfg, max_norm=1.0, accum_steps=w["accum"], t0=t0,
                   beta1_pow0=b1p, beta2_pow0=b2p)
    fused = not args.unfused
    pws = zds.new_plan_workspace(plan)
    rws = zds.new_reduce_workspace(n) if w["mode"] == "intake" else None
    # the grads live in fixed buffers: their pointers are marshalled once
    bound = zds.SourceSet(plan, srcs) if w["mode"] != "intake" else None
    torch.cuda.synchronize()

    ev = {k: [] for k in ("accumulate", "norm", "adam", "scaler")}

    def one_step(record):
        def mark():
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            return e
        e0 = mark() if record else None
        modes = ([zds.ZDS_OVERWRITE] + [zds.ZDS_ACCUMULATE] * (w["accum"] - 1)
                 if w["mode"] == "accumulate" else [] if w["mode"] == "intake" else [zds.ZDS_COPY])
        if w["mode"] == "intake":
            if fused:
                st.intake_norm(peers, bucket, zds.ZDS_OVERWRITE, rws)
            else:
                zds.zds_reduce_peer_slices(peers, bucket, zds.ZDS_OVERWRITE)
        for k, md in enumerate(modes):
            if fused and k == len(modes) - 1:
                st.accumulate_norm(plan, bound, bucket, md, pws)
            else:
                zds.zds_grad_accumulate(plan, bound, bucket, md)
        e1 = mark() if record else None
        if not fused:
            st.norm(bucket)
        e2 = mark() if record else None
        st.adam(bucket, master, m, v, p16)
        e3 = mark() if record else None
        st.scaler()
        e4 = mark() if record else None
        if record:
            ev["accumulate"].append((e0, e1))
            ev["norm"].append((e1, e2))
            ev["adam"].append((e2, e3))
            ev["scaler"].append((e3, e4))

    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        one_step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    state = st.read_state()
    sc = st.read_scalars()
    if sc.overflow or state.steps_skipped:
        raise SystemExit("unexpected overflow in the benchmark workload")

    bpp = _bytes_per_param(w, fused)
    kern = {}
    for k, pairs in ev.items():
        if k == "norm" and fused:
            continue
        ms = sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
        entry = {"ms_avg": round(ms, 5)}
        if k == "accumulate":
            entry["gbs"] = round(bpp["accum_total"] * n / (ms * 1e-3) / 1e9, 1)
            if fused:
                entry["includes"] = ("overflow/norm fused into the intake" if w["mode"] == "intake"
                                     else "overflow/norm fused into the last call")
        elif k in ("norm", "adam"):
            entry["gbs"] = round(bpp[k] * n / (ms * 1e-3) / 1e9, 1)
        kern[k] = entry
    adam_ms = kern["adam"]["ms_avg"]
    achieved = bpp["adam"] * n / (adam_ms * 1e-3) / 1e9
    if w["mode"] == "intake":
        kern["intake"] = kern.pop("accumulate")
    step_bytes = (bpp["accum_total"] + bpp["norm"] + bpp["adam"]) * n
    ms_per_step = elapsed / args.steps * 1e3
    graph = None
    if args.graph and fused and w["mode"] == "copy":
        # the same step captured once into a HIP graph, then replayed
        g = st.capture(plan, bound, bucket, zds.ZDS_COPY, pws, master, m, v, p16)
        for _ in range(max(1, args.warmup)):
            g.replay()
        torch.cuda.synchronize()
        t_g = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t_g) / args.steps * 1e3
        graph = {"ms_per_step": round(g_ms, 4), "params_per_s": round(n / (g_ms * 1e-3), 1),
                 "vs_eager": round(ms_per_step / g_ms, 3)}
    # params counted in params/s: the shard's elements that belong to a
    # tensor (the flat layout's alignment padding is moved but not counted)
    n_real = n if w["mode"] == "intake" else sum(e[2] for e in ents)
    return dict(n=n, n_real=n_real, entries=len(ents), elapsed=elapsed, ms_per_step=ms_per_step, kernels=kern,
                fused=fused,
                graph=graph,
                adam_gbs=achieved, step_gbs=step_bytes / (elapsed / args.steps) / 1e9,
                step_bytes_per_param=bpp["accum_total"] + bpp["norm"] + bpp["adam"],
                adam_bytes_per_param=bpp["adam"])


def run_offload(args, w):
    """The shard's fp32 optimizer state in pinned host memory: flatten on the
    device, then OffloadStep (device norm, chunked download, host AdamW on
    all host threads, upload of the 16-bit params, device scaler). Timed by
    wall clock per step (the host update is synchronous)."""
    import torch
    from zero_sharded_mixed_tensor_amd import zds
    from zero_sharded_mixed_tensor_amd.step import OffloadStep

    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}
    numels = [n for _, n in w["tensors"]]
    _, total = zds.zds_flat_layout(numels, 64)
    lo, hi = zds.zds_shard_range(total, w["world"], w["rank"], 64)
    n = hi - lo
    plan = zds.zds_plan_create(numels, 64, lo, hi)
    dev = torch.device("cuda", 0)
    srcs = [None] * len(numels)
    for t, _, _, _ in plan.entries():
        g = torch.Generator(device=dev)
        g.manual_seed(5000 + t)
        srcs[t] = torch.empty(numels[t], dtype=tdt[w["gdt"]], device=dev).normal_(0.0, w["sigma"], generator=g)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    host = []
    for sig in (0.02, 0.1 * w["sigma"], w["sigma"]):
        d = torch.empty(n, dtype=torch.float32, device=dev).normal_(0.0, sig, generator=gen)
        h = torch.empty(n, dtype=torch.float32, pin_memory=True)
        h.copy_(d)
        host.append(h)
        del d
    host[2].mul_(host[2]).mul_(0.001)
    b1p, b2p = float(torch.tensor(0.9, dtype=torch.float32)), float(torch.tensor(0.999, dtype=torch.float32))
    off = OffloadStep(n, host[0], host[1], host[2], tdt[w["gdt"]], tdt[w["pdt"]], zds.hparams(),
                      zds.scaler_config(dynamic=False, static_scale=1.0), max_norm=1.0, t0=1, beta1_pow0=b1p,
                      beta2_pow0=b2p, threads=args.offload_threads)
    bucket = torch.empty(n, dtype=tdt[w["gdt"]], device=dev)
    p16 = torch.empty(n, dtype=tdt[w["pdt"]], device=dev)

    bound = zds.SourceSet(plan, srcs)

    def one():
        zds.zds_grad_accumulate(plan, bound, bucket, zds.ZDS_COPY)
        off.step(bucket, p16)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    import os as _os
    threads = args.offload_threads or len(_os.sched_getaffinity(0))
    return {
        "metric": METRIC, "value": round(n * args.steps / el, 1), "unit": "params/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(el / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "params": n, "grad_dtype": w["gdt"], "param_dtype": w["pdt"],
                   "optimizer_state": "pinned host memory", "host_threads": threads,
                   "host_bytes_per_param": 28, "pcie_bytes_per_param": 4},
        "host_update_gbs": round(28 * n * args.steps / el / 1e9, 1),
    }


def run_onebit(args, w):
    """One rank's codec work per exchange on its shard: zds_onebit_compress of
    an fp32 buffer with its error buffer, then zds_onebit_decompress of the
    8 peers' messages into an fp32 buffer. Each kernel is timed with HIP
    events on the stream it runs on."""
    import torch
    from zero_sharded_mixed_tensor_amd import zds
    from workloads.device import draw_payload_, fill_normal_

    numels = [n for _, n in w["tensors"]]
    _, total = zds.zds_flat_layout(numels, 64)
    lo, hi = zds.zds_shard_range(total, w["world"], w["rank"], 64)
    n, chunk, N = hi - lo, w["chunk"], w["peers"]
    x = fill_normal_(torch.empty(n, dtype=torch.float32, device="cuda"), w["sigma"], 91)
    err = fill_normal_(torch.empty(n, dtype=torch.float32, device="cuda"), 1e-2 * w["sigma"], 92)
    mine = zds.onebit_payload(n, chunk)
    peers = [draw_payload_(*zds.onebit_payload(n, chunk), w["sigma"], 93 + k) for k in range(N)]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    enc_ms, dec_ms = [], []

    def one(record):
        if record:
            ev[0].record(stream)
        zds.zds_onebit_compress(x, err, chunk, *mine)
        if record:
            ev[1].record(stream)
        zds.zds_onebit_decompress(peers, chunk, out)
        if record:
            ev[2].record(stream)

    for _ in range(args.warmup):
        one(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one(True)
        torch.cuda.synchronize()
        enc_ms.append(ev[0].elapsed_time(ev[1]))
        dec_ms.append(ev[1].elapsed_time(ev[2]))
    el = time.perf_counter() - t0
    payload_b = (n + 2047) // 2048 * 256 + (n + chunk - 1) // chunk * 4  # sign words + scales
    enc_b = 12 * n + payload_b
    dec_b = N * payload_b + 4 * n
    e_ms, d_ms = sum(enc_ms) / len(enc_ms), sum(dec_ms) / len(dec_ms)
    enc_gbs = enc_b / (e_ms * 1e-3) / 1e9
    return {
        "metric": "1-bit codec elements/s (encode + 8-peer decode) and achieved HBM GB/s",
        "value": round(n / ((e_ms + d_ms) * 1e-3), 1), "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(e_ms + d_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "elements": n, "chunk": chunk, "peers": N,
                   "encode_bytes": enc_b, "decode_bytes": dec_b},
        "kernels": {"encode": {"ms_avg": round(e_ms, 5), "gbs": round(enc_gbs, 1)},
                    "decode": {"ms_avg": round(d_ms, 5), "gbs": round(dec_b / (d_ms * 1e-3) / 1e9, 1)}},
        "roofline": {"kernel": "zds_onebit_compress", "bound": "hbm", "achieved": round(enc_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(enc_gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_element": round(enc_b / n, 4),
                     "traffic": _traffic(args.workload, n, "onebit_encode_kernel")},
        "wall_s": round(el, 3),
    }


def run_checkpoint(args, w):
    """Save the rank's device shard (fp32 master, exp_avg, exp_avg_sq and the
    step state) to one file and load it back into fresh device buffers, timed
    by wall clock; the reload is checked bit for bit against what was saved.
    The file goes through the page cache (no fsync), so a reload right after
    a save reads host memory, not the disk."""
    import shutil
    import tempfile
    import torch
    from zero_sharded_mixed_tensor_amd import zds
    from zero_sharded_mixed_tensor_amd.step import ShardStep

    numels = [n for _, n in w["tensors"]]
    _, total = zds.zds_flat_layout(numels, 64)
    lo, hi = zds.zds_shard_range(total, w["world"], w["rank"], 64)
    n = hi - lo
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4321)
    src = [torch.empty(n, dtype=torch.float32, device=dev).normal_(0.0, s, generator=gen)
           for s in (0.02, 0.1 * w["sigma"], w["sigma"])]
    src[2].mul_(src[2]).mul_(0.001)
    st = ShardStep(n, zds.hparams(), zds.scaler_config(dynamic=False, static_scale=1.0), t0=1,
                   beta1_pow0=0.9, beta2_pow0=0.999)
    dst = [torch.empty_like(x) for x in src]
    state2 = zds.new_state()
    meta = zds.checkpoint_meta(numels, w["world"], w["rank"], 64, stage=1)
    made = args.ckpt_dir is None
    d = tempfile.mkdtemp(prefix="zds_ckpt_", dir=os.environ.get("TMPDIR", "/tmp")) if made else args.ckpt_dir
    path = os.path.join(d, "zero_rank%d.zckpt" % w["rank"])
    reps = max(1, min(args.steps, 3))
    file_bytes = 256 + 8 * len(numels) + 12 * n
    try:
        torch.cuda.synchronize()
        saves, loads = [], []
        for _ in range(reps):
            t0 = time.perf_counter()
            zds.zds_checkpoint_save(path, meta, numels, *src, st.state)
            saves.append(time.perf_counter() - t0)
            for x in dst:
                x.fill_(float("nan"))
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            zds.zds_checkpoint_load(path, meta, numels, *dst, state2)
            loads.append(time.perf_counter() - t0)
            exact = all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(src, dst))
            exact = exact and torch.equal(st.state, state2)
            if not exact:
                raise RuntimeError("the reloaded shard differs from the saved one")
        assert os.path.getsize(path) == file_bytes
    finally:
        if made:
            shutil.rmtree(d, ignore_errors=True)
        elif os.path.exists(path):
            os.remove(path)
    save_s, load_s = min(saves), min(loads)
    return {
        "metric": "rank shard checkpoint save + reload throughput", "value": round(2 * file_bytes / (save_s + load_s) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 0,
        "ms_per_step": round((save_s + load_s) * 1e3, 1), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "params": n, "file_bytes": file_bytes,
                   "sections": "master, exp_avg, exp_avg_sq (fp32) + 64-byte step state", "fsync": False},
        "save_gbs": round(file_bytes / save_s / 1e9, 2), "load_gbs": round(file_bytes / load_s / 1e9, 2),
        "save_ms": [round(x * 1e3, 1) for x in saves], "load_ms": [round(x * 1e3, 1) for x in loads],
        "bit_exact_reload": True,
    }


# ------------------------------------------------------------------ CPU oracle part

def _oracle_worker(conn, w, n, c0, c1, chunk):
    """One host process of the CPU baseline: generates its share of the
    workload's inputs (chunks c0 .. c1-1 of `chunk` params; not timed), then
    on each "go" runs the oracle's step on them in two phases, the global
    norm being combined by the parent in between (the scalars of row a2 are
    global over the shard)."""
    import numpy as np
    import oracle as O
    from workloads import draw_grads, draw_master, draw_prior_moments

    scale = 1.0 if w["scale"] is None else 2.0 ** w["scale"]
    nsrc = w["peers"] if w["mode"] == "intake" else (w["accum"] if w["mode"] == "accumulate" else 1)
    parts = []
    for c in range(c0, c1):
        a = c * chunk
        ln = min(chunk, n - a)
        g = [draw_grads(ln, w["gdt"], w["sigma"], scale, 1 + k, 2, 0, offset=a) for k in range(nsrc)]
        master = draw_master(ln, 0.02, 1, 2, offset=a)
        if w["prior"]:
            m, v = draw_prior_moments(ln, w["sigma"], 1, 2, offset=a)
        else:
            m, v = np.zeros(ln, np.float32), np.zeros(ln, np.float32)
        parts.append((ln, g, master, m, v))
    conn.send("ready")
    xdt = w["gdt"] if w["mode"] == "copy" else "fp32"
    while conn.recv() == "go":
        xs, sums, ovf = [], [], 0
        for ln, g, _, _, _ in parts:
            ent = [(0, 0, ln, 0)]
            if w["mode"] == "intake":
                x = O.reduce_peer_slices(g, w["gdt"], None, "fp32", accumulate=False)
            elif w["mode"] == "accumulate":
                x = np.empty(ln, np.float32)
                for k, src in enumerate(g):
                    O.flatten_accumulate([src], w["gdt"], ent, x, overwrite=(k == 0))
            else:
                x = O.flatten_copy(g, ent, np.empty(ln, np.uint16))
            sums.append(O.sum_of_squares(x, xdt))
            ovf |= O.overflow_flag(x, xdt)
            xs.append(x)
        conn.send((sums, ovf))
        gs, consts = conn.recv()
        if gs is not None:
            for x, (_, _, master, m, v) in zip(xs, parts):
                p, _, _ = O.adamw_update(x, xdt, gs, master, m, v, consts)
                O.narrow(p, w["pdt"])
        conn.send("done")


def run_cpu_baseline(w, sample=None, repeats=2, procs=None, chunk=1 << 24):
    """The oracle's whole step (the flatten copy, or the K micro-batch
    accumulation, or the intake of the peers' slices; then overflow + norm,
    AdamW + cast, scaler update) over `sample` params of the workload's shard
    (default: the whole shard up to 2^30 params), in `chunk`-param pieces
    spread over `procs` host processes (default: the CPUs of this process's
    affinity mask). Inputs are generated before timing, each process its own
    pieces; only the compute is timed (wall clock, `repeats` passes). Must
    run before this process touches the GPU: the workers are forked."""
    import multiprocessing as mp
    import oracle as O

    numels = [t for _, t in w["tensors"]]
    _, total = O.flat_layout(numels, 64)
    lo, hi = O.shard_range(total, w["world"], w["rank"], 64)
    n = min(hi - lo, sample or (1 << 30))
    nchunks = (n + chunk - 1) // chunk
    procs = max(1, min(procs or len(os.sched_getaffinity(0)), nchunks))
    ctx = mp.get_context("fork")
    workers, conns = [], []
    for i in range(procs):
        c0, c1 = nchunks * i // procs, nchunks * (i + 1) // procs
        a, b = ctx.Pipe()
        pr = ctx.Process(target=_oracle_worker, args=(b, w, n, c0, c1, chunk), daemon=True)
        pr.start()
        workers.append(pr)
        conns.append(a)
    try:
        for c in conns:
            if c.recv() != "ready":
                raise RuntimeError("oracle worker failed")
        st = O.scaler_init(dynamic=w["scale"] is not None, initial_scale_power=w["scale"] or 0,
                           static_scale=1.0, t=1 if w["prior"] else 0,
                           beta1_pow=float(O.np.float32(0.9)) if w["prior"] else 1.0,
                           beta2_pow=float(O.np.float32(0.999)) if w["prior"] else 1.0)
        times = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            for c in conns:
                c.send("go")
            sumsq, ovf = 0.0, 0
            for c in conns:                      # partials in chunk order
                s, o = c.recv()
                for x in s:
                    sumsq += x
                ovf |= o
            if ovf:
                gs, consts = None, None
            else:
                _, _, gs = O.clip_scalars(sumsq, st.scale, w["accum"], 1.0)
                consts = O.adamw_constants(O.AdamW(), st.beta1_pow, st.beta2_pow)
            for c in conns:
                c.send((gs, consts))
            for c in conns:
                if c.recv() != "done":
                    raise RuntimeError("oracle worker failed")
            O.scaler_update(st, ovf, O.AdamW().beta1, O.AdamW().beta2)
            times.append(time.perf_counter() - t0)
        for c in conns:
            c.send("stop")
    finally:
        for pr in workers:
            pr.join(timeout=60)
            if pr.is_alive():
                pr.kill()
    dt = sum(times)
    what = {"intake": "intake of %d peers' slices" % w.get("peers", 0),
            "accumulate": "accumulation of %d micro-batches" % w["accum"]}.get(w["mode"], "copy")
    return dict(value=n * repeats / dt, seconds=dt, n=n, shard=hi - lo, repeats=repeats, procs=procs,
                chunk=chunk, what=what)


def run_cpu_baseline_onebit(w, sample, repeats, min_seconds=10.0):
    """Time the oracle's codec work per exchange (encode with error feedback,
    then the decode of N peers' payloads) on `sample` elements, at least
    `repeats` times and for at least `min_seconds`."""
    import numpy as np
    import oracle as O
    n, chunk, N = sample, w["chunk"], w["peers"]
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(n) * w["sigma"]).astype(np.float32)
    err = np.zeros(n, np.float32)
    peers = [O.onebit_compress((rng.standard_normal(n) * w["sigma"]).astype(np.float32), np.zeros(n, np.float32),
                               chunk)[:2] for _ in range(N)]
    t0 = time.perf_counter()
    done = 0
    while done < repeats or time.perf_counter() - t0 < min_seconds:
        _, _, err = O.onebit_compress(x, err, chunk)
        O.onebit_decompress(peers, n, chunk, None, False)
        done += 1
    dt = time.perf_counter() - t0
    return dict(value=n * done / dt, seconds=dt, n=n, repeats=done)


def _traffic(workload, n, kernel="adam_wide_kernel"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of this workload (FETCH_SIZE and WRITE_SIZE, each scaled by a
    copy of known size), or None when there is none or the kernel's sources
    changed since it was taken."""
    from zero_sharded_mixed_tensor_amd.profiling import traffic_from_summary
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "%s_step_hbm_counters.md" % workload)
    return traffic_from_summary(path, kernel)


def _copy_calibration():
    """torch's device copy of 1 GiB, 5 times: a kernel of known traffic for
    scaling HBM byte counters."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    return {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "launches": 5}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the step shards by running this same kernel set on each rank's "
              "slice); run with --gpus 1.", file=sys.stderr)
        return 2
    w = _workload(args.workload)
    if w.get("offload"):
        print(json.dumps(run_offload(args, w)), flush=True)
        return 0
    if w.get("onebit"):
        out = run_onebit(args, w)
        if args.copy_calibration:
            out["copy_calibration"] = _copy_calibration()
        if not args.no_cpu_baseline:
            c = run_cpu_baseline_onebit(w, min(args.cpu_sample or (1 << 18), 1 << 18), args.cpu_repeats)
            out["cpu_baseline"] = {
                "value": round(c["value"], 1), "unit": "elements/s", "cores": 1, "kind": "oracle",
                "sample": "%d passes of the oracle's encode (with error feedback) and %d-peer decode over %d "
                          "elements, %.1f s" % (c["repeats"], w["peers"], c["n"], c["seconds"])}
        print(json.dumps(out), flush=True)
        return 0
    if w.get("checkpoint"):
        print(json.dumps(run_checkpoint(args, w)), flush=True)
        return 0
    # the CPU baseline first: its workers are forked, which must happen
    # before this process initialises the GPU
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(w, args.cpu_sample, args.cpu_repeats,
                                                             args.cpu_procs)
    r = run_gpu(args, w)
    out = {
        "metric": METRIC,
        "value": round(r["n_real"] * args.steps / r["elapsed"], 1),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "params": r["n_real"],
            "elements": r["n"],
            "table_entries": r["entries"],
            "grad_dtype": w["gdt"],
            "param_dtype": w["pdt"],
            "state_dtype": "fp32",
            "accum_steps": w["accum"],
            "loss_scale": "static 1" if w["scale"] is None else "dynamic 2^%d" % w["scale"],
            "clip": 1.0,
            "step_bytes_per_param": r["step_bytes_per_param"],
            "norm_fused_into_flatten": r["fused"],
        },
        "step_gbs": round(r["step_gbs"], 1),
        **({"graph": r["graph"]} if r["graph"] else {}),
        "step_hbm_frac": round(r["step_gbs"] / HBM_PEAK_GBS, 4),
        "kernels": r["kernels"],
        "roofline": {
            "kernel": "zds_adam_step",
            "bound": "hbm",
            "achieved": round(r["adam_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["adam_gbs"] / HBM_PEAK_GBS, 4),
            "bytes_per_param": r["adam_bytes_per_param"],
            "traffic": _traffic(args.workload, r["n"]),
        },
    }
    if args.copy_calibration:
        out["copy_calibration"] = _copy_calibration()
    if cpu is not None:
        out["cpu_baseline"] = {
            "value": round(cpu["value"], 1),
            "unit": "params/s",
            "cores": cpu["procs"],
            "kind": "oracle",
            "sample": "%d passes of one whole oracle step (%s, overflow+norm, AdamW, cast, scaler) over "
                      "%s (%d params) in %d-param pieces on %d host processes, %.2f s of compute "
                      "(inputs generated before timing)"
                      % (cpu["repeats"], cpu["what"],
                         "the whole shard" if cpu["n"] == cpu["shard"] else "the first %d params of the shard"
                         % cpu["n"], cpu["n"], cpu["chunk"], cpu["procs"], cpu["seconds"]),
        }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
