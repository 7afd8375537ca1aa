"""Benchmark of one ConvKV AR step on one MI355X.

A step is one pass of the whole hot path for one cache (one layer, one diffusion step):
lact_rope_reset_apply -> lact_block_attention -> lact_kv_ring_append ->
lact_convkv_compress, at steady state (memory full: 16 slots + 8 window frames + the
8-frame block, Lq 8192, Lk 32768 at 512x512).  Inputs are seeded synthetic tensors of the
workload's shapes, generated before timing and resident in HBM (a pool of 7 blocks cycled
through, so consecutive steps read different data).

Prints one JSON line: whole-step latent frames/s as `value`, the attention kernel's
achieved TFLOP/s against the bf16 MFMA peak in `roofline`, the CPU oracle timed on a
bounded sample of the same step in `cpu_baseline`, and in `parity` the device's output for
that sample (computed after the timed region) against the oracle's.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload s512_bf16]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("ConvKV block-attn TFLOP/s + latent frames/s per AR step (512×512); "
          "% of roofline")
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}  # dense MFMA TFLOP/s, MI355X
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="s512_bf16")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--pool-blocks", type=int, default=7)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=512, help="oracle rows per head in the sample")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="run one device copy of MIB MiB first (reference for HBM byte counters)")
    p.add_argument("--cold", type=int, default=5, metavar="STEPS",
                   help="after the timed steps, run STEPS more with a 512 MiB read before each "
                        "RoPE, append and compress call (last-level cache flushed) and report "
                        "those calls' times as 'cold' (0: skip)")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured ceilings (matrix-core loop, streaming copies)")
    return p.parse_args()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "compressed_kv_causal_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_file, launches_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    ent = d.get(launches_key)
    if not ent or ent.get("source_hash") != source_hash(kernel_file):
        return None
    return ent.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the ConvKV step is measured on a single MI355X "
              "(the library has no sharding or collectives); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import compressed_kv_causal_amd as L
    import synth

    w = synth.workload(args.workload)
    if w.get("train_blocks"):
        return train_main(args, w)
    if w.get("members", 1) > 1:
        return set_main(args, w)
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    B = w["block"]
    dt = {0: "f32", 1: "bf16", 2: "fp8"}[w["kv_dtype"]]   # storage of the cache
    op = "f32" if w["q_dtype"] == 0 else "bf16"          # arithmetic of the attention
    io = torch.float32 if w["q_dtype"] == 0 else torch.bfloat16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs: a pool of blocks resident in HBM ------------------------------------
    pool = []
    for blk in range(args.pool_blocks):
        ids = list(range(blk * B, (blk + 1) * B))
        trip = []
        for tensor in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V):
            x = synth.frames(w, args.seed, tensor, ids).reshape(B * T, H, D)
            trip.append(torch.from_numpy(x).to(io).to(dev))
        pool.append(trip)
    wk, bk = synth.conv_weights(w, args.seed, synth.TENSOR_WK)
    wv, bv = synth.conv_weights(w, args.seed, synth.TENSOR_WV)
    d_wk, d_bk, d_wv, d_bv = (torch.from_numpy(a).to(dev) for a in (wk, bk, wv, bv))

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cache = L.Cache(L.make_cfg(**w), device=dev)
    if w.get("ref_frames", 0):
        kr, vr = synth.ref_frames(w, args.seed)
        n_ref = kr.shape[0]
        cache.ref_set(*(torch.from_numpy(x.reshape(n_ref * T, H, D)).to(io).to(dev)
                        for x in (kr, vr)))
    Lq = B * T
    out = torch.empty((Lq, H, D), dtype=io, device=dev)
    lse = torch.empty((H, Lq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    h = cache.h
    first_block = w["first_block"]

    def step(i, ev=None):
        q, k, v = pool[i % len(pool)]
        n = first_block if i == 0 else B
        if n != B:
            q, k, v = q[: n * T], k[: n * T], v[: n * T]
        if ev is not None:
            ev[0].record(stream)
        L.lact_rope_reset_apply(h, q, k, v, n, stream)
        if ev is not None:
            ev[1].record(stream)
        L.lact_block_attention(h, None, out[: n * T], lse[:, : n * T] if n == B else None, stream)
        if ev is not None:
            ev[2].record(stream)
        L.lact_kv_ring_append(h, k, v, n, stream)
        if ev is not None:
            ev[3].record(stream)
        L.lact_convkv_compress(h, d_wk, d_bk, d_wv, d_bv, stream)
        if ev is not None:
            ev[4].record(stream)

    # fill the memory: after 11 blocks of 8 frames, 80 frames were evicted -> 16 slots
    i = 0
    while True:
        st = cache.state()
        if st["mem_len"] == w["mem_slots"] and st["win_len"] == w["window_frames"] and i > 0:
            break
        step(i)
        i += 1
    for _ in range(args.warmup):
        step(i)
        i += 1
    torch.cuda.synchronize()
    n_hist = cache.state()["mem_len"] + cache.state()["win_len"] + w.get("ref_frames", 0)
    Lk = (n_hist + B) * T

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(i, evs[s])
        i += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part = np.array([[evs[s][j].elapsed_time(evs[s][j + 1]) for j in range(4)]
                     for s in range(args.steps)])  # ms

    # the first block (no history) of a second, fresh cache, timed on its own
    first = L.Cache(L.make_cfg(**w), device=dev)
    if w.get("ref_frames", 0):
        first.ref_set(*(torch.from_numpy(x.reshape(n_ref * T, H, D)).to(io).to(dev)
                        for x in (kr, vr)))
    fq, fk, fv = (t[: first_block * T] for t in pool[0])
    fev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    fev[0].record(stream)
    L.lact_rope_reset_apply(first.h, fq, fk, fv, first_block, stream)
    fev[1].record(stream)
    L.lact_block_attention(first.h, None, out[: first_block * T], None, stream)
    fev[2].record(stream)
    L.lact_kv_ring_append(first.h, fk, fv, first_block, stream)
    fev[3].record(stream)
    L.lact_convkv_compress(first.h, d_wk, d_bk, d_wv, d_bv, stream)
    fev[4].record(stream)
    torch.cuda.synchronize()
    first_ms = [fev[j].elapsed_time(fev[j + 1]) for j in range(4)]
    first.close()
    del first
    ms = part.mean(axis=0)
    ms_step_events = float(part.sum(axis=1).mean())
    step_pct = np.percentile(part.sum(axis=1), [10, 50, 90])
    ms_per_step = wall * 1e3 / args.steps

    fe = T * H * D                                   # elements per frame
    kvb = {"f32": 4, "bf16": 2, "fp8": 1}[dt]        # stored bytes per element
    ob = 4 if w["q_dtype"] == 0 else 2               # input / staged operand bytes
    sb = T * H * 4 if dt == "fp8" else 0             # f32 row scales per stored frame
    attn_flop = 4.0 * Lq * Lk * D * H
    attn_tflops = attn_flop / (ms[1] * 1e-3) / 1e12
    peak = PEAK[op]
    # algorithmic bytes of the streaming kernels (per step)
    hist_k = n_hist * (fe * (kvb + ob) + sb)         # stored K read, rotated operand written
    # the block: q, k read and qrot, krot written in the operand dtype; an FP8 cache's V
    # also read and written as codes + row scales (a bf16 or f32 cache's attention reads the
    # block's V where the caller passed it, so the pass does not touch it)
    cur = B * (fe * (5 * ob + kvb) + sb) if dt == "fp8" else B * fe * 4 * ob
    # FP8: every key's V scale read, its three attention-order terms written
    vstage = Lk * H * 16 if dt == "fp8" else 0
    rope_bytes = hist_k + cur + vstage
    append_bytes = 2 * B * (fe * (ob + kvb) + sb)
    slots_per_step = B / w["ratio"]
    compress_bytes = slots_per_step * 2 * (fe * kvb + sb) * (w["ratio"] + 1)
    traffic = load_traffic("k_attn.hip", f"attn_{args.workload}")
    # query tiles the fast attention pass handed to the exact pass in the last step
    n_flags = H * ((Lq + 255) // 256)
    flags = cache.buf[cache.layout.attn_flags:].view(torch.int32)[:n_flags]
    exact_tiles = int(flags.sum().item()) if w["q_dtype"] != 0 else 0

    rec = {
        "metric": METRIC,
        "value": round(B / (ms_per_step * 1e-3), 2),
        "unit": "latent frames/s (one layer, one diffusion step, steady state)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": op,
        "data": "synthetic (seeded N(0,1) Q/K/V, N(0,0.2) conv weights; HDTF/EMTD stand-in)",
        "config": {"workload": args.workload, "kv_storage": dt, "heads": H, "head_dim": D, "tokens_per_frame": T,
                   "block_frames": B, "window_frames": w["window_frames"],
                   "mem_slots": w["mem_slots"], "ratio": w["ratio"], "Lq": Lq, "Lk": Lk},
        "attn_tflops": round(attn_tflops, 2),
        "attn_exact_pass_tiles": f"{exact_tiles}/{n_flags}",
        "first_block": {"frames": first_block, "Lq": first_block * T,
                        "Lk": (first_block + w.get("ref_frames", 0)) * T,
                        "ms": {"rope_reset_apply": round(first_ms[0], 4),
                               "block_attention": round(first_ms[1], 4),
                               "kv_ring_append": round(first_ms[2], 4),
                               "convkv_compress": round(first_ms[3], 4)}},
        "step_breakdown_ms": {"rope_reset_apply": round(ms[0], 4),
                              "block_attention": round(ms[1], 4),
                              "kv_ring_append": round(ms[2], 4),
                              "convkv_compress": round(ms[3], 4),
                              "sum_of_events": round(ms_step_events, 4),
                              "step_p10_p50_p90": [round(float(x), 4) for x in step_pct]},
        "stream_gbs": {"rope_reset_apply": round(rope_bytes / (ms[0] * 1e-3) / 1e9, 1),
                       "kv_ring_append": round(append_bytes / (ms[2] * 1e-3) / 1e9, 1),
                       "convkv_compress": round(compress_bytes / (ms[3] * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": traffic,
                     "kernel": "k_attn (block attention)",
                     "algorithmic_per_launch": f"{attn_flop:.4e} flop = 4*Lq*Lk*D*H"},
        "cpu_baseline": None,
    }
    if dt == "fp8":
        # QK^T runs on bf16 matrix cores and PV on fp8 ones: half the flops at each rate
        mixed = 1.0 / (0.5 / PEAK["bf16"] + 0.5 / PEAK["fp8"])
        rec["attn_vs_peaks"] = {"bf16": round(attn_tflops / PEAK["bf16"], 4),
                                "fp8": round(attn_tflops / PEAK["fp8"], 4),
                                "qk_bf16_pv_fp8": round(attn_tflops / mixed, 4),
                                "qk_bf16_pv_fp8_peak_tflops": round(mixed, 1)}

    if args.cold:
        # the streaming calls with their inputs out of the last-level cache: a 512 MiB read
        # before each (no dirty lines, so no write-back overlaps the timed call; the
        # attention call between them keeps the step order)
        import microbench as MB
        flush = MB.read_flush(torch)
        cold = []
        for _ in range(args.cold):
            q, k, v = pool[i % len(pool)]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
            flush()
            e[0].record(stream)
            L.lact_rope_reset_apply(h, q, k, v, B, stream)
            e[1].record(stream)
            L.lact_block_attention(h, None, out, lse, stream)
            flush()
            e[2].record(stream)
            L.lact_kv_ring_append(h, k, v, B, stream)
            e[3].record(stream)
            flush()
            e[4].record(stream)
            L.lact_convkv_compress(h, d_wk, d_bk, d_wv, d_bv, stream)
            e[5].record(stream)
            cold.append(e)
            i += 1
        torch.cuda.synchronize()
        # mean over the steps: the compressor's slot count per step cycles (1, 2, 1, 2, 2)
        cm = np.mean(np.array([[e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3]),
                                e[4].elapsed_time(e[5])] for e in cold]), axis=0)
        rec["cold"] = {"steps": args.cold,
                       "mean_ms": {"rope_reset_apply": round(float(cm[0]), 4),
                                     "kv_ring_append": round(float(cm[1]), 4),
                                     "convkv_compress": round(float(cm[2]), 4)},
                       "gbs": {"rope_reset_apply": round(rope_bytes / (cm[0] * 1e-3) / 1e9, 1),
                               "kv_ring_append": round(append_bytes / (cm[1] * 1e-3) / 1e9, 1),
                               "convkv_compress": round(compress_bytes / (cm[2] * 1e-3) / 1e9, 1)}}
        del flush
    stream_bytes = {"rope_reset_apply": rope_bytes, "kv_ring_append": append_bytes,
                    "convkv_compress": compress_bytes}
    if not args.no_ceilings:
        rec["ceilings"], rec["stream"] = ceilings(stream_bytes, rec, w)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["parity"] = cpu_baseline(w, args, n_hist, B, Lq, Lk, cache, pool,
                                                          i, wk, bk, wv, bv)
    print(json.dumps(rec), flush=True)


def ceilings(stream_bytes, rec, w):
    """Measured ceilings (microbench/: a matrix-core loop per dtype, the bf16 loop fed from
    LDS, the softmax's exponentials beside MFMAs, and streaming copies with each streaming
    kernel's read:write mix and bytes, hot and with the last-level cache flushed), and each
    streaming kernel against the 8 TB/s peak and its copy ceiling."""
    import torch
    import microbench as MB
    r = w["ratio"]
    out = {"mfma_loop_tflops": {"bf16": round(MB.mfma_tflops(torch, False), 1),
                                "fp8": round(MB.mfma_tflops(torch, True), 1)},
           "mfma_lds_tflops": {"ds_read_b128": round(MB.mfma_lds_tflops(torch, False), 1),
                               "ds_read_b64_tr_b16": round(MB.mfma_lds_tflops(torch, True), 1)},
           "softmax_overlap_ms": MB.overlap_ms(torch),
           "read_only_gbs": {"bytes": 1 << 30,
                             "hot": round(MB.copy_gbs(torch, 1 << 30, 0, cold=False), 1),
                             "cold": round(MB.copy_gbs(torch, 1 << 30, 0, cold=True), 1)},
           "copy_gbs": {}}
    mix = {"rope_reset_apply": 1, "kv_ring_append": 1, "convkv_compress": r}
    ours = {}
    for name, total in stream_bytes.items():
        k = mix[name]
        write = int(total / (k + 1))
        read = k * write
        if k != 1 and k != 5:
            continue
        hot = MB.copy_gbs(torch, read, write, cold=False)
        cold = MB.copy_gbs(torch, read, write, cold=True)
        out["copy_gbs"][name] = {"read_bytes": read, "write_bytes": write, "mix": f"{k}:1",
                                 "hot": round(hot, 1), "cold": round(cold, 1)}
        got = rec["stream_gbs"][name]
        ent = {"gbs": got, "frac_hbm_peak": round(got / HBM_PEAK_GBS, 3),
               "frac_copy_hot": round(got / hot, 3)}
        if "cold" in rec:
            gc = rec["cold"]["gbs"][name]
            ent.update({"cold_gbs": gc, "cold_frac_hbm_peak": round(gc / HBM_PEAK_GBS, 3),
                        "cold_frac_copy_cold": round(gc / cold, 3)})
        ours[name] = ent
    return out, ours


def train_main(args, w):
    """Training form of the block-causal attention: one RoPE pass and one attention call
    over the whole sequence of blocks (no history), timed per call.  The attention work
    counted is the visible part only: block b of n_b frames sees the frames of blocks
    0..b, so flop = 4 D H T^2 sum_b n_b * (n_0 + .. + n_b)."""
    import torch
    import compressed_kv_causal_amd as L
    import synth
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    blocks = list(w["train_blocks"])
    n = sum(blocks)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ids = list(range(n))
    q, k, v = (torch.from_numpy(synth.frames(w, args.seed, t, ids).reshape(n * T, H, D))
               .to(torch.bfloat16).to(dev) for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V))
    cache = L.Cache(L.make_cfg(**w), device=dev)
    Lq = n * T
    out = torch.empty((Lq, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    h = cache.h

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        L.lact_rope_reset_apply(h, q, k, v, n, stream)
        if ev is not None:
            ev[1].record(stream)
        L.lact_block_attention(h, blocks, out, None, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(2)] for e in evs])
    ms = part.mean(axis=0)
    cum, pairs = 0, 0
    for nb in blocks:
        cum += nb
        pairs += nb * cum
    attn_flop = 4.0 * D * H * T * T * pairs
    attn_tflops = attn_flop / (ms[1] * 1e-3) / 1e12
    ms_per_step = wall * 1e3 / args.steps
    rec = {
        "metric": METRIC,
        "value": round(n / (ms_per_step * 1e-3), 2),
        "unit": "latent frames/s (training-form call: RoPE + block-causal attention over the whole sequence)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V)",
        "config": {"workload": args.workload, "heads": H, "head_dim": D, "tokens_per_frame": T,
                   "blocks_frames": blocks, "Lq": Lq, "Lk": Lq,
                   "visible_fraction": round(pairs / float(n * n), 4)},
        "attn_tflops": round(attn_tflops, 2),
        "step_breakdown_ms": {"rope_reset_apply": round(ms[0], 4), "block_attention": round(ms[1], 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK["bf16"],
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK["bf16"], 4), "traffic": None,
                     "kernel": "k_attn (block attention)",
                     "algorithmic_per_launch": f"{attn_flop:.4e} flop = 4*D*H*T^2*sum_b n_b*cum_b"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle.stream import OracleCache
        oc = OracleCache(w)
        qh, kh, vh = (t.float().cpu().numpy() for t in (q, k, v))
        rows = np.linspace(0, Lq - 1, args.cpu_rows).astype(np.int64)
        heads = np.repeat(np.arange(H, dtype=np.int32), len(rows))
        rr = np.tile(rows, H)
        threads = min(16, os.cpu_count() or 1)
        t1 = time.perf_counter()
        oc.attention(qh, kh, vh, block_frames=blocks, sel=(heads, rr), threads=threads)
        secs = time.perf_counter() - t1
        ends = np.cumsum(blocks) * T
        vis = ends[np.searchsorted(ends, rows, side="right")]
        frac = H * float(vis.sum()) / (H * T * T * pairs)
        full = secs / frac
        rec["cpu_baseline"] = {
            "value": round(n / full, 6), "unit": rec["unit"], "cores": threads, "kind": "oracle",
            "sample": (f"attention of all {H} heads x {len(rows)} query rows over their visible "
                       f"keys ({secs:.1f} s, double precision), extrapolated by visible key "
                       f"pairs (x{1 / frac:.0f}) to the whole call; RoPE not counted")}
    print(json.dumps(rec), flush=True)


def set_main(args, w):
    """A set of caches, one per (layer, denoising step), at model scale: per AR block every
    member runs RoPE + attention over its own history, then one append launch and one
    compress launch advance all members.  Timed per block."""
    import torch
    import compressed_kv_causal_amd as L
    import synth
    T, H, D, B = w["tokens"], w["heads"], w["head_dim"], w["block"]
    nm = w["members"]
    dt = {0: "f32", 1: "bf16", 2: "fp8"}[w["kv_dtype"]]
    io = torch.float32 if w["q_dtype"] == 0 else torch.bfloat16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = L.make_cfg(**w)
    set_bytes = L.lact_set_footprint(cfg, nm)
    solo_bytes = L.lact_cache_footprint(cfg)
    cache = L.Cache(cfg, device=dev, members=nm)
    # inputs resident in HBM: a pool of P seeded blocks; at AR step i member m takes pool
    # block (i + m) mod P.  K and V are laid out once, before timing, as nm + P - 1 blocks
    # (block j = pool block j mod P), so the stacked input of step i is the contiguous run
    # of nm blocks from block i mod P.
    pool = []
    for blk in range(args.pool_blocks):
        ids = list(range(blk * B, (blk + 1) * B))
        pool.append([torch.from_numpy(synth.frames(w, args.seed, t, ids).reshape(B * T, H, D))
                     .to(io).to(dev) for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V)])
    P = len(pool)
    nb = nm + P - 1
    k_run = torch.stack([pool[j % P][1] for j in range(nb)])
    v_run = torch.stack([pool[j % P][2] for j in range(nb)])
    wts = [synth.conv_weights(w, args.seed + m, synth.TENSOR_WK) + synth.conv_weights(w, args.seed + m, synth.TENSOR_WV)
           for m in range(nm)]
    d_wk, d_bk, d_wv, d_bv = (torch.from_numpy(np.stack([x[i] for x in wts])).to(dev) for i in range(4))
    Lq = B * T
    out = torch.empty((Lq, H, D), dtype=io, device=dev)
    stream = torch.cuda.current_stream()
    h = cache.h

    def stacked(i):
        o = i % P
        return (k_run[o: o + nm].reshape(nm * B * T, H, D), v_run[o: o + nm].reshape(nm * B * T, H, D))

    def advance(i):
        k_all, v_all = stacked(i)
        L.lact_kv_ring_append(h, k_all, v_all, B, stream)
        L.lact_convkv_compress(h, d_wk, d_bk, d_wv, d_bv, stream)

    def block(i, ev=None):
        o = i % P
        for m in range(nm):
            if ev is not None:
                ev[0][m].record(stream)
            L.lact_member_rope_reset_apply(h, m, pool[(o + m) % P][0], k_run[o + m], v_run[o + m],
                                           B, stream)
            if ev is not None:
                ev[1][m].record(stream)
            L.lact_member_block_attention(h, m, None, out, None, stream)
        if ev is not None:
            ev[2].record(stream)
        k_all, v_all = stacked(i)
        L.lact_kv_ring_append(h, k_all, v_all, B, stream)
        if ev is not None:
            ev[3].record(stream)
        L.lact_convkv_compress(h, d_wk, d_bk, d_wv, d_bv, stream)
        if ev is not None:
            ev[4].record(stream)

    # fill the memory with the batched append + compress alone (attention changes no state)
    i = 0
    while True:
        st = cache.state()
        if st["mem_len"] == w["mem_slots"] and st["win_len"] == w["window_frames"]:
            break
        advance(i)
        i += 1
    for _ in range(args.warmup):
        block(i)
        i += 1
    torch.cuda.synchronize()
    n_hist = cache.state()["mem_len"] + cache.state()["win_len"]
    Lk = (n_hist + B) * T
    E = lambda: torch.cuda.Event(enable_timing=True)
    evs = [[[E() for _ in range(nm)], [E() for _ in range(nm)], E(), E(), E()]
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        block(i, evs[s_])
        i += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # query tiles the fast attention pass handed to the exact pass (last member's call)
    n_flags = H * ((Lq + 255) // 256)
    flags = cache.buf[cache.layout.attn_flags:].view(torch.int32)[:n_flags]
    exact_tiles = int(flags.sum().item())
    rope_ms = np.mean([sum(e[0][m].elapsed_time(e[1][m]) for m in range(nm)) for e in evs])
    attn_ms = np.mean([sum(e[1][m].elapsed_time(e[0][m + 1]) for m in range(nm - 1)) +
                       e[1][nm - 1].elapsed_time(e[2]) for e in evs])
    app_ms = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    cmp_ms = np.mean([e[3].elapsed_time(e[4]) for e in evs])
    ms_block = wall * 1e3 / args.steps
    fe = T * H * D
    kvb = {"f32": 4, "bf16": 2, "fp8": 1}[dt]
    ob = 4 if w["q_dtype"] == 0 else 2
    sb = T * H * 4 if dt == "fp8" else 0
    append_bytes = nm * 2 * B * (fe * (ob + kvb) + sb)
    compress_bytes = nm * (B / w["ratio"]) * 2 * (fe * kvb + sb) * (w["ratio"] + 1)
    attn_flop = 4.0 * Lq * Lk * D * H * nm
    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    peak = PEAK["f32" if w["q_dtype"] == 0 else "bf16"]
    rec = {
        "metric": METRIC,
        "value": round(B / (ms_block * 1e-3), 3),
        "unit": f"latent frames/s (all {nm} caches of the set: layers x denoising steps, steady state)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_block, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if w["q_dtype"] == 0 else "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, N(0,0.2) conv weights per member)",
        "config": {"workload": args.workload, "members": nm, "kv_storage": dt, "heads": H,
                   "head_dim": D, "tokens_per_frame": T, "block_frames": B,
                   "window_frames": w["window_frames"], "mem_slots": w["mem_slots"],
                   "ratio": w["ratio"], "Lq": Lq, "Lk": Lk},
        "footprint_gib": {"set": round(set_bytes / 2 ** 30, 2),
                          "independent_caches": round(nm * solo_bytes / 2 ** 30, 2)},
        "attn_tflops": round(attn_tflops, 2),
        "attn_exact_pass_tiles_last_member": f"{exact_tiles}/{n_flags}",
        "step_breakdown_ms": {"rope_reset_apply_all_members": round(rope_ms, 3),
                              "block_attention_all_members": round(attn_ms, 3),
                              "kv_ring_append_batched": round(app_ms, 3),
                              "convkv_compress_batched": round(cmp_ms, 3),
                              "per_member": round(ms_block / nm, 4)},
        "stream_gbs": {"kv_ring_append_batched": round(append_bytes / (app_ms * 1e-3) / 1e9, 1),
                       "convkv_compress_batched": round(compress_bytes / (cmp_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4), "traffic": None,
                     "kernel": "k_attn (block attention, all members)",
                     "algorithmic_per_launch": f"{attn_flop / nm:.4e} flop = 4*Lq*Lk*D*H"},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _tiny_full():
    """The oracle on the tiny workload, whole: 27 history blocks and 20 AR steps, every
    step's attention on every row, append and compress.  Returns (seconds, steps)."""
    import synth
    from oracle.stream import OracleCache
    w = synth.workload("tiny_f32")
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    wk, bk = synth.conv_weights(w, 0, synth.TENSOR_WK)
    wv, bv = synth.conv_weights(w, 0, synth.TENSOR_WV)
    oc = OracleCache(w)
    steps = w["history_blocks"] + w["steps"]
    t0 = time.perf_counter()
    f = 0
    for _ in range(steps):
        ids = list(range(f, f + 2))
        q, k, v = (synth.frames(w, 0, t, ids).reshape(2 * T, H, D)
                   for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V))
        oc.attention(q, k, v, threads=1)
        oc.append(k.reshape(2, -1), v.reshape(2, -1))
        oc.compress(wk, bk, wv, bv)
        f += 2
    return time.perf_counter() - t0, steps


def cpu_baseline(w, args, n_hist, B, Lq, Lk, cache, pool, next_step, wk, bk, wv, bv):
    """The oracle, as it stands, on a bounded sample of the same steady-state step, every
    part of the step timed (the plan of the CPU baseline: full where it is small,
    row-sampled attention extrapolated and labelled as such):
      attention   all heads x args.cpu_rows query rows over the full key set, all cores
                  and (on a sixteenth of that sample) one thread; extrapolated by rows;
      RoPE        the oracle's rotation of the step's history keys and block Q, K (timed
                  on the block's Q, scaled by the frame count);
      append      the oracle's storage of the block's K and V (bf16 rounding or FP8 rows);
      compress    the oracle's compression of one group of 5 frames (K and V), times the
                  groups of an average step (B / r);
      bookkeeping 1000 steps of the oracle's planner, per step;
    plus, reported beside, the tiny workload run whole and the 80 -> 16 memory build."""
    import oracle as O
    import synth
    from oracle.bookkeeping import Bookkeeping
    from oracle.stream import OracleCache
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    io_bf16 = w["q_dtype"] == 1
    import torch

    # Rebuild the oracle state of the GPU cache at this step (its frames come from the pool:
    # block n uses pool block n mod len(pool)).
    st = cache.state()
    oc = OracleCache(w)
    if w.get("ref_frames", 0):
        # the reference segment as the device holds it (converted to the input dtype)
        io = torch.bfloat16 if io_bf16 else torch.float32
        kr, vr = (torch.from_numpy(x).to(io).float().numpy() for x in synth.ref_frames(w, args.seed))
        oc.set_ref(kr, vr)
    np_pool = [[t.float().cpu().numpy().reshape(B, -1) for t in trip] for trip in pool]
    t_setup = time.perf_counter()
    oc.bk.F, oc.bk.G = st["F"], st["G"] - st["mem_len"]
    # frames still needed: the groups in memory and the window
    E = st["E"]
    need = list(range(w["ratio"] * oc.bk.G, st["F"]))
    for f in need:
        blk = f // B
        k = np_pool[blk % len(pool)][1][f % B]
        v = np_pool[blk % len(pool)][2][f % B]
        oc.raw[f] = (oc._store(k), oc._store(v))
    oc.bk.F = st["F"]
    r = w["ratio"]
    group_s = []
    while len(group_s) < st["mem_len"]:
        # compress the groups present in memory (each from its own r frames), timed per group
        g = oc.bk.G
        tg = time.perf_counter()
        xk = np.stack([oc._f32(oc.raw[r * g + k][0]) for k in range(r)])
        xv = np.stack([oc._f32(oc.raw[r * g + k][1]) for k in range(r)])
        oc.mem[g % w["mem_slots"]] = (g, oc._store(O.compress_chain_f32(xk, wk, bk)),
                                      oc._store(O.compress_chain_f32(xv, wv, bv)))
        group_s.append(time.perf_counter() - tg)
        oc.bk.G += 1
    setup_s = time.perf_counter() - t_setup
    assert oc.bk.E == E and len(oc.keys(0)) == n_hist
    q, k, v = (np_pool[(next_step) % len(pool)][j].reshape(B * T, H, D) for j in range(3))

    # attention, row-sampled
    rows = np.linspace(0, Lq - 1, args.cpu_rows).astype(np.int64)
    heads = np.repeat(np.arange(H, dtype=np.int32), len(rows))
    rr = np.tile(rows, H)
    threads = min(16, os.cpu_count() or 1)
    t0 = time.perf_counter()
    O_ref = oc.attention(q, k, v, sel=(heads, rr), threads=threads)[0]
    secs = time.perf_counter() - t0
    frac = len(rr) / float(H * Lq)
    attn_full = secs / frac
    few = np.arange(0, len(rr), 16)          # one thread on the same rows of every 16th head
    t1 = time.perf_counter()
    oc.attention(q, k, v, sel=(heads[few], rr[few]), threads=1)
    secs1 = time.perf_counter() - t1
    attn_full1 = secs1 / (len(few) / float(H * Lq))

    # RoPE: the block's Q (B frames) rotated at its reset positions, scaled to the step's
    # n_hist + 2 B rotated frames
    t_pos = np.repeat(np.arange(B, dtype=np.int32) + n_hist, T)
    u_pos = np.tile(np.arange(T, dtype=np.int32), B)
    t2 = time.perf_counter()
    O.rope_rotate(q, t_pos, u_pos, w["rope_mode"], w["rope_split"], T, w["grid_w"], w["rope_theta"])
    rope_s = (time.perf_counter() - t2) * (n_hist + 2 * B) / B
    # append: storing the block's K and V
    t3 = time.perf_counter()
    for i in range(B):
        oc._store(k.reshape(B, -1)[i])
        oc._store(v.reshape(B, -1)[i])
    append_s = time.perf_counter() - t3
    compress_s = float(np.mean(group_s)) * B / r
    # bookkeeping: the planner over 1000 steps
    bkp = Bookkeeping(w["window_frames"], w["mem_slots"], r, B, w.get("ref_frames", 0))
    t4 = time.perf_counter()
    for _ in range(1000):
        bkp.keys(B)
        bkp.append(B)
        bkp.compress()
    book_s = (time.perf_counter() - t4) / 1000
    tiny_s, tiny_steps = _tiny_full()
    step_s = attn_full + rope_s + append_s + compress_s + book_s
    step_s1 = attn_full1 + rope_s + append_s + compress_s + book_s

    # The timed configuration's own output for that step (RoPE + attention on the device,
    # after the timed region) on the same rows, against the oracle's.
    cache.rope_reset_apply(*pool[next_step % len(pool)])
    got = cache.block_attention()
    torch.cuda.synchronize()
    got = got.float().cpu().numpy()[rr, heads, :].astype(np.float64)
    err = float(np.linalg.norm(got - O_ref) / np.linalg.norm(O_ref))
    bar = {0: 1e-5, 1: 1e-2, 2: 5e-2}[w["kv_dtype"]]
    parity = {"rel_l2": float(f"{err:.3e}"), "bar": bar, "ok": err <= bar,
              "rows": f"all {H} heads x {len(rows)} query rows of the next steady-state step, "
                      "attention output against the oracle"}
    return {"value": round(B / step_s, 6), "unit": "latent frames/s (one layer, one diffusion step)",
            "cores": threads, "kind": "oracle", "cpu_model": _cpu_model(),
            "value_1_thread": round(B / step_s1, 6),
            "step_seconds": {"attention_extrapolated": round(attn_full, 2),
                             "attention_extrapolated_1_thread": round(attn_full1, 2),
                             "rope": round(rope_s, 3), "append": round(append_s, 3),
                             "compress": round(compress_s, 3), "bookkeeping": round(book_s, 6)},
            "tiny_full": {"steps": tiny_steps, "seconds": round(tiny_s, 2),
                          "steps_per_s_1_thread": round(tiny_steps / tiny_s, 2)},
            "memory_build_80_to_16_seconds": round(float(np.sum(group_s)), 2),
            "sample": (f"attention of all {H} heads x {len(rows)} query rows over Lk={Lk} keys "
                       f"({secs:.1f} s on {threads} threads, double precision), extrapolated "
                       f"x{1 / frac:.0f} by rows to the full step; one thread on a sixteenth of "
                       f"those rows ({secs1:.1f} s); RoPE ({rope_s:.2f} s), append "
                       f"({append_s:.2f} s), compress ({compress_s:.2f} s for {B / r:.1f} groups) "
                       "and bookkeeping timed on the oracle's single-threaded routines and "
                       "added; memory of 16 slots built in "
                       f"{setup_s:.1f} s before timing")}, parity


if __name__ == "__main__":
    main()
