"""Seeded synthetic inputs (random numbers only; none of the method's arithmetic).

Shared by the tests, ``bench.py`` and the callers of the oracle, so that the GPU path and
the oracle see the same inputs.  The generator itself is ``synth.c`` (counter-based
SplitMix64 + Box-Muller); this module loads it with ctypes and describes the workloads.

The workloads stand in for the pages' HDTF/EMTD videos at 512x512 and 720x416, which are
not available: Q/K/V ~ N(0, 1), conv weights ~ N(0, 0.2) (standard deviation), bias 0, and
for the FP8 KV workload each element independently x8 with probability 0.01.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

# Stream ids: one counter stream per (seed, tensor, frame).
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_WK, TENSOR_WV = 1, 2, 3, 4, 5
TENSOR_REF_K, TENSOR_REF_V = 6, 7   # the reference segment's K and V
TENSOR_SAMPLE = 8            # uniform stream used to pick sampled query rows
OUTLIER_BASE = 16            # outlier mask of tensor t uses stream OUTLIER_BASE + t

_lib = None


def build(verbose=False):
    """Compile libsynth.so with gcc (plain C, no GPU)."""
    import subprocess
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           os.path.join(_HERE, "synth.c"), "-o", LIB_PATH, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        fp = ctypes.POINTER(ctypes.c_float)
        L.synth_normal.argtypes = [u64, u32, u64, u64, u64, ctypes.c_double, fp, i32]
        L.synth_outliers.argtypes = [u64, u32, u64, u64, u64, ctypes.c_double, ctypes.c_float, fp,
                                     i32]
        L.synth_uniform.argtypes = [u64, u32, u64, u64, u64, fp, i32]
        L.synth_stream_key.argtypes = [u64, u32, u64]
        L.synth_stream_key.restype = u64
        _lib = L
    return _lib


def _threads():
    return min(16, os.cpu_count() or 1)


def normal(seed, tensor, frame, count, stddev=1.0, first=0):
    out = np.empty(count, dtype=np.float32)
    lib().synth_normal(seed, tensor, frame, first, count, stddev,
                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _threads())
    return out


def uniform(seed, tensor, frame, count, first=0):
    out = np.empty(count, dtype=np.float32)
    lib().synth_uniform(seed, tensor, frame, first, count,
                        out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _threads())
    return out


def apply_outliers(arr, seed, tensor, frame, prob=0.01, factor=8.0):
    """In place: each element x8 with probability prob (stream OUTLIER_BASE + tensor)."""
    assert arr.dtype == np.float32 and arr.flags.c_contiguous
    lib().synth_outliers(seed, OUTLIER_BASE + tensor, frame, 0, arr.size, prob, factor,
                         arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _threads())
    return arr


# ---------------------------------------------------------------------------------------
# Workloads (sizes and schedules only).
# ---------------------------------------------------------------------------------------

F32, BF16, FP8 = 0, 1, 2

WORKLOADS = {
    # 2 heads x 64, 4x4 grid, blocks of 2, window 4, memory 10 at 5:1; 1D RoPE; f32.
    "tiny_f32": dict(heads=2, head_dim=64, grid_h=4, grid_w=4, window_frames=4, mem_slots=10,
                     ratio=5, max_block_frames=2, kv_dtype=F32, q_dtype=F32, rope_mode=1,
                     rope_split=(64, 0, 0), rope_theta=10000.0,
                     first_block=2, block=2, history_blocks=27, steps=20, pool_blocks=0),
    # 512x512 video -> 32x32 patch grid; 40 heads x 128; blocks of 8, window 8, memory 16.
    "s512_bf16": dict(heads=40, head_dim=128, grid_h=32, grid_w=32, window_frames=8,
                      mem_slots=16, ratio=5, max_block_frames=8, kv_dtype=BF16, q_dtype=BF16,
                      rope_mode=3, rope_split=(44, 42, 42), rope_theta=10000.0,
                      first_block=8, block=8, history_blocks=11, steps=1, pool_blocks=7),
    # 720x416 video -> 26 rows x 45 columns = 1170 tokens; first block 6 frames, then 8.
    "s720_bf16": dict(heads=40, head_dim=128, grid_h=26, grid_w=45, window_frames=8,
                      mem_slots=16, ratio=5, max_block_frames=8, kv_dtype=BF16, q_dtype=BF16,
                      rope_mode=3, rope_split=(44, 42, 42), rope_theta=10000.0,
                      first_block=6, block=8, history_blocks=11, steps=1, pool_blocks=7),
    # 512 shapes, 1000 consecutive AR steps (frame pool of 7 blocks, coprime with r = 5).
    "long_run": dict(heads=40, head_dim=128, grid_h=32, grid_w=32, window_frames=8,
                     mem_slots=16, ratio=5, max_block_frames=8, kv_dtype=BF16, q_dtype=BF16,
                     rope_mode=3, rope_split=(44, 42, 42), rope_theta=10000.0,
                     first_block=8, block=8, history_blocks=0, steps=1000, pool_blocks=7),
    # 512 shapes, K/V stored e4m3 + per-(token, head) f32 scale, Q bf16, 1% outliers x8.
    "fp8_kv": dict(heads=40, head_dim=128, grid_h=32, grid_w=32, window_frames=8,
                   mem_slots=16, ratio=5, max_block_frames=8, kv_dtype=FP8, q_dtype=BF16,
                   rope_mode=3, rope_split=(44, 42, 42), rope_theta=10000.0,
                   first_block=8, block=8, history_blocks=11, steps=1, pool_blocks=7,
                   outliers=True),
    # Training form of the block-causal attention (walkthrough "Neighbor Forcing"): one
    # call over 46 frames in blocks of 6, 8, 8, 8, 8, 8, no history, block-causal mask.
    "train_s512": dict(heads=40, head_dim=128, grid_h=32, grid_w=32, window_frames=8,
                       mem_slots=16, ratio=5, max_block_frames=46, kv_dtype=BF16, q_dtype=BF16,
                       rope_mode=3, rope_split=(44, 42, 42), rope_theta=10000.0,
                       first_block=6, block=8, history_blocks=0, steps=1, pool_blocks=7,
                       train_blocks=(6, 8, 8, 8, 8, 8)),
}

# With the reference segment (the reference image's part of the context): 2 frames.
WORKLOADS["tiny_ref"] = dict(WORKLOADS["tiny_f32"], ref_frames=2)
WORKLOADS["s512_ref2"] = dict(WORKLOADS["s512_bf16"], ref_frames=2)

# Model scale: one cache per (layer, denoising step), 40 layers (the 40 x 128-channel heads
# are those of the 14B Wan2.1 DiT the model is initialised from) x 3 distilled steps.
WORKLOADS["model_s512"] = dict(WORKLOADS["s512_bf16"], members=120)
WORKLOADS["model_s512_fp8"] = dict(WORKLOADS["fp8_kv"], members=120)

# The memory-block / current-block grid of the model card's ablation table (Table 5):
# window ("memory block") W and block B in frames, 512x512 shapes, memory 16 slots at 5:1.
for _w, _b in ((6, 6), (8, 8), (6, 8)):
    WORKLOADS[f"grid_w{_w}_b{_b}"] = dict(WORKLOADS["s512_bf16"], window_frames=_w,
                                          max_block_frames=_b, first_block=_b, block=_b)

CFG_KEYS = ("heads", "head_dim", "grid_h", "grid_w", "window_frames", "mem_slots", "ratio",
            "max_block_frames", "kv_dtype", "q_dtype", "rope_mode", "rope_split", "rope_theta",
            "ref_frames")


def workload(name, **overrides):
    w = dict(WORKLOADS[name])
    w.update(overrides)
    w["name"] = name
    w["tokens"] = w["grid_h"] * w["grid_w"]
    w["channels"] = w["heads"] * w["head_dim"]
    return w


def block_sizes(w, n_blocks):
    """Frames per AR block: the first block, then the steady block size."""
    return [w["first_block"] if i == 0 else w["block"] for i in range(n_blocks)]


def source_frame(w, f):
    """Generator frame id for absolute frame f: a pool of pool_blocks blocks if set."""
    pool = w.get("pool_blocks", 0) * w["block"]
    return f % pool if pool else f


def frames(w, seed, tensor, frame_ids):
    """[len(frame_ids), T*C] float32 of N(0, 1) (x8 outliers where the workload has them)."""
    n = w["tokens"] * w["channels"]
    out = np.empty((len(frame_ids), n), dtype=np.float32)
    for i, f in enumerate(frame_ids):
        sf = source_frame(w, f)
        out[i] = normal(seed, tensor, sf, n)
        if w.get("outliers"):
            apply_outliers(out[i], seed, tensor, sf)
    return out


def ref_frames(w, seed):
    """The reference segment's K and V: [ref_frames][T*C] float32 each, N(0, 1) (x8 outliers
    where the workload has them), from their own streams."""
    ids = list(range(w.get("ref_frames", 0)))
    n = w["tokens"] * w["channels"]
    out = []
    for tensor in (TENSOR_REF_K, TENSOR_REF_V):
        x = np.empty((len(ids), n), dtype=np.float32)
        for i in ids:
            x[i] = normal(seed, tensor, i, n)
            if w.get("outliers"):
                apply_outliers(x[i], seed, tensor, i)
        out.append(x)
    return out[0], out[1]


def conv_weights(w, seed, tensor):
    """[C][r] float32 ~ N(0, 0.2) (standard deviation 0.2) and a zero bias [C]."""
    C, r = w["channels"], w["ratio"]
    wt = normal(seed, tensor, 0, C * r, stddev=0.2).reshape(C, r)
    return wt, np.zeros(C, dtype=np.float32)
