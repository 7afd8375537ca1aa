"""Measurement kernels for bench.py (microbench/mb.hip): a matrix-core loop for bf16 and
fp8 and streaming copies with the step's read:write mixes, timed with HIP events on the
stream they run on.  They give the measured ceilings the step's kernels are read against
beside the published peaks.  Not part of the method's path; only bench.py uses them.
"""
import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmb.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
_lib = None


def build(verbose=False):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "mb.hip"), "-o", LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on mb.hip:\n{r.stderr}")
    os.replace(LIB_PATH + ".tmp", LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.mb_mfma_loop.argtypes = [i32, i32, i32, vp, vp, vp]
        L.mb_copy.argtypes = [vp, vp, i64, vp]
        L.mb_copy5.argtypes = [vp, vp, i64, vp]
        L.mb_read.argtypes = [vp, i64, vp, vp]
        L.mb_mfma_lds.argtypes = [i32, i32, i32, vp, vp, vp]
        L.mb_overlap.argtypes = [i32, i32, i32, vp, vp, vp]
        for f in (L.mb_mfma_loop, L.mb_copy, L.mb_copy5, L.mb_read, L.mb_mfma_lds, L.mb_overlap):
            f.restype = i32
        _lib = L
    return _lib


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} launch failed (hipError {rc})")


def read_flush(torch, nbytes=512 << 20):
    """A callable that evicts the last-level cache by reading nbytes once (mb_read on the
    current stream).  A read leaves no dirty lines behind, so no write-back of the flush
    overlaps the call timed after it, as it would after a fill."""
    dev = torch.device("cuda")
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    bp, sp = ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(sink.data_ptr())

    def flush():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        _check(lib().mb_read(bp, nbytes, sp, s), "mb_read")
    flush.buffers = (buf, sink)   # keeps the buffers alive with the callable
    return flush


def _timed(torch, fn, reps, flush=None):
    """Median over reps of fn() timed with events on the current stream; flush() (a
    last-level cache flush) runs before each rep, outside the timed interval."""
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    return times[len(times) // 2]


def mfma_tflops(torch, fp8, cus=256, iters=4096, reps=5):
    """Dense matrix-core rate of back-to-back MFMAs, 2 waves per SIMD on every CU."""
    dev = torch.device("cuda")
    seed = torch.rand(64, device=dev)
    sink = torch.zeros(cus, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        _check(lib().mb_mfma_loop(int(fp8), cus, iters, ctypes.c_void_p(seed.data_ptr()),
                                  ctypes.c_void_p(sink.data_ptr()), s), "mb_mfma_loop")
    run()
    ms = _timed(torch, run, reps)
    flop_per = 2.0 * 32 * 32 * (64 if fp8 else 16)
    flops = cus * 8 * iters * 4 * flop_per
    return flops / (ms * 1e-3) / 1e12


def mfma_lds_tflops(torch, transposed, cus=256, iters=512, reps=5):
    """bf16 MFMA rate with every A operand read from LDS (1 KiB per MFMA), 2 waves per SIMD:
    ds_read_b128 fragments, or (transposed) pairs of ds_read_b64_tr_b16."""
    dev = torch.device("cuda")
    seed = torch.rand(64, device=dev)
    sink = torch.zeros(cus, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        _check(lib().mb_mfma_lds(int(transposed), cus, iters, ctypes.c_void_p(seed.data_ptr()),
                                 ctypes.c_void_p(sink.data_ptr()), s), "mb_mfma_lds")
    run()
    ms = _timed(torch, run, reps)
    flops = cus * 8 * iters * 16 * 2.0 * 32 * 32 * 16
    return flops / (ms * 1e-3) / 1e12


def overlap_ms(torch, cus=256, iters=4096, reps=5):
    """Times (ms) of an MFMA stream and of the softmax's exponentials with their sums (one
    exp2 and one add per MFMA): each alone, in two waves sharing a SIMD, and interleaved in
    one wave."""
    dev = torch.device("cuda")
    seed = torch.rand(64, device=dev)
    sink = torch.zeros(cus, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    for mode, name in enumerate(("mfma_alone", "exp_alone", "two_waves", "one_wave")):
        def run():
            _check(lib().mb_overlap(mode, cus, iters, ctypes.c_void_p(seed.data_ptr()),
                                    ctypes.c_void_p(sink.data_ptr()), s), "mb_overlap")
        run()
        out[name] = round(_timed(torch, run, reps), 4)
    return out


def copy_gbs(torch, read_bytes, write_bytes, reps=7, cold=False):
    """GB/s (bytes read + written per second) of a streaming kernel with the given read and
    write sizes: 1:1 (read == write), 5:1 (read == 5 * write) or read-only (write == 0).
    cold: a 512 MiB read before each rep evicts the inputs from the last-level cache."""
    dev = torch.device("cuda")
    five = write_bytes > 0 and read_bytes == 5 * write_bytes
    ronly = write_bytes == 0
    assert five or ronly or read_bytes == write_bytes
    n = ((read_bytes if ronly else write_bytes) // 16) * 16
    src = torch.empty(5 * n if five else n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(1024 * 4 if ronly else n, dtype=torch.uint8, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flush = read_flush(torch) if cold else None
    sp, dp = ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr())

    def run():
        if ronly:
            _check(lib().mb_read(sp, n, dp, s), "mb_read")
        else:
            _check((lib().mb_copy5 if five else lib().mb_copy)(sp, dp, n, s), "mb_copy")
    run()
    ms = _timed(torch, run, reps, flush=flush)
    total = n if ronly else (5 * n if five else n) + n
    del src, dst, flush
    return total / (ms * 1e-3) / 1e9
