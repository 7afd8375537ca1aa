"""CPU oracle of the ConvKV-memory block-causal attention step.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg are the only users.  Nothing in the GPU package imports it, and it
imports nothing from the GPU package.  The numerics live in ``lact_oracle.c`` (plain C,
double precision except the storage definitions); this module marshals numpy arrays and
holds the bookkeeping (``bookkeeping.py``) and the streaming driver (``stream.py``).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblact_oracle.so")
_lib = None

_f = ctypes.POINTER(ctypes.c_float)
_d = ctypes.POINTER(ctypes.c_double)
_u8 = ctypes.POINTER(ctypes.c_uint8)
_u16 = ctypes.POINTER(ctypes.c_uint16)
_i32 = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.POINTER(ctypes.c_int64)


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("Lq", ctypes.c_int64), ("Lhist", ctypes.c_int64),
        ("q", _f), ("q_scale", _f),
        ("k_hist", _f), ("k_hist_scale", _f),
        ("v_hist", _f), ("v_hist_scale", _f),
        ("k_cur", _f), ("k_cur_scale", _f),
        ("v_cur", _f), ("v_cur_scale", _f),
        ("hist_t", _i32), ("hist_u", _i32),
        ("cur_t", _i32), ("cur_u", _i32),
        ("rope_mode", ctypes.c_int32), ("rope_split", ctypes.c_int32 * 3),
        ("T", ctypes.c_int32), ("grid_w", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("n_blocks", ctypes.c_int32), ("block_start", _i64),
        ("n_sel", ctypes.c_int64), ("sel_head", _i32), ("sel_row", _i64),
        ("form", ctypes.c_int32), ("threads", ctypes.c_int32),
        ("out", _d), ("lse", _d), ("rms", _d),
    ]


def build(verbose=False):
    """Compile liblact_oracle.so with gcc (plain C; no HIP)."""
    import subprocess
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           os.path.join(_HERE, "lact_oracle.c"), "-o", LIB_PATH, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.lacto_bf16_value.argtypes = [ctypes.c_uint16]
        L.lacto_bf16_value.restype = ctypes.c_double
        L.lacto_bf16_encode.argtypes = [ctypes.c_float]
        L.lacto_bf16_encode.restype = ctypes.c_uint16
        L.lacto_bf16_encode_array.argtypes = [_f, _u16, ctypes.c_int64]
        L.lacto_e4m3_value.argtypes = [ctypes.c_uint8]
        L.lacto_e4m3_value.restype = ctypes.c_double
        L.lacto_e4m3_encode.argtypes = [ctypes.c_float]
        L.lacto_e4m3_encode.restype = ctypes.c_uint8
        L.lacto_quant_e4m3_rows.argtypes = [_f, ctypes.c_int64, ctypes.c_int32, _u8, _f]
        L.lacto_e4m3_dequant_f32.argtypes = [_u8, _f, ctypes.c_int64, ctypes.c_int32, _f]
        L.lacto_compress_chain_f32.argtypes = [_f, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                               _f, _f, _f]
        L.lacto_compress_exact.argtypes = [_f, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                           _f, _f, _d]
        L.lacto_rope_rotate.argtypes = [_d, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _i32,
                                        _i32, ctypes.c_int32, _i32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_double]
        L.lacto_attention.argtypes = [ctypes.POINTER(AttnArgs)]
        L.lacto_attention.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a, ptype):
    return a.ctypes.data_as(ptype) if a is not None else None


# ---- codecs --------------------------------------------------------------------------

def bf16_encode(x):
    """Nearest bf16 code (round to nearest, ties to even) of every float32 in x."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().lacto_bf16_encode_array(_p(x, _f), _p(out, _u16), x.size)
    return out


def bf16_value(codes):
    """Exact values of bf16 codes as float32 (a bf16 value is a float32 value)."""
    codes = _c(codes, np.uint16)
    return (codes.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x):
    return bf16_value(bf16_encode(x))


def e4m3_value(code):
    return lib().lacto_e4m3_value(int(code))


def e4m3_encode(x):
    return lib().lacto_e4m3_encode(float(x))


_E4M3_TABLE = None


def e4m3_table():
    """float64 value of each of the 256 codes (NaN for 0x7F, 0xFF)."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = np.array([lib().lacto_e4m3_value(c) for c in range(256)])
    return _E4M3_TABLE


def quant_e4m3_rows(x, D):
    """x [..., D] float32 -> (codes uint8 same shape, scales float32 [...])."""
    x = _c(x, np.float32)
    rows = x.size // D
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    lib().lacto_quant_e4m3_rows(_p(x, _f), rows, D, _p(codes, _u8), _p(scales, _f))
    return codes, scales


def e4m3_dequant_f32(codes, scales, D):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    out = np.empty(codes.shape, dtype=np.float32)
    lib().lacto_e4m3_dequant_f32(_p(codes, _u8), _p(scales, _f), codes.size // D, D, _p(out, _f))
    return out


def e4m3_stored_value(codes, scales, D):
    """Exact stored value code * scale in float64 (what attention sees)."""
    t = e4m3_table()
    return t[codes] * scales.astype(np.float64)[..., None]


# ---- compression -----------------------------------------------------------------------

def compress_chain_f32(x, w, b):
    """x [r][T*C] float32 (stored values), w [C][r], b [C] -> [T*C] float32 via the f32 fma chain."""
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    b = _c(b, np.float32)
    r, TC = x.shape
    C = w.shape[0]
    out = np.empty(TC, dtype=np.float32)
    lib().lacto_compress_chain_f32(_p(x, _f), r, TC, C, _p(w, _f), _p(b, _f), _p(out, _f))
    return out


def compress_exact(x, w, b):
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    b = _c(b, np.float32)
    r, TC = x.shape
    C = w.shape[0]
    out = np.empty(TC, dtype=np.float64)
    lib().lacto_compress_exact(_p(x, _f), r, TC, C, _p(w, _f), _p(b, _f), _p(out, _d))
    return out


# ---- RoPE --------------------------------------------------------------------------------

def rope_rotate(x, t, u, mode, split, T, grid_w, theta=10000.0):
    """x [n][H][D] -> rotated copy (float64); token i at (t[i], u[i])."""
    x = np.array(x, dtype=np.float64, order="C", copy=True)
    n, H, D = x.shape
    t = _c(t, np.int32)
    u = _c(u, np.int32)
    sp = _c(list(split) + [0] * (3 - len(split)), np.int32)
    lib().lacto_rope_rotate(_p(x, _d), n, H, D, _p(t, _i32), _p(u, _i32), mode, _p(sp, _i32), T,
                            grid_w, theta)
    return x


# ---- attention ---------------------------------------------------------------------------

def attention(q, k_cur, v_cur, k_hist, v_hist, hist_t, hist_u, cur_t, cur_u, block_frames,
              T, rope_mode, rope_split, grid_w, theta=10000.0, sel=None, form=1,
              q_scale=None, k_cur_scale=None, v_cur_scale=None, k_hist_scale=None,
              v_hist_scale=None, threads=None, want_rms=False):
    """Oracle attention of the current queries over [history | current].

    q, k_cur, v_cur: [Lq][H][D]; k_hist, v_hist: [Lhist][H][D] (float32 stored values, or
    e4m3 code values with the *_scale arrays [L][H]).  block_frames: query block sizes in
    frames.  sel: (heads, rows) int arrays of outputs to compute (default all), which are
    sorted by head here.  Returns (O [n_sel][D] float64, LSE [n_sel] float64, heads, rows)
    in the sorted order, and with want_rms also RMS [n_sel] = sqrt(sum_j w_j^2 |v_j|^2)
    (w the softmax weights of the row).
    """
    q = _c(q, np.float32)
    Lq, H, D = q.shape
    k_cur = _c(k_cur, np.float32)
    v_cur = _c(v_cur, np.float32)
    Lhist = 0 if k_hist is None else k_hist.shape[0]
    if Lhist == 0:
        k_hist = np.zeros((1, H, D), np.float32)
        v_hist = np.zeros((1, H, D), np.float32)
        hist_t = np.zeros(1, np.int32)
        hist_u = np.zeros(1, np.int32)
    k_hist = _c(k_hist, np.float32)
    v_hist = _c(v_hist, np.float32)
    hist_t = _c(hist_t, np.int32)
    hist_u = _c(hist_u, np.int32)
    cur_t = _c(cur_t, np.int32)
    cur_u = _c(cur_u, np.int32)
    starts = np.concatenate([[0], np.cumsum(np.asarray(block_frames, np.int64) * T)]).astype(np.int64)
    if starts[-1] != Lq:
        raise ValueError("block_frames do not sum to the query length")
    if sel is None:
        heads = np.repeat(np.arange(H, dtype=np.int32), Lq)
        rows = np.tile(np.arange(Lq, dtype=np.int64), H)
    else:
        heads = np.asarray(sel[0], np.int32)
        rows = np.asarray(sel[1], np.int64)
        order = np.lexsort((rows, heads))
        heads = _c(heads[order], np.int32)
        rows = _c(rows[order], np.int64)
    n_sel = heads.size
    out = np.zeros((n_sel, D), np.float64)
    lse = np.zeros(n_sel, np.float64)
    rms = np.zeros(n_sel, np.float64) if want_rms else None
    keep = []

    def sc(a):
        if a is None:
            return None
        a = _c(a, np.float32)
        keep.append(a)
        return _p(a, _f)

    if Lhist == 0:
        k_hist_scale = v_hist_scale = None
    args = AttnArgs()
    args.H, args.D, args.Lq, args.Lhist = H, D, Lq, Lhist
    args.q, args.q_scale = _p(q, _f), sc(q_scale)
    args.k_hist, args.k_hist_scale = _p(k_hist, _f), sc(k_hist_scale)
    args.v_hist, args.v_hist_scale = _p(v_hist, _f), sc(v_hist_scale)
    args.k_cur, args.k_cur_scale = _p(k_cur, _f), sc(k_cur_scale)
    args.v_cur, args.v_cur_scale = _p(v_cur, _f), sc(v_cur_scale)
    args.hist_t, args.hist_u = _p(hist_t, _i32), _p(hist_u, _i32)
    args.cur_t, args.cur_u = _p(cur_t, _i32), _p(cur_u, _i32)
    args.rope_mode = rope_mode
    sp = list(rope_split) + [0] * (3 - len(rope_split))
    args.rope_split = (ctypes.c_int32 * 3)(*sp)
    args.T, args.grid_w, args.rope_theta = T, grid_w, theta
    args.n_blocks = len(block_frames)
    args.block_start = _p(starts, _i64)
    args.n_sel = n_sel
    args.sel_head, args.sel_row = _p(heads, _i32), _p(rows, _i64)
    args.form = form
    args.threads = threads if threads else min(16, os.cpu_count() or 1)
    args.out, args.lse, args.rms = _p(out, _d), _p(lse, _d), _p(rms, _d)
    rc = lib().lacto_attention(ctypes.byref(args))
    if rc != 0:
        raise ValueError(f"lacto_attention failed with {rc}")
    if want_rms:
        return out, lse, heads, rows, rms
    return out, lse, heads, rows
