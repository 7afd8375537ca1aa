"""ConvKV-memory block-causal attention for MI355X (gfx950): Python binding of liblact.so.

Argument marshalling only.  Every step of the path runs in the HIP kernels behind the C
ABI of ``include/lact.h``; torch provides device memory and streams.  If liblact.so is
missing, every call raises -- there is no fallback path.

The functions carry the C names: ``lact_rope_reset_apply``, ``lact_block_attention``,
``lact_kv_ring_append``, ``lact_convkv_compress``, their ``lact_member_*`` forms for cache
sets, and the sizing, lifetime, inspection and planner calls.  ``Cache`` bundles one cache
buffer (or a set of ``members`` caches in one buffer) and its handle for convenience.
"""
import ctypes
import os

import torch  # loads the HIP runtime first; liblact.so binds to the same one

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblact.so")

LACT_F32, LACT_BF16, LACT_FP8_E4M3 = 0, 1, 2
LACT_MAX_KEY_FRAMES = 256
LACT_MAX_Q_BLOCKS = 16
LACT_MAX_MEMBERS = 1024
LACT_MAX_TOKENS = 262144
LACT_STATIC_QUEUE_MAX = 16384
SEG_MEMORY, SEG_WINDOW, SEG_CURRENT, SEG_REF = 0, 1, 2, 3
STATUS = {0: "LACT_OK", 1: "LACT_E_INVALID", 2: "LACT_E_SHAPE", 3: "LACT_E_CAPACITY",
          4: "LACT_E_DTYPE", 5: "LACT_E_STATE", 6: "LACT_E_HIP"}

_TORCH_DTYPE = {LACT_F32: torch.float32, LACT_BF16: torch.bfloat16}


class lact_cfg(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("window_frames", ctypes.c_int32), ("mem_slots", ctypes.c_int32),
                ("ratio", ctypes.c_int32), ("max_block_frames", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("rope_mode", ctypes.c_int32), ("rope_split", ctypes.c_int32 * 3),
                ("rope_theta", ctypes.c_float), ("ref_frames", ctypes.c_int32)]


class lact_key_frame(ctypes.Structure):
    _fields_ = [("segment", ctypes.c_int32), ("physical_slot", ctypes.c_int32),
                ("absolute_id", ctypes.c_int64), ("t_pos", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class lact_state(ctypes.Structure):
    _fields_ = [("F", ctypes.c_int64), ("E", ctypes.c_int64), ("G", ctypes.c_int64),
                ("win_len", ctypes.c_int32), ("mem_len", ctypes.c_int32),
                ("pending", ctypes.c_int32), ("ring_slots", ctypes.c_int32),
                ("version", ctypes.c_uint64), ("staged_frames", ctypes.c_int32),
                ("staged_valid", ctypes.c_int32), ("ref_valid", ctypes.c_int32),
                ("staged_member", ctypes.c_int32)]


_PERSISTENT = ("ring_k", "ring_v", "mem_k", "mem_v", "ref_k", "ref_v", "ring_k_scale",
               "ring_v_scale", "mem_k_scale", "mem_v_scale", "ref_k_scale", "ref_v_scale")

_LAYOUT_FIELDS = ["total", "ring_k", "ring_v", "mem_k", "mem_v", "ref_k", "ref_v", "krot", "qrot",
                  "vcur", "vcur_scale", "vscale", "ring_k_scale", "ring_v_scale", "mem_k_scale", "mem_v_scale",
                  "ref_k_scale", "ref_v_scale", "rope_table", "attn_flags", "vmax", "frame_bytes"]


class lact_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _LAYOUT_FIELDS] + \
               [("ring_slots", ctypes.c_int32), ("key_frames_max", ctypes.c_int32),
                ("member_bytes", ctypes.c_size_t), ("members", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class LactError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


EXPORTS = ["lact_cache_footprint", "lact_cache_layout", "lact_cache_init", "lact_cache_destroy",
           "lact_set_footprint", "lact_set_layout", "lact_set_init",
           "lact_ref_set", "lact_rope_reset_apply", "lact_block_attention",
           "lact_member_ref_set", "lact_member_rope_reset_apply", "lact_member_block_attention",
           "lact_member_block_attention_static", "lact_kv_ring_append",
           "lact_convkv_compress", "lact_cache_state", "lact_cache_keys", "lact_plan_create",
           "lact_plan_destroy", "lact_plan_append", "lact_plan_compress", "lact_plan_state",
           "lact_plan_keys", "lact_last_error"]

_lib = None


def lib():
    """The loaded liblact.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
                           "python -m compressed_kv_causal_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, vp, i32, i64 = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "lact_cache_footprint": [P(lact_cfg), P(ctypes.c_size_t)],
        "lact_cache_layout": [P(lact_cfg), P(lact_layout)],
        "lact_cache_init": [P(lact_cfg), vp, ctypes.c_size_t, P(vp)],
        "lact_cache_destroy": [vp],
        "lact_set_footprint": [P(lact_cfg), i32, P(ctypes.c_size_t)],
        "lact_set_layout": [P(lact_cfg), i32, P(lact_layout)],
        "lact_set_init": [P(lact_cfg), i32, vp, ctypes.c_size_t, P(vp)],
        "lact_ref_set": [vp, vp, vp, i32, vp],
        "lact_rope_reset_apply": [vp, vp, vp, vp, i32, vp],
        "lact_block_attention": [vp, P(i32), i32, vp, vp, vp],
        "lact_member_ref_set": [vp, i32, vp, vp, i32, vp],
        "lact_member_rope_reset_apply": [vp, i32, vp, vp, vp, i32, vp],
        "lact_member_block_attention": [vp, i32, P(i32), i32, vp, vp, vp],
        "lact_member_block_attention_static": [vp, i32, P(i32), i32, vp, vp, vp],
        "lact_kv_ring_append": [vp, vp, vp, i32, vp],
        "lact_convkv_compress": [vp, vp, vp, vp, vp, vp, P(i32)],
        "lact_cache_state": [vp, P(lact_state)],
        "lact_cache_keys": [vp, i32, P(lact_key_frame), i32, P(i32)],
        "lact_plan_create": [P(lact_cfg), P(vp)],
        "lact_plan_destroy": [vp],
        "lact_plan_append": [vp, i32],
        "lact_plan_compress": [vp, P(i64), i32, P(i32), P(i32)],
        "lact_plan_state": [vp, P(lact_state)],
        "lact_plan_keys": [vp, i32, P(lact_key_frame), i32, P(i32)],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.lact_last_error.argtypes = []
    L.lact_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise LactError(status, lib().lact_last_error().decode())


def make_cfg(heads, head_dim, grid_h, grid_w, window_frames, mem_slots, ratio, max_block_frames,
             kv_dtype, q_dtype, rope_mode, rope_split, rope_theta=10000.0, ref_frames=0,
             **_ignored):
    c = lact_cfg()
    c.heads, c.head_dim, c.grid_h, c.grid_w = heads, head_dim, grid_h, grid_w
    c.window_frames, c.mem_slots, c.ratio = window_frames, mem_slots, ratio
    c.max_block_frames, c.kv_dtype, c.q_dtype = max_block_frames, kv_dtype, q_dtype
    c.rope_mode = rope_mode
    sp = list(rope_split) + [0] * (3 - len(rope_split))
    c.rope_split = (ctypes.c_int32 * 3)(*sp)
    c.rope_theta = rope_theta
    c.ref_frames = ref_frames
    return c


def _ptr(t, dtype=None, name="tensor"):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, shape, dtype, device, name):
    """Checks a tensor handed to a kernel: exact shape, dtype and device (the C calls take
    bare pointers and trust these, so a mismatch must stop here)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the cache on {device}")


def _frames(t, T, name):
    """Frames in a [n * T, ...] tensor (n >= 1 whole frames)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() < 1 or t.shape[0] == 0 or t.shape[0] % T:
        raise ValueError(f"{name} has {tuple(t.shape)[:1]} rows, not a whole number of {T}-token frames")
    return t.shape[0] // T


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ---- C calls -----------------------------------------------------------------------------

def lact_cache_footprint(cfg):
    n = ctypes.c_size_t()
    _check(lib().lact_cache_footprint(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def lact_cache_layout(cfg):
    L = lact_layout()
    _check(lib().lact_cache_layout(ctypes.byref(cfg), ctypes.byref(L)))
    return L


def lact_cache_init(cfg, device_buf_ptr, nbytes):
    h = ctypes.c_void_p()
    _check(lib().lact_cache_init(ctypes.byref(cfg), ctypes.c_void_p(device_buf_ptr), nbytes,
                                 ctypes.byref(h)))
    return h


def lact_cache_destroy(h):
    _check(lib().lact_cache_destroy(h))


def lact_set_footprint(cfg, n_members):
    n = ctypes.c_size_t()
    _check(lib().lact_set_footprint(ctypes.byref(cfg), n_members, ctypes.byref(n)))
    return n.value


def lact_set_layout(cfg, n_members):
    L = lact_layout()
    _check(lib().lact_set_layout(ctypes.byref(cfg), n_members, ctypes.byref(L)))
    return L


def lact_set_init(cfg, n_members, device_buf_ptr, nbytes):
    h = ctypes.c_void_p()
    _check(lib().lact_set_init(ctypes.byref(cfg), n_members, ctypes.c_void_p(device_buf_ptr),
                               nbytes, ctypes.byref(h)))
    return h


def lact_rope_reset_apply(h, q, k_cur, v_cur, n_frames, stream=None):
    _check(lib().lact_rope_reset_apply(h, _ptr(q, name="q"), _ptr(k_cur, name="k_cur"),
                                       _ptr(v_cur, name="v_cur"), n_frames, _stream(stream)))


def _blocks(q_block_frames):
    if q_block_frames is None:
        return None, 0
    n = len(q_block_frames)
    return (ctypes.c_int32 * n)(*q_block_frames), n


def lact_block_attention(h, q_block_frames, out, lse=None, stream=None):
    arr, n = _blocks(q_block_frames)
    lse_p = _ptr(lse, torch.float32, "lse") if lse is not None else None
    _check(lib().lact_block_attention(h, arr, n, _ptr(out, name="out"), lse_p, _stream(stream)))


def lact_ref_set(h, k_ref, v_ref, n_frames, stream=None):
    _check(lib().lact_ref_set(h, _ptr(k_ref, name="k_ref"), _ptr(v_ref, name="v_ref"), n_frames,
                              _stream(stream)))


def lact_member_rope_reset_apply(h, member, q, k_cur, v_cur, n_frames, stream=None):
    _check(lib().lact_member_rope_reset_apply(h, member, _ptr(q, name="q"),
                                              _ptr(k_cur, name="k_cur"), _ptr(v_cur, name="v_cur"),
                                              n_frames, _stream(stream)))


def lact_member_block_attention(h, member, q_block_frames, out, lse=None, stream=None):
    arr, n = _blocks(q_block_frames)
    lse_p = _ptr(lse, torch.float32, "lse") if lse is not None else None
    _check(lib().lact_member_block_attention(h, member, arr, n, _ptr(out, name="out"), lse_p,
                                             _stream(stream)))


def lact_member_block_attention_static(h, member, q_block_frames, out, lse=None, stream=None):
    """lact_member_block_attention with the exact pass's work queue in the library's static
    device array (no workspace of the cache buffer is used)."""
    arr, n = _blocks(q_block_frames)
    lse_p = _ptr(lse, torch.float32, "lse") if lse is not None else None
    _check(lib().lact_member_block_attention_static(h, member, arr, n, _ptr(out, name="out"),
                                                    lse_p, _stream(stream)))


def lact_member_ref_set(h, member, k_ref, v_ref, n_frames, stream=None):
    _check(lib().lact_member_ref_set(h, member, _ptr(k_ref, name="k_ref"),
                                     _ptr(v_ref, name="v_ref"), n_frames, _stream(stream)))


def lact_kv_ring_append(h, k_new, v_new, n_frames, stream=None):
    _check(lib().lact_kv_ring_append(h, _ptr(k_new, name="k_new"), _ptr(v_new, name="v_new"),
                                     n_frames, _stream(stream)))


def lact_convkv_compress(h, w_k, b_k, w_v, b_v, stream=None):
    n = ctypes.c_int32()
    f = torch.float32
    _check(lib().lact_convkv_compress(h, _ptr(w_k, f, "w_k"), _ptr(b_k, f, "b_k"),
                                      _ptr(w_v, f, "w_v"), _ptr(b_v, f, "b_v"), _stream(stream),
                                      ctypes.byref(n)))
    return n.value


def _state_dict(st):
    return {n: getattr(st, n) for n, _ in lact_state._fields_}


def _keys_list(arr, n):
    return [dict(segment=arr[i].segment, slot=arr[i].physical_slot, id=arr[i].absolute_id,
                 t_pos=arr[i].t_pos) for i in range(n)]


def lact_cache_state(h):
    st = lact_state()
    _check(lib().lact_cache_state(h, ctypes.byref(st)))
    return _state_dict(st)


def lact_cache_keys(h, n_cur):
    arr = (lact_key_frame * LACT_MAX_KEY_FRAMES)()
    n = ctypes.c_int32()
    _check(lib().lact_cache_keys(h, n_cur, arr, LACT_MAX_KEY_FRAMES, ctypes.byref(n)))
    return _keys_list(arr, n.value)


class Plan:
    """Host-only bookkeeping planner (no device)."""

    def __init__(self, cfg):
        self.h = ctypes.c_void_p()
        _check(lib().lact_plan_create(ctypes.byref(cfg), ctypes.byref(self.h)))

    def __del__(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.lact_plan_destroy(self.h)
            self.h = None

    def append(self, n):
        _check(lib().lact_plan_append(self.h, n))

    def compress(self):
        arr = (ctypes.c_int64 * 64)()
        n, w = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().lact_plan_compress(self.h, arr, 64, ctypes.byref(n), ctypes.byref(w)))
        return [arr[i] for i in range(min(n.value, 64))], w.value

    def state(self):
        st = lact_state()
        _check(lib().lact_plan_state(self.h, ctypes.byref(st)))
        return _state_dict(st)

    def keys(self, n_cur):
        arr = (lact_key_frame * LACT_MAX_KEY_FRAMES)()
        n = ctypes.c_int32()
        _check(lib().lact_plan_keys(self.h, n_cur, arr, LACT_MAX_KEY_FRAMES, ctypes.byref(n)))
        return _keys_list(arr, n.value)


class Cache:
    """One ConvKV cache, or a set of ``members`` caches advanced together (one per layer and
    diffusion step): a device buffer of lact_set_footprint bytes plus its handle.  With one
    member the plain calls are used, with several the lact_member_* forms (``member=``)."""

    def __init__(self, cfg, device="cuda", members=1):
        self.cfg = cfg if isinstance(cfg, lact_cfg) else make_cfg(**cfg)
        self.members = members
        if members == 1:
            self.nbytes = lact_cache_footprint(self.cfg)
            self.layout = lact_cache_layout(self.cfg)
        else:
            self.nbytes = lact_set_footprint(self.cfg, members)
            self.layout = lact_set_layout(self.cfg, members)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        if members == 1:
            self.h = lact_cache_init(self.cfg, self.buf.data_ptr(), self.nbytes)
        else:
            self.h = lact_set_init(self.cfg, members, self.buf.data_ptr(), self.nbytes)
        c = self.cfg
        self.T = c.grid_h * c.grid_w
        self.H, self.D = c.heads, c.head_dim
        self.io_dtype = _TORCH_DTYPE[c.q_dtype]
        self._v_held = None   # v_cur of the last RoPE call (see rope_reset_apply)

    def close(self):
        if self.h:
            lact_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            if getattr(self, "h", None) and _lib is not None:
                _lib.lact_cache_destroy(self.h)
                self.h = None
        except Exception:
            pass

    # the four hot-path calls (every tensor is checked for shape, dtype and device first;
    # the lact_* functions above take the caller's sizes on trust)
    def _io(self, t, rows, name):
        _expect(t, (rows, self.H, self.D), self.io_dtype, self.buf.device, name)

    def rope_reset_apply(self, q, k_cur, v_cur, stream=None, member=0):
        n = _frames(q, self.T, "q")
        for t, name in ((q, "q"), (k_cur, "k_cur"), (v_cur, "v_cur")):
            self._io(t, n * self.T, name)
        if self.members == 1 and member == 0:
            lact_rope_reset_apply(self.h, q, k_cur, v_cur, n, stream)
        else:
            lact_member_rope_reset_apply(self.h, member, q, k_cur, v_cur, n, stream)
        # a bf16 or f32 cache's attention reads the block's V from v_cur: hold the tensor so
        # its memory is not handed to another tensor before that attention call has run
        self._v_held = v_cur

    def block_attention(self, q_block_frames=None, out=None, lse=None, stream=None, member=0):
        st = self.state()
        Lq = st["staged_frames"] * self.T
        if out is None:
            out = torch.empty((Lq, self.H, self.D), dtype=self.io_dtype, device=self.buf.device)
        self._io(out, Lq, "out")
        if lse is not None:
            _expect(lse, (self.H, Lq), torch.float32, self.buf.device, "lse")
        if self.members == 1 and member == 0:
            lact_block_attention(self.h, q_block_frames, out, lse, stream)
        else:
            lact_member_block_attention(self.h, member, q_block_frames, out, lse, stream)
        return out

    def block_attention_static(self, q_block_frames=None, out=None, lse=None, stream=None,
                               member=0):
        """block_attention through lact_member_block_attention_static."""
        st = self.state()
        Lq = st["staged_frames"] * self.T
        if out is None:
            out = torch.empty((Lq, self.H, self.D), dtype=self.io_dtype, device=self.buf.device)
        self._io(out, Lq, "out")
        if lse is not None:
            _expect(lse, (self.H, Lq), torch.float32, self.buf.device, "lse")
        lact_member_block_attention_static(self.h, member, q_block_frames, out, lse, stream)
        return out

    def ref_set(self, k_ref, v_ref, stream=None, member=0):
        n = _frames(k_ref, self.T, "k_ref")
        self._io(k_ref, n * self.T, "k_ref")
        self._io(v_ref, n * self.T, "v_ref")
        if self.members == 1 and member == 0:
            lact_ref_set(self.h, k_ref, v_ref, n, stream)
        else:
            lact_member_ref_set(self.h, member, k_ref, v_ref, n, stream)

    def kv_ring_append(self, k_new, v_new, stream=None):
        """k_new, v_new: [members * n * T, H, D] (members stacked) or [n * T, H, D]."""
        n = _frames(k_new, self.T * self.members, "k_new")
        self._io(k_new, self.members * n * self.T, "k_new")
        self._io(v_new, self.members * n * self.T, "v_new")
        lact_kv_ring_append(self.h, k_new, v_new, n, stream)

    def convkv_compress(self, w_k, b_k, w_v, b_v, stream=None):
        """w_k, w_v: [C, r] f32 ([members, C, r] for a set); b_k, b_v: [C] ([members, C])."""
        C, r = self.H * self.D, self.cfg.ratio
        lead = () if self.members == 1 else (self.members,)
        for t, shape, name in ((w_k, lead + (C, r), "w_k"), (w_v, lead + (C, r), "w_v"),
                               (b_k, lead + (C,), "b_k"), (b_v, lead + (C,), "b_v")):
            _expect(t, shape, torch.float32, self.buf.device, name)
        return lact_convkv_compress(self.h, w_k, b_k, w_v, b_v, stream)

    def state(self):
        return lact_cache_state(self.h)

    def keys(self, n_cur):
        return lact_cache_keys(self.h, n_cur)

    # views into the buffer (inspection / tests)
    def region(self, name, slots, dtype, per_slot_elems, member=0):
        off = getattr(self.layout, name)
        if name in _PERSISTENT:
            off += member * self.layout.member_bytes
        itemsize = torch.empty((), dtype=dtype).element_size()
        n = slots * per_slot_elems
        return self.buf[off: off + n * itemsize].view(dtype).view(slots, per_slot_elems)
