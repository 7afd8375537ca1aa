"""Oracle streaming driver: the stored KV of every live frame and memory slot, and the
attention of one AR step over it (test infrastructure).

Per AR step and per cache the pages' order is: attend with the current block over
[reference | memory | window | current], append the block's KV (append-only), compress once between
blocks (walkthrough "SoulX-LiveAct", sections "ConvKV Memory" and "Streaming Pipeline").

Stored values: F32 and BF16 caches keep the input values (BF16 inputs are bf16-exact);
the FP8 cache keeps e4m3 codes and one f32 scale per (token, head) ("--fp8_kv_cache":
store in FP8, dequantise on use; model card, Command Line Arguments).  The compressor
reads the dequantised value in f32 and its result is stored in the cache dtype again.
The attention sees the exact stored values; the current block's q, k, v are used as given
(their quantisation for FP8 matrix cores is arithmetic of the GPU path, not storage).
"""
import numpy as np

import oracle as O
from oracle.bookkeeping import Bookkeeping, SEG_MEMORY, SEG_REF

F32, BF16, FP8 = 0, 1, 2


class OracleCache:
    def __init__(self, cfg):
        self.cfg = dict(cfg)
        self.H, self.D = cfg["heads"], cfg["head_dim"]
        self.T = cfg["grid_h"] * cfg["grid_w"]
        self.C = self.H * self.D
        self.kv = cfg["kv_dtype"]
        self.bk = Bookkeeping(cfg["window_frames"], cfg["mem_slots"], cfg["ratio"],
                              cfg["max_block_frames"], cfg.get("ref_frames", 0))
        self.raw = {}   # absolute frame -> (k, v) stored
        self.mem = {}   # memory slot -> (group, k, v) stored
        self.ref = {}   # reference frame index -> (k, v) stored

    # ---- storage ---------------------------------------------------------------------
    def _store(self, x):
        """x [T*C] float32 -> stored representation."""
        if self.kv == FP8:
            codes, scales = O.quant_e4m3_rows(x.reshape(self.T * self.H, self.D), self.D)
            return ("fp8", codes.reshape(-1), scales.reshape(-1))
        if self.kv == BF16:
            return ("val", O.bf16_round(x))
        return ("val", np.array(x, dtype=np.float32, copy=True))

    def _f32(self, s):
        """Stored -> f32 value as the compressor reads it."""
        if s[0] == "fp8":
            return O.e4m3_dequant_f32(s[1].reshape(-1, self.D), s[2], self.D).reshape(-1)
        return s[1]

    def stored_value(self, s):
        """Stored -> (values float32 [T][H][D], scales float32 [T][H] or None) for attention."""
        if s[0] == "fp8":
            vals = O.e4m3_table()[s[1]].astype(np.float32)
            return vals.reshape(self.T, self.H, self.D), s[2].reshape(self.T, self.H)
        return s[1].reshape(self.T, self.H, self.D), None

    @classmethod
    def at_state(cls, cfg, F, frame_kv, wk, bk, wv, bv):
        """The cache after F frames were appended and every complete group compressed,
        built directly: memory slots are each compressed once from their own r frames, so
        only the groups still present and the live raw frames are needed.
        frame_kv(f) -> (k, v) float32 [T*C] input values of absolute frame f."""
        oc = cls(cfg)
        bk_ = oc.bk
        bk_.F = F
        G = bk_.E // bk_.r
        first = max(0, G - bk_.M) if bk_.M > 0 else G
        bk_.G = first
        for f in range(bk_.r * first, F):
            k, v = frame_kv(f)
            oc.raw[f] = (oc._store(k), oc._store(v))
        oc.compress(wk, bk, wv, bv)
        assert bk_.G == G
        return oc

    def set_ref(self, k_ref, v_ref):
        """Reference segment: [ref_frames][T*C] float32 input values, stored like any frame."""
        assert k_ref.shape[0] == self.bk.ref
        for i in range(self.bk.ref):
            self.ref[i] = (self._store(k_ref[i]), self._store(v_ref[i]))

    # ---- the four operations ---------------------------------------------------------
    def append(self, k_new, v_new):
        """k_new, v_new: [n][T*C] float32 input values."""
        n = k_new.shape[0]
        placed = self.bk.append(n)
        for i, (f, _slot) in enumerate(placed):
            self.raw[f] = (self._store(k_new[i]), self._store(v_new[i]))
        return placed

    def compress(self, wk, bk, wv, bv):
        groups = self.bk.compress()
        r, M = self.bk.r, self.bk.M
        for g in groups:
            if M > 0:
                xk = np.stack([self._f32(self.raw[r * g + k][0]) for k in range(r)])
                xv = np.stack([self._f32(self.raw[r * g + k][1]) for k in range(r)])
                mk = O.compress_chain_f32(xk, wk, bk)
                mv = O.compress_chain_f32(xv, wv, bv)
                self.mem[g % M] = (g, self._store(mk), self._store(mv))
        live_from = r * self.bk.G
        for f in [f for f in self.raw if f < live_from]:
            del self.raw[f]
        return groups

    def keys(self, n_cur):
        return self.bk.keys(n_cur)

    def history(self):
        """Stored K, V of [reference | memory | window] in attention order, with positions.
        Returns (k_vals, k_scales, v_vals, v_scales, t, u) with [L][H][D] values."""
        ks, kss, vs, vss, ts = [], [], [], [], []
        for kf in self.keys(0):
            if kf["segment"] == SEG_MEMORY:
                g, sk, sv = self.mem[kf["slot"]]
                assert g == kf["id"]
            elif kf["segment"] == SEG_REF:
                sk, sv = self.ref[kf["slot"]]
            else:
                sk, sv = self.raw[kf["id"]]
            kv_, ksc = self.stored_value(sk)
            vv_, vsc = self.stored_value(sv)
            ks.append(kv_)
            vs.append(vv_)
            kss.append(ksc)
            vss.append(vsc)
            ts.append(np.full(self.T, kf["t_pos"], np.int32))
        if not ks:
            return None, None, None, None, np.zeros(0, np.int32), np.zeros(0, np.int32)
        L = len(ks)
        u = np.tile(np.arange(self.T, dtype=np.int32), L)
        cat = np.concatenate
        fp8 = self.kv == FP8
        return (cat(ks), cat(kss) if fp8 else None, cat(vs), cat(vss) if fp8 else None,
                cat(ts), u)

    def attention(self, q, k_cur, v_cur, block_frames=None, sel=None, form=1, threads=None,
                  want_rms=False):
        """q, k_cur, v_cur: [n*T][H][D] float32 input values of the current block.
        Returns (O, LSE, heads, rows[, RMS]) for the selected outputs (see oracle.attention)."""
        n = q.shape[0] // self.T
        if block_frames is None:
            block_frames = [n]
        kh, khs, vh, vhs, ht, hu = self.history()
        n_hist_frames = len(self.keys(0))
        cur_t = np.repeat(np.arange(n, dtype=np.int32) + n_hist_frames, self.T)
        cur_u = np.tile(np.arange(self.T, dtype=np.int32), n)
        c = self.cfg
        return O.attention(q, k_cur, v_cur, kh, vh, ht, hu, cur_t, cur_u, block_frames, self.T,
                           c["rope_mode"], c["rope_split"], c["grid_w"], c["rope_theta"],
                           sel=sel, form=form, k_hist_scale=khs, v_hist_scale=vhs,
                           threads=threads, want_rms=want_rms)
