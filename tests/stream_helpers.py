"""Drives one cache through AR steps on the GPU (via the C ABI) and the oracle side by
side, on the same seeded inputs.  Test infrastructure."""
import numpy as np
import torch

import compressed_kv_causal_amd as L
import synth
from oracle.stream import OracleCache

F32, BF16, FP8 = 0, 1, 2


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


ATTN_BAR = {F32: 1e-5, BF16: 1e-2, FP8: 5e-2}


def row_bounds(O, rms, qnorm, kpair, heads, kv_dtype, D):
    """Per-row bound on |O_gpu - O| (L2 over the row's D outputs) from a rounding model:
    each key's softmax weight w_j gets an independent relative error -- the rounding of
    the probability fed to the PV product (unit roundoff u_P: 2^-8 in bf16, 2^-4 in e4m3),
    the block's own V rounded to e4m3 on the FP8 path (u_V = 2^-4), and the score error
    from bf16 Q and K (each element rounded with relative error <= 2^-8, uniform), whose
    variance per key is at most (2 u^2 / 3D) |q_i|^2 k_pair^2 (k_pair: the largest norm of
    a channel pair of any visible key of the head; RoPE keeps pair norms).  The error is
    then a sum of independent terms w_j e_j v_j whose RMS is at most
    sqrt(u_P^2/3 + u_V^2/3 + sigma_s^2) * RMS_i, RMS_i = sqrt(sum_j w_j^2 |v_j|^2) from the
    oracle; the bound takes 4 of those plus the bf16 rounding of the output.  None for the
    f32 path (no rounding beyond f32)."""
    if kv_dtype == F32:
        return None
    u = 2.0 ** -8
    uP = 2.0 ** -4 if kv_dtype == FP8 else u
    uV = 2.0 ** -4 if kv_dtype == FP8 else 0.0
    ss = u * np.sqrt(2.0 / (3.0 * D)) * qnorm * kpair[heads]
    sigma = np.sqrt(uP ** 2 / 3 + uV ** 2 / 3 + ss ** 2)
    return 4.0 * sigma * rms + u * np.linalg.norm(O, axis=1) + 1e-6


def check_heads_and_rows(got, O, heads, kv_dtype, bounds=None, label=""):
    """Every head's relative L2 within the dtype's bar, and (bounds) every row within its
    bound.  Returns (worst head rel L2, worst row error / bound)."""
    bar = ATTN_BAR[kv_dtype]
    worst_head, worst_h = 0.0, -1
    for h in np.unique(heads):
        sel = heads == h
        e = rel_l2(got[sel], O[sel])
        if e > worst_head:
            worst_head, worst_h = e, int(h)
    assert worst_head <= bar, f"{label}: head {worst_h} rel L2 {worst_head:.3e} > {bar}"
    worst_row = 0.0
    if bounds is not None:
        e = np.linalg.norm(np.asarray(got, np.float64) - O, axis=1)
        ratio = e / bounds
        i = int(np.argmax(ratio))
        worst_row = float(ratio[i])
        assert worst_row <= 1.0, (f"{label}: row {i} (head {int(heads[i])}) error {e[i]:.3e} > "
                                  f"bound {bounds[i]:.3e}")
    return worst_head, worst_row


def pair_norm_max(vals):
    """vals [..., H, D] -> [H]: the largest norm of a channel pair (2i, 2i+1)."""
    x = np.asarray(vals, np.float64)
    pn = np.sqrt(x[..., 0::2] ** 2 + x[..., 1::2] ** 2)      # [..., H, D/2]
    return pn.reshape(-1, pn.shape[-2], pn.shape[-1]).max(axis=(0, 2))


def io_dtype(w):
    return torch.float32 if w["q_dtype"] == F32 else torch.bfloat16


class Runner:
    """One cache, or (cache=, member=) one member of a set that a SetRunner advances."""

    def __init__(self, w, seed=0, with_oracle=True, kernel=None, cache=None, member=0):
        self.w = w
        self.seed = seed
        self.T, self.H, self.D = w["tokens"], w["heads"], w["head_dim"]
        self.cfg = L.make_cfg(**w)
        self.cache = cache if cache is not None else L.Cache(self.cfg)
        self.member = member
        self.mbase = member * self.cache.layout.member_bytes
        self.oc = OracleCache(w) if with_oracle else None
        if kernel is None:
            self.wk, self.bk = synth.conv_weights(w, seed, synth.TENSOR_WK)
            self.wv, self.bv = synth.conv_weights(w, seed, synth.TENSOR_WV)
        else:
            self.wk, self.bk, self.wv, self.bv = kernel
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.d_wk, self.d_bk, self.d_wv, self.d_bv = map(dev, (self.wk, self.bk, self.wv, self.bv))
        self.f = 0
        self.step_index = 0
        if w.get("ref_frames", 0):
            self.set_ref()

    def set_ref(self):
        """The reference segment from its own seeded streams, on the device cache and the
        oracle (the oracle gets the values as converted to the input dtype)."""
        kr, vr = synth.ref_frames(self.w, self.seed)
        n = kr.shape[0]
        tk, tv = (torch.from_numpy(x.reshape(n * self.T, self.H, self.D)).to(io_dtype(self.w))
                  for x in (kr, vr))
        self.cache.ref_set(tk.cuda(), tv.cuda(), member=self.member)
        if self.oc is not None:
            self.oc.set_ref(tk.float().numpy().reshape(n, -1), tv.float().numpy().reshape(n, -1))

    def inputs(self, n, tag=False):
        """(device tensor, host float32 values) for Q, K, V of frames f .. f+n-1."""
        ids = list(range(self.f, self.f + n))
        out = []
        for tensor in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V):
            x = synth.frames(self.w, self.seed, tensor, ids)
            if tag and tensor == synth.TENSOR_K:
                x[:, 0] = np.asarray(ids, np.float32)
            t = torch.from_numpy(x.reshape(n * self.T, self.H, self.D)).to(io_dtype(self.w))
            out.append((t.cuda(), t.float().numpy()))
        return out

    def step(self, n, attend=True, blocks=None, sel=None, lse=True, tag=False, form=1):
        """One AR step: rope -> attention -> append -> compress, on the GPU and the oracle.
        Returns dict(out, lse, ref) where ref = (O, LSE, heads, rows) of the oracle or None."""
        res = self.attend_part(n, attend, blocks, sel, lse, tag, form)
        self.cache.kv_ring_append(res["dk"], res["dv"])
        res["slots"] = self.cache.convkv_compress(self.d_wk, self.d_bk, self.d_wv, self.d_bv)
        self.oracle_advance(res)
        return res

    def oracle_advance(self, res):
        n = res["n"]
        if self.oc is not None:
            self.oc.append(res["k"].reshape(n, -1), res["v"].reshape(n, -1))
            res["groups"] = self.oc.compress(self.wk, self.bk, self.wv, self.bv)
        self.f += n
        self.step_index += 1

    def attend_part(self, n, attend=True, blocks=None, sel=None, lse=True, tag=False, form=1):
        """The step's inputs, and (attend) its RoPE + attention on the GPU and the oracle."""
        (q, qh), (k, kh), (v, vh) = self.inputs(n, tag)
        res = {"n": n, "dk": k, "dv": v, "k": kh, "v": vh}
        if attend:
            self.cache.rope_reset_apply(q, k, v, member=self.member)
            Lq = n * self.T
            lse_t = torch.empty((self.H, Lq), dtype=torch.float32, device="cuda") if lse else None
            out = self.cache.block_attention(blocks, lse=lse_t, member=self.member)
            res["out"], res["lse"] = out, lse_t
            if self.oc is not None and sel is not False:
                *ref, rms = self.oc.attention(qh, kh, vh, block_frames=blocks, sel=sel, form=form,
                                              want_rms=True)
                res["ref"] = tuple(ref)
                res["rms"] = rms
                res["kpair"] = np.maximum(self._hist_kpair(), pair_norm_max(kh))
                if self.w["kv_dtype"] == FP8:
                    res["hist_kmax"] = self._hist_kmax()
            res["q"] = qh
        return res

    # ---- comparisons -------------------------------------------------------------------
    def compare_attention(self, res):
        """(rel L2 of O over the oracle's selected rows, max |dLSE|).  Also holds every
        head's rel L2 to the dtype's bar and, with the oracle's per-row RMS, every row to
        its bound (row_bounds); records them as res["worst_head"], res["worst_row"]."""
        O, LSE, heads, rows = res["ref"]
        out = res["out"].float().cpu().numpy()           # [Lq][H][D]
        got = out[rows, heads, :]
        err = rel_l2(got, O)
        if "rms" in res:
            kv = self.w["kv_dtype"]
            qn = np.linalg.norm(res["q"][rows, heads, :].astype(np.float64), axis=1)
            b = row_bounds(O, res["rms"], qn, res["kpair"], heads, kv, self.D)
            res["worst_head"], res["worst_row"] = check_heads_and_rows(
                got, O, heads, kv, b, label=f"{self.w['name']} step {self.step_index}")
        dl = 0.0
        if res.get("lse") is not None:
            lse = res["lse"].cpu().numpy()
            dl = float(np.abs(lse[heads, rows] - LSE).max())
        return err, dl

    def _hist_kpair(self):
        """Per head, the largest channel-pair norm of a stored history key (0 if none)."""
        from oracle.bookkeeping import SEG_MEMORY, SEG_REF
        kp = np.zeros(self.H)
        for kf in self.oc.keys(0):
            if kf["segment"] == SEG_MEMORY:
                sk = self.oc.mem[kf["slot"]][1]
            elif kf["segment"] == SEG_REF:
                sk = self.oc.ref[kf["slot"]][0]
            else:
                sk = self.oc.raw[kf["id"]][0]
            vals, scales = self.oc.stored_value(sk)
            v = vals.astype(np.float64)
            if scales is not None:
                v = v * scales[..., None]
            kp = np.maximum(kp, pair_norm_max(v))
        return kp

    def _hist_kmax(self):
        """Per head, the largest norm of a stored history key at the present state."""
        from oracle.bookkeeping import SEG_MEMORY, SEG_REF
        kmax = np.zeros(self.H)
        for kf in self.oc.keys(0):
            if kf["segment"] == SEG_MEMORY:
                sk = self.oc.mem[kf["slot"]][1]
            elif kf["segment"] == SEG_REF:
                sk = self.oc.ref[kf["slot"]][0]
            else:
                sk = self.oc.raw[kf["id"]][0]
            vals, scales = self.oc.stored_value(sk)
            n = np.linalg.norm(vals.astype(np.float64), axis=2)
            if scales is not None:
                n = n * scales
            kmax = np.maximum(kmax, n.max(axis=0))
        return kmax

    def lse_bound(self, res):
        """Per selected row, a bound on |dLSE| from bf16 operands: RoPE'd q and k are rounded
        to bf16 (relative error <= 2^-9 per element), so every score moves by at most
        2^-8 |q_i| |k_j| / sqrt(D) (Cauchy-Schwarz), and the LSE, 1-Lipschitz in the
        max-norm of the scores, by at most the largest such move.  RoPE keeps norms, so the
        norms of the unrotated stored / input vectors serve.  10% slack + 1e-4 for the f32
        exp/log/sum arithmetic."""
        O_, LSE_, heads, rows = res["ref"]
        kmax = np.maximum(np.linalg.norm(res["k"], axis=2).max(axis=0), res["hist_kmax"])
        qn = np.linalg.norm(res["q"][rows, heads, :].astype(np.float64), axis=1)
        return 2.0 ** -8 * qn * kmax[heads] / np.sqrt(self.D) * 1.1 + 1e-4

    def lse_errors(self, res):
        O_, LSE_, heads, rows = res["ref"]
        return np.abs(res["lse"].cpu().numpy()[heads, rows] - LSE_)

    def mem_slot_bytes(self, tensor, slot):
        """Raw bytes of memory slot `slot` of K (0) or V (1) as stored on the device."""
        lay = self.cache.layout
        fb = lay.frame_bytes
        off = self.mbase + (lay.mem_k if tensor == 0 else lay.mem_v) + slot * fb
        return self.cache.buf[off: off + fb].cpu().numpy()

    def ref_slot_bytes(self, tensor, i):
        lay = self.cache.layout
        fb = lay.frame_bytes
        off = self.mbase + (lay.ref_k if tensor == 0 else lay.ref_v) + i * fb
        return self.cache.buf[off: off + fb].cpu().numpy()

    def ring_slot_bytes(self, tensor, slot):
        lay = self.cache.layout
        fb = lay.frame_bytes
        off = self.mbase + (lay.ring_k if tensor == 0 else lay.ring_v) + slot * fb
        return self.cache.buf[off: off + fb].cpu().numpy()

    def scale_slot(self, name, slot):
        lay = self.cache.layout
        n = self.T * self.H
        off = self.mbase + getattr(lay, name) + slot * n * 4
        return self.cache.buf[off: off + n * 4].cpu().numpy().view(np.float32)

    def oracle_stored_bytes(self, stored):
        """Oracle stored representation -> (value bytes, scales or None) as the device keeps it."""
        if stored[0] == "fp8":
            return stored[1].view(np.uint8), stored[2]
        if self.w["kv_dtype"] == BF16:
            from oracle import bf16_encode
            return bf16_encode(stored[1]).view(np.uint8), None
        return stored[1].view(np.uint8), None


def sample_rows(w, n_frames, seed, per_head=16, heads=None):
    """Seeded query rows per head, always with the first and last row of every block and
    the rows around every 128-row tile edge's tail."""
    T = w["tokens"]
    Lq = n_frames * T
    base = {0, Lq - 1}
    for f in range(n_frames):
        base.add(f * T)
        base.add(f * T + T - 1)
    tail = (Lq // 128) * 128
    base.update(r for r in (tail, tail + 1, Lq - 2) if 0 <= r < Lq)
    u = synth.uniform(seed, synth.TENSOR_SAMPLE, 0, per_head)
    extra = {int(x * Lq) % Lq for x in u}
    rows = sorted(base | extra)
    H = w["heads"]
    hs = range(H) if heads is None else heads
    hh = np.repeat(np.asarray(list(hs), np.int32), len(rows))
    rr = np.tile(np.asarray(rows, np.int64), len(list(hs)))
    return hh, rr


class SetRunner:
    """A set of `members` caches (one per layer and denoising step) in one buffer: member m
    has its own seeded inputs (seed base + m), conv weights, reference segment and oracle;
    per step every member runs RoPE + attention, then one append and one compress launch
    advance all of them."""

    def __init__(self, w, members, seed=0, with_oracle=True):
        self.w = w
        self.cache = L.Cache(L.make_cfg(**w), members=members)
        self.runs = [Runner(w, seed=seed + m, with_oracle=with_oracle, cache=self.cache, member=m)
                     for m in range(members)]
        stack = lambda name: torch.stack([getattr(r, name) for r in self.runs]).contiguous()
        self.d_wk, self.d_bk, self.d_wv, self.d_bv = (stack(n) for n in ("d_wk", "d_bk", "d_wv", "d_bv"))

    def step(self, n, attend=True, **kw):
        res = [r.attend_part(n, attend, **kw) for r in self.runs]
        k = torch.cat([x["dk"] for x in res]).contiguous()
        v = torch.cat([x["dv"] for x in res]).contiguous()
        self.cache.kv_ring_append(k, v)
        slots = self.cache.convkv_compress(self.d_wk, self.d_bk, self.d_wv, self.d_bv)
        for r, x in zip(self.runs, res):
            x["slots"] = slots
            r.oracle_advance(x)
        return res
