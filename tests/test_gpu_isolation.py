"""What a step may read, and what a bad value may reach (walkthrough "SoulX-LiveAct",
section "ConvKV Memory": a step's context is the reference, the long-term memory, the
short-term window and the current block -- nothing else).

* Canary: before every RoPE + attention call, every ring slot outside the window (free
  or holding pending frames), every memory slot not yet written and every staging tail
  past the call's extent (rotated keys past Lk, queries past Lq, block V past its frames;
  FP8: their scales) is filled with NaN; the outputs stay finite and bit-identical to a
  twin cache that was never filled.  Pending frames are put back after the call (the
  compressor still reads them).
* NaN isolation: a NaN in one element of one head's K or V input leaves every other
  head's outputs bit-identical to a clean twin, through append, compression and the
  following steps.
"""
import numpy as np
import pytest
import torch

import compressed_kv_causal_amd as L
import synth
from stream_helpers import FP8, Runner

pytestmark = pytest.mark.gpu

SEG_MEMORY, SEG_WINDOW = 0, 1


def say(msg):
    print(msg, flush=True)


CASES = {
    "bf16_d128": dict(name="s512_bf16", grid_h=16, grid_w=16, heads=8, window_frames=4,
                      mem_slots=4, max_block_frames=4),
    "fp8_d128": dict(name="fp8_kv", grid_h=16, grid_w=16, heads=8, window_frames=4,
                     mem_slots=4, max_block_frames=4),
    "bf16_d64_t48": dict(name="s512_bf16", grid_h=6, grid_w=8, heads=4, head_dim=64,
                         rope_split=(22, 22, 20), window_frames=4, mem_slots=4,
                         max_block_frames=4),
}
SCHEDULE = [4, 2, 3, 4, 4, 1, 4, 3, 4, 4, 2, 4, 4, 4]   # memory fills after a few blocks


def _workload(case):
    kw = dict(CASES[case])
    return synth.workload(kw.pop("name"), **kw)


class _Region:
    """Byte views of one cache's regions."""

    def __init__(self, run):
        self.c = run.cache
        self.lay = run.cache.layout
        self.w = run.w
        self.T, self.H, self.D = run.T, run.H, run.D
        self.fp8 = self.w["kv_dtype"] == FP8
        self.fb = self.lay.frame_bytes
        self.sb = self.T * self.H * 4                  # one frame of f32 row scales

    def span(self, off, nbytes):
        return self.c.buf[off: off + nbytes]

    def nan_fill(self, view, kind):
        if kind == "kv":             # a stored frame: bf16 NaN or e4m3 NaN codes
            view.view(torch.uint8).fill_(0x7F) if self.fp8 else view.view(torch.int16).fill_(0x7FC0)
        elif kind == "op":           # bf16 operands
            view.view(torch.int16).fill_(0x7FC0)
        else:                        # f32
            view.view(torch.int32).fill_(0x7FC00000)


def _canary(run, n):
    """NaN-fills what the coming call must not read; returns the pending frames' bytes to
    restore afterwards."""
    r = _Region(run)
    lay, T, H, D = r.lay, r.T, r.H, r.D
    keys = run.cache.keys(n)
    win_slots = {k["slot"] for k in keys if k["segment"] == SEG_WINDOW}
    mem_slots = {k["slot"] for k in keys if k["segment"] == SEG_MEMORY}
    saved = []
    for slot in range(lay.ring_slots):
        if slot in win_slots:
            continue
        for base, sbase in ((lay.ring_k, lay.ring_k_scale), (lay.ring_v, lay.ring_v_scale)):
            v = r.span(base + slot * r.fb, r.fb)
            saved.append((v, v.clone()))
            r.nan_fill(v, "kv")
            if r.fp8:
                sv = r.span(sbase + slot * r.sb, r.sb)
                saved.append((sv, sv.clone()))
                r.nan_fill(sv, "f32")
    for slot in range(run.w["mem_slots"]):
        if slot in mem_slots:
            continue
        for base, sbase in ((lay.mem_k, lay.mem_k_scale), (lay.mem_v, lay.mem_v_scale)):
            r.nan_fill(r.span(base + slot * r.fb, r.fb), "kv")
            if r.fp8:
                r.nan_fill(r.span(sbase + slot * r.sb, r.sb), "f32")
    KF, B = lay.key_frames_max, run.w["max_block_frames"]
    Lk, Lq = len(keys) * T, n * T
    ob = 2                                              # operand bytes (bf16)
    for h in range(H):
        head = lay.krot + h * KF * T * D * ob
        r.nan_fill(r.span(head + Lk * D * ob, (KF * T - Lk) * D * ob), "op")
        head = lay.qrot + h * B * T * D * ob
        if Lq < B * T:
            r.nan_fill(r.span(head + Lq * D * ob, (B * T - Lq) * D * ob), "op")
    if n < B:
        r.nan_fill(r.span(lay.vcur + n * r.fb, (B - n) * r.fb), "kv")
        if r.fp8:
            r.nan_fill(r.span(lay.vcur_scale + n * r.sb, (B - n) * r.sb), "f32")
    if r.fp8:
        row = KF * T + 64                                # each head's row ends in a zero pad
        P = H * row
        for plane in range(3):
            for h in range(H):
                at = lay.vscale + (plane * P + h * row + Lk) * 4
                r.nan_fill(r.span(at, (row - Lk) * 4), "f32")
    return saved


def _attend(run, q, k, v):
    run.cache.rope_reset_apply(q, k, v)
    lse = torch.empty((run.H, q.shape[0]), dtype=torch.float32, device="cuda")
    out = run.cache.block_attention(lse=lse)
    return out, lse


@pytest.mark.parametrize("case", list(CASES))
def test_canary_outside_the_context(case):
    w = _workload(case)
    say(f"canary: {case}")
    a = Runner(w, with_oracle=False)
    b = Runner(w, with_oracle=False)
    for step, n in enumerate(SCHEDULE):
        (q, _), (k, _), (v, _) = a.inputs(n)
        saved = _canary(a, n)
        out_a, lse_a = _attend(a, q, k, v)
        out_b, lse_b = _attend(b, q, k, v)
        torch.cuda.synchronize()
        for view, keep in saved:
            view.copy_(keep)
        assert torch.isfinite(out_a.float()).all() and torch.isfinite(lse_a).all(), step
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), step
        assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32)), step
        for run in (a, b):
            run.cache.kv_ring_append(k, v)
            run.cache.convkv_compress(run.d_wk, run.d_bk, run.d_wv, run.d_bv)
            run.f += n
    st = a.cache.state()
    assert st["mem_len"] == w["mem_slots"] and st["G"] > w["mem_slots"]
    lay = a.cache.layout
    persist = lay.member_bytes
    # both caches hold the same persistent state, except ring slots outside the window
    # (free or pending; a canary was put back in the pending ones)
    assert torch.equal(a.cache.buf[lay.mem_k: lay.ref_k], b.cache.buf[lay.mem_k: lay.ref_k])
    for kf in a.cache.keys(0):
        if kf["segment"] == SEG_WINDOW:
            for base in (lay.ring_k, lay.ring_v):
                off = base + kf["slot"] * lay.frame_bytes
                assert torch.equal(a.cache.buf[off: off + lay.frame_bytes],
                                   b.cache.buf[off: off + lay.frame_bytes])
    assert persist > 0


@pytest.mark.parametrize("case,tensor", [("bf16_d128", "k"), ("bf16_d128", "v"),
                                         ("fp8_d128", "k"), ("fp8_d128", "v"),
                                         ("bf16_d64_t48", "v")])
def test_nan_in_one_head_stays_in_that_head(case, tensor):
    w = _workload(case)
    H, T = w["heads"], w["tokens"]
    h0, tok, ch, at_step = 3 % H, T // 3, 5, 1
    say(f"NaN isolation: {case}, NaN in {tensor} head {h0}")
    a = Runner(w, with_oracle=False)
    b = Runner(w, with_oracle=False)
    others = [h for h in range(H) if h != h0]
    seen_nan = False
    for step, n in enumerate(SCHEDULE):
        (q, _), (k, _), (v, _) = a.inputs(n)
        ka, va = k.clone(), v.clone()
        if step == at_step:
            (ka if tensor == "k" else va)[tok, h0, ch] = float("nan")
        a.cache.rope_reset_apply(q, ka, va)
        b.cache.rope_reset_apply(q, k, v)
        lse_a = torch.empty((H, n * T), dtype=torch.float32, device="cuda")
        lse_b = torch.empty_like(lse_a)
        out_a = a.cache.block_attention(lse=lse_a)
        out_b = b.cache.block_attention(lse=lse_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a[:, others].view(torch.int16), out_b[:, others].view(torch.int16)), step
        assert torch.equal(lse_a[others].view(torch.int32), lse_b[others].view(torch.int32)), step
        seen_nan = seen_nan or not bool(torch.isfinite(out_a[:, h0].float()).all())
        a.cache.kv_ring_append(ka, va)
        b.cache.kv_ring_append(k, v)
        for run in (a, b):
            run.cache.convkv_compress(run.d_wk, run.d_bk, run.d_wv, run.d_bv)
            run.f += n
    assert a.cache.state()["G"] > w["mem_slots"]      # the NaN frame went through the memory
    say(f"  head {h0} outputs touched by the NaN: {seen_nan}")
