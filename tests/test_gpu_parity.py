"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.  Bars: bookkeeping and indices bit-exact; compressed memory and ring
contents bit-exact (they are f32 fma chains and RNE/e4m3 encodes on both sides);
attention relative L2 <= 1e-5 (f32), 1e-2 (bf16), 5e-2 (FP8 KV)."""
import numpy as np
import pytest
import torch

import compressed_kv_causal_amd as L
import synth
from stream_helpers import BF16, F32, FP8, Runner, SetRunner, sample_rows

pytestmark = pytest.mark.gpu

ATTN_TOL = {F32: 1e-5, BF16: 1e-2, FP8: 5e-2}
LSE_TOL = {F32: 1e-5, BF16: 2e-2}


def say(msg):
    print(msg, flush=True)


def assert_state_matches(run):
    st = run.cache.state()
    ob = run.oc.bk.state()
    for key in ("F", "E", "G", "pending", "mem_len", "win_len", "ring_slots"):
        assert st[key] == ob[key], (key, st, ob)


def assert_keys_match(run, n):
    got = run.cache.keys(n)
    want = run.oc.keys(n)
    assert len(got) == len(want)
    for g, k in zip(got, want):
        assert (g["segment"], g["slot"], g["id"], g["t_pos"]) == \
            (k["segment"], k["slot"], k["id"], k["t_pos"])


def assert_memory_bitexact(run, slots=None):
    M = run.w["mem_slots"]
    for slot, (g, sk, sv) in sorted(run.oc.mem.items()):
        if slots is not None and slot not in slots:
            continue
        for tensor, stored in ((0, sk), (1, sv)):
            want, scales = run.oracle_stored_bytes(stored)
            got = run.mem_slot_bytes(tensor, slot)
            assert np.array_equal(got, want), f"memory slot {slot} (group {g}) tensor {tensor}"
            if scales is not None:
                name = "mem_k_scale" if tensor == 0 else "mem_v_scale"
                assert np.array_equal(run.scale_slot(name, slot), scales), f"scales of slot {slot}"
    assert len(run.oc.mem) == min(run.oc.bk.G, M)


def assert_ring_bitexact(run):
    for f, (sk, sv) in run.oc.raw.items():
        slot = run.oc.bk.raw_slot(f)
        for tensor, stored in ((0, sk), (1, sv)):
            want, scales = run.oracle_stored_bytes(stored)
            assert np.array_equal(run.ring_slot_bytes(tensor, slot), want), f"frame {f}"
            if scales is not None:
                name = "ring_k_scale" if tensor == 0 else "ring_v_scale"
                assert np.array_equal(run.scale_slot(name, slot), scales), f"scales frame {f}"


# ------------------------------------------------------------------------------------------
def test_tiny_f32_stream_full_parity():
    """Tiny f32: 27 history blocks then 20 AR steps, every step attended and compared on
    every output row, bookkeeping and key table compared every step."""
    w = synth.workload("tiny_f32")
    run = Runner(w)
    worst = 0.0
    for s in range(w["history_blocks"] + w["steps"]):
        assert_keys_match(run, 2)
        res = run.step(2)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[F32] and dl <= LSE_TOL[F32], (s, err, dl)
        assert_state_matches(run)
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    say(f"tiny f32: worst rel L2 {worst:.2e} over 47 steps")


def test_tiny_reference_stream_full_parity():
    """Tiny f32 with a 2-frame reference segment: 27 history blocks then 20 AR steps, every
    output row against the oracle, key table every step (reference first, positions 0, 1);
    the reference, ring and memory contents bit-exact; the reference replaced halfway."""
    w = synth.workload("tiny_ref")
    run = Runner(w)
    worst = 0.0
    for s in range(w["history_blocks"] + w["steps"]):
        if s == 30:
            run.seed += 1          # a new reference segment: the next steps must see it
            run.set_ref()
            run.seed -= 1
        assert_keys_match(run, 2)
        res = run.step(2)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[F32] and dl <= LSE_TOL[F32], (s, err, dl)
        assert_state_matches(run)
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    assert_ref_bitexact(run)
    say(f"tiny reference stream: worst rel L2 {worst:.2e} over 47 steps")


def test_s512_reference_step_parity():
    """512x512-shaped bf16 with a 2-frame reference segment (Lk = 34 frames)."""
    _big_step_parity("s512_ref2", 11, 8)


def test_fp8_reference_step_parity():
    """FP8 KV cache with a 2-frame reference segment (stored e4m3, dequantised by the RoPE
    pass like the rest of the history); 512x512 frames with 8 heads (the FP8 oracle's
    cost grows with the channel count; the kernels' paths do not)."""
    _big_step_parity("fp8_kv", 11, 8, ref_frames=2, heads=8)


@pytest.mark.parametrize("blocks", [[1, 2, 3], [2, 2, 2], [3, 3], [6]])
def test_tiny_multiblock_mask_vs_bruteforce(blocks):
    """Several query blocks in one call: the GPU's block-causal prefix against the oracle's
    explicit 0/-inf mask matrix (form 0), with memory and window present."""
    w = synth.workload("tiny_f32", max_block_frames=6)
    run = Runner(w)
    for _ in range(14):
        run.step(2, attend=False)
    res = run.step(6, blocks=blocks, form=0)
    err, dl = run.compare_attention(res)
    assert err <= ATTN_TOL[F32] and dl <= LSE_TOL[F32], (blocks, err, dl)


def test_tiny_window_only_and_no_memory():
    """M = 0 (window only): groups are consumed and dropped; attention over window + block."""
    w = synth.workload("tiny_f32", mem_slots=0)
    run = Runner(w)
    for s in range(12):
        res = run.step(2)
        err, dl = run.compare_attention(res)
        assert err <= ATTN_TOL[F32], (s, err)
        assert res["slots"] == 0
        assert_state_matches(run)


def test_tiny_no_window_memory_only():
    """W = 0 (every frame leaves the window at once): the context is [memory | current]
    with up to r - 1 pending frames unseen; 15 steps of 2 frames, every row against the
    oracle, state and memory bit-exact."""
    w = synth.workload("tiny_f32", window_frames=0, mem_slots=4)
    run = Runner(w)
    for s in range(15):
        assert_keys_match(run, 2)
        res = run.step(2)
        err, dl = run.compare_attention(res)
        assert err <= ATTN_TOL[F32] and dl <= LSE_TOL[F32], (s, err, dl)
        assert_state_matches(run)
    assert_memory_bitexact(run)


@pytest.mark.parametrize("tap", [None, 0, 3])
def test_frame_id_tag_on_device(tap):
    """No oracle: K element 0 of every frame holds the frame's absolute id.  With the
    uniform 1/5 kernel memory slot g holds 5g + 2 (5-frame mean); with a delta at tap k it
    holds exactly 5g + k."""
    w = synth.workload("tiny_f32")
    C = w["channels"]
    wt = np.zeros((C, 5), np.float32)
    if tap is None:
        wt[:] = np.float32(0.2)
    else:
        wt[:, tap] = 1.0
    b = np.zeros(C, np.float32)
    run = Runner(w, with_oracle=False, kernel=(wt, b, wt, b))
    for _ in range(40):
        run.step(2, attend=False, tag=True)
    st = run.cache.state()
    for g in range(st["G"] - st["mem_len"], st["G"]):
        val = run.mem_slot_bytes(0, g % w["mem_slots"]).view(np.float32)[0]
        if tap is None:
            assert abs(val - (5 * g + 2)) <= 1e-5 * (5 * g + 2), (g, val)
        else:
            assert val == 5 * g + tap, (g, val)


def assert_lse(run, res, kv):
    """FP8 workload (x8 outliers make scores large): the per-row bound that bf16 operand
    rounding implies; otherwise the fixed bar."""
    if kv == FP8:
        dl, bound = run.lse_errors(res), run.lse_bound(res)
        worst = int(np.argmax(dl / bound))
        say(f"  dLSE/bound worst {dl[worst]:.3e} / {bound[worst]:.3e}")
        assert np.all(dl <= bound)
    else:
        assert run.compare_attention(res)[1] <= LSE_TOL[kv]


def assert_ref_bitexact(run):
    for i, (sk, sv) in sorted(run.oc.ref.items()):
        for tensor, stored in ((0, sk), (1, sv)):
            want, scales = run.oracle_stored_bytes(stored)
            assert np.array_equal(run.ref_slot_bytes(tensor, i), want), f"reference frame {i}"
            if scales is not None:
                name = "ref_k_scale" if tensor == 0 else "ref_v_scale"
                assert np.array_equal(run.scale_slot(name, i), scales), f"scales of reference {i}"


def _big_step_parity(name, warm, n_last, per_head=6, first_check=False, **overrides):
    w = synth.workload(name, **overrides)
    run = Runner(w)
    kv = w["kv_dtype"]
    sizes = synth.block_sizes(w, warm + 1)
    errs = []
    for s, n in enumerate(sizes[:-1]):
        if first_check and s == 0:
            sel = sample_rows(w, n, seed=s, per_head=per_head)
            res = run.step(n, sel=sel)
            err, dl = run.compare_attention(res)
            say(f"{name} step 1 ({n} frames, no history): rel L2 {err:.3e}, worst head "
                f"{res['worst_head']:.3e}, worst row / bound {res['worst_row']:.3f}, max dLSE {dl:.2e}")
            assert err <= ATTN_TOL[kv]
            assert_lse(run, res, kv)
            errs.append(err)
        else:
            run.step(n, attend=False)
        assert_state_matches(run)
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    assert_ref_bitexact(run)
    assert_keys_match(run, n_last)
    sel = sample_rows(w, n_last, seed=99, per_head=per_head)
    res = run.step(n_last, sel=sel)
    err, dl = run.compare_attention(res)
    say(f"{name} step {warm + 1}: Lq {n_last * w['tokens']}, rel L2 {err:.3e}, worst head "
        f"{res['worst_head']:.3e}, worst row / bound {res['worst_row']:.3f}, max dLSE {dl:.2e}")
    assert err <= ATTN_TOL[kv]
    assert_lse(run, res, kv)
    return run


def test_s512_bf16_step_parity():
    """512x512-shaped bf16: 11 warm-up blocks (80 evicted -> 16 slots, bit-exact), then a
    full step (Lq 8192, Lk 32768) compared on sampled rows of all 40 heads."""
    _big_step_parity("s512_bf16", 11, 8)


def test_s720_bf16_step_parity():
    """720x416-shaped bf16: T = 1170 (non-power-of-two tails), first block 6 frames then 8."""
    _big_step_parity("s720_bf16", 11, 8, first_check=True)


@pytest.mark.parametrize("wb", [(6, 8), (6, 6), (8, 8)], ids=["w6_b8", "w6_b6", "w8_b8"])
def test_grid_step_parity(wb):
    """The model card's memory-block / current-block pairs (window W, blocks of B, memory
    16; 6 / 8 is the chosen one): ring R = W + B + 4, memory and ring bit-exact after the
    warm-up, then a step's attention against the oracle on sampled rows."""
    W, B = wb
    _big_step_parity(f"grid_w{W}_b{B}", 11, B)


def test_train_form_long_sequence():
    """Training form: one call over 46 frames in blocks 6, 8, 8, 8, 8, 8 (47104 query and
    key tokens, no history) under the block-causal mask; sampled rows of all 40 heads,
    always the first and last row of every frame, against the oracle."""
    w = synth.workload("train_s512")
    blocks = list(w["train_blocks"])
    n = sum(blocks)
    run = Runner(w)
    sel = sample_rows(w, n, seed=7, per_head=4)
    res = run.step(n, blocks=blocks, sel=sel)
    err, dl = run.compare_attention(res)
    say(f"train form {blocks}: Lq {n * w['tokens']}, rel L2 {err:.3e}, max dLSE {dl:.2e}")
    assert err <= ATTN_TOL[BF16] and dl <= LSE_TOL[BF16]


def test_fp8_s720_step_parity():
    """FP8 KV cache on the 720x416 grid (T = 1170, not a multiple of 64: key tiles straddle
    frames while V comes from the dequantised FP8 history), first block of 6 frames then 8,
    8 heads: stored codes and scales bit-exact after the warm-up, step attention against
    the oracle on sampled rows."""
    _big_step_parity("s720_bf16", 11, 8, first_check=True, kv_dtype=FP8, heads=8, outliers=True)


def test_fp8_append_compress_bitexact():
    """FP8 KV: ring codes and scales and the re-quantised memory slots bit-exact."""
    w = synth.workload("fp8_kv")
    run = Runner(w)
    for n in synth.block_sizes(w, 12):
        run.step(n, attend=False)
        assert_state_matches(run)
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)


@pytest.mark.parametrize("kv,ratio", [(BF16, 3), (BF16, 4), (FP8, 3), (FP8, 4)],
                         ids=["bf16_r3", "bf16_r4", "fp8_r3", "fp8_r4"])
def test_other_ratio_compress_bitexact(kv, ratio):
    """Ratios other than 5 take the generic compressor (any r, tokens one after another):
    over a stream whose memory wraps, every memory slot and ring frame (FP8: codes and
    scales) bit-exact against the oracle, the bookkeeping every step, and attention
    parity at the end."""
    name = "fp8_kv" if kv == FP8 else "s512_bf16"
    w = synth.workload(name, heads=8, grid_h=16, grid_w=16, window_frames=4, mem_slots=4,
                       max_block_frames=4, ratio=ratio)
    run = Runner(w)
    for s_ in range(14):
        run.step(4 if s_ % 3 else 3, attend=False)
        assert_state_matches(run)
    assert run.oc.bk.G > w["mem_slots"]
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    sel = sample_rows(w, 4, seed=5, per_head=16)
    res = run.step(4, sel=sel)
    err, dl = run.compare_attention(res)
    say(f"ratio {ratio} {name}: rel L2 {err:.3e}, worst head {res['worst_head']:.3e}")
    assert err <= ATTN_TOL[kv]
    assert_lse(run, res, kv)


def test_fp8_kv_step_parity():
    """512x512-shaped FP8 KV cache with 1% x8 outliers: first step (no history) and the
    step after 11 warm-up blocks, attention over the stored e4m3 history against the oracle
    on sampled rows of all 40 heads; ring and memory codes and scales bit-exact."""
    _big_step_parity("fp8_kv", 11, 8, first_check=True)


@pytest.mark.parametrize("blocks", [[1, 2, 3], [6]])
def test_fp8_d128_multiblock_mask_vs_bruteforce(blocks):
    """FP8 KV with D = 128 and T = 96 against the explicit mask matrix (several blocks)."""
    w = synth.workload("fp8_kv", heads=4, grid_h=8, grid_w=12, window_frames=4,
                       mem_slots=6, max_block_frames=6)
    run = Runner(w)
    for _ in range(9):
        run.step(2, attend=False)
    res = run.step(6, blocks=blocks, form=0)
    err, dl = run.compare_attention(res)
    say(f"fp8 d128 blocks {blocks}: rel L2 {err:.3e}, max dLSE {dl:.2e}")
    assert err <= ATTN_TOL[FP8], (blocks, err, dl)
    assert_lse(run, res, FP8)


@pytest.mark.parametrize("D", [64, 128], ids=["d64", "d128"])
def test_fp8_small_stream_memory_wraps(D):
    """FP8 KV, 60 steps of the tiny schedule with bf16 inputs (23 groups into 10 memory
    slots, so slots and their scales are overwritten twice): D = 64 on a 4x4 grid (the
    generic kernels) and D = 128 on an 8x8 grid (the production compressor and attention
    kernels); every step's attention against the oracle, state bit-exact every step and
    memory every 10 steps."""
    grid = dict(grid_h=4, grid_w=4) if D == 64 else dict(grid_h=8, grid_w=8, rope_mode=3,
                                                        rope_split=(44, 42, 42))
    w = synth.workload("tiny_f32", head_dim=D, kv_dtype=FP8, q_dtype=BF16, outliers=True, **grid)
    run = Runner(w)
    worst = 0.0
    for s in range(60):
        res = run.step(2)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[FP8], (s, err, dl)
        assert_lse(run, res, FP8)
        assert_state_matches(run)
        if s % 10 == 9:
            assert_memory_bitexact(run)
    assert run.oc.bk.G > 2 * w["mem_slots"]
    assert_ring_bitexact(run)
    say(f"fp8 d{D} stream: worst rel L2 {worst:.3e}, {run.oc.bk.G} groups")


@pytest.mark.parametrize("kv", [BF16, FP8], ids=["bf16", "fp8"])
def test_odd_tokens_stream(kv):
    """T = 81 (a 9x9 grid, odd): the RoPE pass's workgroups take two tokens, so the last one
    holds one token and the other's loads repeat it; the D = 128 attention kernel's key
    tiles straddle frames and its query tiles end mid-frame; the compressor's 42 (channel
    block, token run) items fill the 8 XCDs unevenly.  14 steps of 1-4 frames, every row
    against the oracle (each head and row to its bound), state every step, memory and
    ring bit-exact."""
    name = "fp8_kv" if kv == FP8 else "s512_bf16"
    w = synth.workload(name, heads=8, grid_h=9, grid_w=9, window_frames=4, mem_slots=4,
                       max_block_frames=4)
    run = Runner(w)
    worst = 0.0
    for s, n in enumerate([4, 2, 3, 4, 4, 1, 4, 3, 4, 4, 2, 4, 4, 4]):
        res = run.step(n)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[kv], (s, err, dl)
        assert_lse(run, res, kv)
        assert_state_matches(run)
    assert run.oc.bk.G > w["mem_slots"]
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    say(f"T=81 {'fp8' if kv == FP8 else 'bf16'} stream: worst rel L2 {worst:.3e}")


@pytest.mark.parametrize("kv", [BF16, FP8], ids=["bf16", "fp8"])
def test_many_heads_stream(kv):
    """72 heads x 128 on an 8x8 grid with a reference frame: one token's rows take 1152
    RoPE lanes, more than a workgroup's 1024, so the pass's lanes loop over them; 10 steps
    with history rebuilt from reference, memory and window, every row against the oracle,
    state and memory bit-exact."""
    w = synth.workload("tiny_ref", heads=72, head_dim=128, grid_h=8, grid_w=8, kv_dtype=kv,
                       q_dtype=BF16, rope_mode=3, rope_split=(44, 42, 42),
                       outliers=(kv == FP8))
    run = Runner(w)
    worst = 0.0
    for s in range(10):
        res = run.step(2)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[kv], (s, err, dl)
        assert_lse(run, res, kv)
        assert_state_matches(run)
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    assert_ref_bitexact(run)
    say(f"72-head {'fp8' if kv == FP8 else 'bf16'} stream: worst rel L2 {worst:.3e}")


def test_binding_rejects_mismatched_tensors():
    """Tensors of the wrong shape, dtype or device (or not whole frames) are refused by the
    binding before anything is launched, and the bookkeeping is left as it was."""
    w = synth.workload("tiny_f32")
    run = Runner(w, with_oracle=False)
    for _ in range(3):
        run.step(2, attend=False)
    c = run.cache
    T, H, D, C = w["tokens"], w["heads"], w["head_dim"], w["channels"]
    before = {k: c.state()[k] for k in ("F", "E", "G", "version")}
    good = torch.zeros((2 * T, H, D), dtype=torch.float32, device="cuda")
    bad = [torch.zeros((2 * T + 1, H, D), device="cuda"), torch.zeros((2 * T, H + 1, D), device="cuda"),
           torch.zeros((2 * T, H, D), dtype=torch.bfloat16, device="cuda"), torch.zeros((2 * T, H, D))]
    for x in bad:
        for args in ((x, good, good), (good, x, good), (good, good, x)):
            with pytest.raises(ValueError):
                c.rope_reset_apply(*args)
        with pytest.raises(ValueError):
            c.kv_ring_append(good, x)
    c.rope_reset_apply(good, good, good)
    with pytest.raises(ValueError):
        c.block_attention(out=torch.zeros((T, H, D), device="cuda"))
    with pytest.raises(ValueError):
        c.block_attention(lse=torch.zeros((H, T), device="cuda"))
    wk = torch.zeros((C, 5), device="cuda")
    bk = torch.zeros((C,), device="cuda")
    for args in ((wk[:, :4].contiguous(), bk, wk, bk), (wk, bk[:-1].contiguous(), wk, bk),
                 (wk, bk, wk.double(), bk)):
        with pytest.raises(ValueError):
            c.convkv_compress(*args)
    torch.cuda.synchronize()
    assert {k: c.state()[k] for k in before} == before


@pytest.mark.parametrize("D, dt", [(64, BF16), (128, F32)], ids=["bf16_d64", "f32_d128"])
def test_stream_t96(D, dt):
    """bf16 at D = 64 (the generic MFMA kernel) and f32 at D = 128 (the f32 kernel) on an
    8x12 grid, T = 96: key tiles straddle frames and query tiles end mid-frame; 30 steps
    with multi-block calls every third step, every row against the oracle, state
    bit-exact, memory overwritten (13 groups into 6 slots) and bit-exact."""
    rope = {} if D == 64 else dict(rope_mode=3, rope_split=(44, 42, 42))
    w = synth.workload("tiny_f32", heads=3, head_dim=D, grid_h=8, grid_w=12, kv_dtype=dt,
                       q_dtype=dt, mem_slots=6, max_block_frames=4, **rope)
    run = Runner(w)
    worst = 0.0
    for s in range(30):
        blocks = [1, 1] if s % 3 == 2 else None
        res = run.step(2, blocks=blocks, form=0 if blocks else 1)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[dt] and dl <= LSE_TOL[dt], (s, err, dl)
        assert_state_matches(run)
    assert run.oc.bk.G > w["mem_slots"]
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    say(f"D={D} T=96 stream: worst rel L2 {worst:.3e}")


def test_f32_d128_small_stream():
    """f32 cache and operands at D = 128 (the one-lane-per-row f32 kernel at its larger
    width), T = 16, 3D RoPE split (44, 42, 42): 20 steps of the tiny schedule, every row
    against the oracle, state and stored contents bit-exact."""
    w = synth.workload("tiny_f32", head_dim=128, rope_mode=3, rope_split=(44, 42, 42))
    run = Runner(w)
    worst = 0.0
    for s in range(20):
        res = run.step(2)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[F32] and dl <= LSE_TOL[F32], (s, err, dl)
        assert_state_matches(run)
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    say(f"f32 d128 stream: worst rel L2 {worst:.3e}")


def test_bf16_d128_short_frames_stream():
    """bf16 at D = 128 with T = 16 < 64 (a key tile would span several frames, so the
    exact online-softmax kernel serves these shapes): 20 steps, every row against the
    oracle, multi-block calls included."""
    w = synth.workload("tiny_f32", head_dim=128, kv_dtype=BF16, q_dtype=BF16, max_block_frames=4)
    run = Runner(w)
    worst = 0.0
    for s in range(20):
        blocks = [1, 1] if s % 3 == 2 else None
        res = run.step(2, blocks=blocks, form=0 if blocks else 1)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[BF16] and dl <= LSE_TOL[BF16], (s, err, dl)
        assert_state_matches(run)
    assert_memory_bitexact(run)
    say(f"bf16 d128 T=16 stream: worst rel L2 {worst:.3e}")


@pytest.mark.parametrize("grid_w", [8, 12], ids=["t64", "t96"])
@pytest.mark.parametrize("name", ["s512_bf16", "fp8_kv"], ids=["bf16", "fp8"])
def test_d128_dual_kernel_tile_counts(name, grid_w):
    """The two-block kernels' control flow (bf16 cache: k_attn_bf16_d128_dual; FP8 cache
    with x8 outliers: k_attn_f8v_d128_dual) over every short key-tile count.  T = 64 (one
    key tile per frame) or 96 (tiles straddle frames, a ragged last tile when the frame
    count is odd); one-frame blocks from an empty cache up to the full context of 4 memory
    + 4 window + 1 block frames, so 1 to 9 (T = 64) or 2 to 14 (T = 96) key tiles: no
    pipelined pass, one or two passes of four and every remainder after them; every fifth
    call two frames split into two query blocks (masked tiles).  Every row against the
    oracle, with the per-head and per-row checks."""
    w = synth.workload(name, heads=2, grid_h=8, grid_w=grid_w, window_frames=4, mem_slots=4,
                       max_block_frames=4)
    kv = w["kv_dtype"]
    run = Runner(w)
    worst = 0.0
    for s in range(24):
        blocks = [1, 1] if s % 5 == 4 else None
        res = run.step(2 if blocks else 1, blocks=blocks, form=0 if blocks else 1)
        err, dl = run.compare_attention(res)
        worst = max(worst, err)
        assert err <= ATTN_TOL[kv], (s, err, dl)
        assert_lse(run, res, kv)
        assert_state_matches(run)
    assert_memory_bitexact(run)
    say(f"{name} dual kernel tile counts, T = {8 * grid_w}: worst rel L2 {worst:.3e}")


@pytest.mark.parametrize("name", ["s512_bf16", "fp8_kv"])
def test_attention_repeats_bit_identical_and_unflagged(name):
    """The 512x512 step's attention (bf16 cache: k_attn_bf16_d128_dual; FP8:
    k_attn_f8v_d128_dual) called three times on one staged block, memory full: outputs and LSE bit-identical
    (the kernels have fixed reduction orders, so a difference would mean a race in the LDS
    ring or a result used before its MFMA wrote it), and no query tile handed to the exact
    pass on these inputs."""
    w = synth.workload(name)
    run = Runner(w, with_oracle=False)
    for n in synth.block_sizes(w, 11):
        run.step(n, attend=False)
    (q, _), (k, _), (v, _) = run.inputs(8)
    run.cache.rope_reset_apply(q, k, v)
    T, H = w["tokens"], w["heads"]
    got = []
    for _ in range(3):
        lse = torch.empty((H, 8 * T), dtype=torch.float32, device="cuda")
        out = run.cache.block_attention(lse=lse)
        torch.cuda.synchronize()
        got.append((out.clone(), lse.clone()))
    n_items = (8 * T + 255) // 256 * H
    flags = run.cache.buf[run.cache.layout.attn_flags:].view(torch.int32)[:n_items].cpu().numpy()
    say(f"{name}: flagged tiles {int(flags.sum())} of {n_items}, repeats identical "
        f"{[torch.equal(o, got[0][0]) and torch.equal(l, got[0][1]) for o, l in got[1:]]}")
    assert flags.max() == 0
    assert torch.isfinite(got[0][0].float()).all()
    for o, l in got[1:]:
        assert torch.equal(o, got[0][0]) and torch.equal(l, got[0][1])


@pytest.mark.parametrize("seed", [1, 2])
def test_s512_bf16_step_parity_other_seeds(seed):
    """The 512x512 bf16 step on two more input seeds (sampled rows of all heads)."""
    w = synth.workload("s512_bf16")
    run = Runner(w, seed=seed)
    for n in synth.block_sizes(w, 11):
        run.step(n, attend=False)
    assert_memory_bitexact(run)
    sel = sample_rows(w, 8, seed=seed, per_head=4)
    res = run.step(8, sel=sel)
    err, dl = run.compare_attention(res)
    say(f"s512 seed {seed}: rel L2 {err:.3e}, max dLSE {dl:.2e}")
    assert err <= ATTN_TOL[BF16] and dl <= LSE_TOL[BF16]


@pytest.mark.parametrize("ref", [0, 2], ids=["noref", "ref2"])
@pytest.mark.parametrize("blocks", [[1, 2, 3], [3, 3], [6], [2, 1, 1, 2]])
def test_bf16_d128_multiblock_mask_vs_bruteforce(blocks, ref):
    """D = 128 bf16 kernel with several query blocks per call and T = 96 (tiles of 32 keys
    and 256 query rows straddle frames and blocks), without and with a 2-frame reference
    segment at the head of the history: against the explicit mask matrix."""
    w = synth.workload("s512_bf16", heads=4, grid_h=8, grid_w=12, window_frames=4,
                       mem_slots=6, max_block_frames=6, ref_frames=ref)
    run = Runner(w)
    for _ in range(9):
        run.step(2, attend=False)
    res = run.step(6, blocks=blocks, form=0)
    err, dl = run.compare_attention(res)
    say(f"bf16 d128 blocks {blocks}: rel L2 {err:.3e}, max dLSE {dl:.2e}")
    assert err <= ATTN_TOL[BF16] and dl <= LSE_TOL[BF16], (blocks, err, dl)


def test_bf16_d128_max_query_blocks():
    """The largest call the ABI takes in query blocks: 16 blocks of one frame each (T = 64,
    so every block is one 64-key tile and every tile boundary is a block boundary) over a
    history, against the explicit mask matrix on every row."""
    w = synth.workload("s512_bf16", heads=2, grid_h=8, grid_w=8, window_frames=6,
                       mem_slots=4, max_block_frames=16, first_block=16, block=16)
    run = Runner(w)
    for _ in range(3):
        run.step(16, attend=False)
    blocks = [1] * 16
    res = run.step(16, blocks=blocks, form=0)
    err, dl = run.compare_attention(res)
    say(f"16 query blocks: rel L2 {err:.3e}, max dLSE {dl:.2e}")
    assert err <= ATTN_TOL[BF16] and dl <= LSE_TOL[BF16]


def test_bf16_d128_max_key_frames():
    """The largest key set the ABI takes: reference 2 + memory 120 + window 118 + block 16 =
    256 key frames (T = 64: 16384 keys, 256 tiles).  The memory is filled through the
    stream (605 evicted frames), then a full step is compared with the oracle on sampled
    rows of both heads; the stored memory, ring and reference stay bit-exact."""
    w = synth.workload("s512_bf16", heads=2, grid_h=8, grid_w=8, window_frames=118,
                       mem_slots=120, max_block_frames=16, first_block=16, block=16,
                       ref_frames=2, pool_blocks=0)
    cfg_kf = w["ref_frames"] + w["mem_slots"] + w["window_frames"] + w["max_block_frames"]
    assert cfg_kf == L.LACT_MAX_KEY_FRAMES
    run = Runner(w)
    n = 0
    while run.cache.state()["mem_len"] < w["mem_slots"]:
        run.step(16, attend=False)
        n += 1
    assert n < 60
    assert_state_matches(run)
    assert len(run.cache.keys(16)) == cfg_kf
    assert_keys_match(run, 16)
    sel = sample_rows(w, 16, seed=5, per_head=64)
    res = run.step(16, sel=sel)
    err, dl = run.compare_attention(res)
    say(f"256 key frames (Lk {cfg_kf * w['tokens']}): rel L2 {err:.3e}, max dLSE {dl:.2e}")
    assert err <= ATTN_TOL[BF16] and dl <= LSE_TOL[BF16]
    assert_memory_bitexact(run)
    assert_ring_bitexact(run)
    assert_ref_bitexact(run)


@pytest.mark.parametrize("name, key, flagged", [("s512_bf16", 7.0, False), ("fp8_kv", 7.0, False),
                                                 ("fp8_kv", 2000.0, True)],
                         ids=["bf16-60nats", "fp8-60nats", "fp8-overflow"])
def test_d128_late_preferred_key(name, key, flagged):
    """A late key that every query prefers (its channels set to `key`, the queries' to
    their magnitudes), by ~60 nats: probabilities near 2^35 under the reference, which
    lies 56 log2 units above the first tile's row maximum, so the fast kernels keep every
    tile (FP8: the per-row tile scales reach E ~ 30); or (key 2000) by far more than the
    f32 range: the FP8 fast kernel flags its query tiles and the exact pass redoes them
    (the bf16 case is test_bf16_d128_overflow_falls_back_to_exact_pass).  The result
    matches the oracle either way."""
    w = synth.workload(name, heads=2, grid_h=8, grid_w=8, window_frames=4,
                       mem_slots=4, max_block_frames=4)
    kv = w["kv_dtype"]
    run = Runner(w)
    for _ in range(6):
        run.step(2, attend=False)
    (q, qh), (k, kh), (v, vh) = run.inputs(4)
    T = w["tokens"]
    last = 4 * T - 1
    qh[:, :, :] = np.abs(qh)
    kh[last, :, :] = key
    q = torch.from_numpy(qh).to(torch.bfloat16).cuda()
    k = torch.from_numpy(kh).to(torch.bfloat16).cuda()
    qh, kh = q.float().cpu().numpy(), k.float().cpu().numpy()
    run.cache.rope_reset_apply(q, k, v)
    lse = torch.empty((w["heads"], 4 * T), dtype=torch.float32, device="cuda")
    out = run.cache.block_attention(lse=lse)
    flags = run.cache.buf[run.cache.layout.attn_flags:].view(torch.int32)[: w["heads"]].cpu().numpy()
    ref = run.oc.attention(qh, kh, vh)
    err, dl = run.compare_attention(dict(out=out, lse=lse, ref=ref))
    O_ref, LSE_ref, heads, rows = ref
    rel_lse = float(np.abs(lse.cpu().numpy()[heads, rows] - LSE_ref).max() / np.abs(LSE_ref).max())
    say(f"late preferred key {key} ({name}): flags {flags.tolist()}, rel L2 {err:.3e}, "
        f"max dLSE {dl:.2e}, rel dLSE {rel_lse:.2e}")
    assert flags.tolist() == [1 if flagged else 0] * w["heads"]
    assert err <= ATTN_TOL[kv] and rel_lse <= 2e-3


def test_bf16_d128_overflow_falls_back_to_exact_pass():
    """A late key whose score exceeds the first-tile reference by far more than the f32
    range (one current-frame key scaled x2000): the fast pass flags its tiles and the exact
    online-softmax pass redoes them; the result still matches the oracle."""
    w = synth.workload("s512_bf16", heads=2, grid_h=8, grid_w=8, window_frames=4,
                       mem_slots=4, max_block_frames=4)
    run = Runner(w)
    for _ in range(6):
        run.step(2, attend=False)
    (q, qh), (k, kh), (v, vh) = run.inputs(4)
    T = w["tokens"]
    last = 4 * T - 1
    qh[:, :, :] = np.abs(qh)                      # every query has positive channels
    kh[last, :, :] = 2000.0                       # the very last key aligns with all of them
    q = torch.from_numpy(qh).to(torch.bfloat16).cuda()
    k = torch.from_numpy(kh).to(torch.bfloat16).cuda()
    qh, kh = q.float().cpu().numpy(), k.float().cpu().numpy()
    run.cache.rope_reset_apply(q, k, v)
    lse = torch.empty((w["heads"], 4 * T), dtype=torch.float32, device="cuda")
    out = run.cache.block_attention(lse=lse)
    flags = run.cache.buf[run.cache.layout.attn_flags:].view(torch.int32)[: w["heads"]].cpu().numpy()
    assert flags.max() == 1, "the fast pass should have flagged its tile"
    ref = run.oc.attention(qh, kh, vh)
    res = dict(out=out, lse=lse, ref=ref)
    err, _ = run.compare_attention(res)
    O_ref, LSE_ref, heads, rows = ref
    lse_got = lse.cpu().numpy()[heads, rows]
    # scores here are ~2e4; bf16 storage of the rotated keys (~2000, ulp 8) moves them by
    # tens, so the LSE is held to a relative bar
    rel_lse = float(np.abs(lse_got - LSE_ref).max() / np.abs(LSE_ref).max())
    say(f"overflow fallback: flags {flags.tolist()}, rel L2 {err:.3e}, rel dLSE {rel_lse:.2e}")
    assert err <= ATTN_TOL[BF16] and rel_lse <= 2e-3


def test_fp8_codes_of_every_bf16_value():
    """The FP8 append's codes and scales against the oracle's quantiser for every finite
    bf16 value of magnitude <= 448: K rows carry 448 (scale 1, so the codes are of the
    values themselves: every rounding case of e4m3, ties and subnormals included); V rows
    carry 446 (scale 446/448, so the quantiser's f32 products land between bf16 values)."""
    w = synth.workload("fp8_kv", heads=8, grid_h=8, grid_w=8, window_frames=2, mem_slots=2,
                       max_block_frames=1, first_block=1, block=1)
    run = Runner(w)
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    bits = np.arange(0, 0x43E1, dtype=np.uint32)                 # +0 .. 448
    pos = (bits << 16).view(np.float32)
    vals = np.concatenate([pos, -pos])
    rows = T * H
    k = np.zeros((rows, D), np.float32)
    v = np.zeros((rows, D), np.float32)
    kv_vals = vals
    vv_vals = vals[np.abs(vals) <= 446.0]
    assert len(kv_vals) <= rows * (D - 1)
    for arr, lead, src in ((k, 448.0, kv_vals), (v, 446.0, vv_vals)):
        arr[:, 0] = lead
        flat = arr[:, 1:].reshape(-1)
        flat[: len(src)] = src
        arr[:, 1:] = flat.reshape(rows, D - 1)
    kt = torch.from_numpy(k.reshape(T, H, D)).to(torch.bfloat16)
    vt = torch.from_numpy(v.reshape(T, H, D)).to(torch.bfloat16)
    assert np.array_equal(kt.float().numpy().reshape(rows, D), k)   # bf16 values as given
    assert np.array_equal(vt.float().numpy().reshape(rows, D), v)
    run.cache.kv_ring_append(kt.cuda(), vt.cuda())
    run.oc.append(k.reshape(1, -1), v.reshape(1, -1))
    assert_ring_bitexact(run)
    say(f"fp8 codes: {len(kv_vals)} + {len(vv_vals)} values bit-exact")


def test_rope_attention_graph_replay():
    """The RoPE pass and the attention (which change no bookkeeping) captured in a HIP graph
    and replayed three times, with eager work and synchronisation between the replays:
    every replay's output and LSE equal the eager call's bit for bit."""
    w = synth.workload("s512_bf16", heads=2, grid_h=8, grid_w=8, window_frames=4,
                       mem_slots=4, max_block_frames=2)
    run = Runner(w, with_oracle=False)
    for _ in range(8):
        run.step(2, attend=False)
    (q, _), (k, _), (v, _) = run.inputs(2)
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    out = torch.empty((2 * T, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, 2 * T), dtype=torch.float32, device="cuda")
    run.cache.rope_reset_apply(q, k, v)
    run.cache.block_attention(out=out, lse=lse)
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.cache.rope_reset_apply(q, k, v)
        run.cache.block_attention(out=out, lse=lse)
    for rep in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_l), rep
        scratch = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
    say("rope + attention graph: 3 replays bit-identical to the eager call")


def test_first_rope_call_captured():
    """A fresh cache whose first RoPE + attention call is captured into a HIP graph: an
    eager call made before the graph has ever run still computes the cos/sin table and the
    history itself, and each replay stages everything on its own; both give the bits of a
    second cache that ran eagerly throughout."""
    w = synth.workload("s512_bf16", heads=2, grid_h=8, grid_w=8, window_frames=4,
                       mem_slots=4, max_block_frames=2)
    a, b = Runner(w, with_oracle=False), Runner(w, with_oracle=False)
    for _ in range(8):
        a.step(2, attend=False)
        b.step(2, attend=False)
    (q, _), (k, _), (v, _) = a.inputs(2)
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    new = lambda: (torch.empty((2 * T, H, D), dtype=torch.bfloat16, device="cuda"),
                   torch.empty((H, 2 * T), dtype=torch.float32, device="cuda"))
    (want_o, want_l), (out_g, lse_g), (out_e, lse_e) = new(), new(), new()
    b.cache.rope_reset_apply(q, k, v)
    b.cache.block_attention(out=want_o, lse=want_l)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        a.cache.rope_reset_apply(q, k, v)
        a.cache.block_attention(out=out_g, lse=lse_g)
    a.cache.rope_reset_apply(q, k, v)                 # eager, before any replay
    a.cache.block_attention(out=out_e, lse=lse_e)
    torch.cuda.synchronize()
    assert torch.equal(out_e, want_o) and torch.equal(lse_e, want_l)
    for rep in range(2):
        out_g.zero_()
        lse_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, want_o) and torch.equal(lse_g, want_l), rep
        b.cache.rope_reset_apply(q, k, v)             # other eager work between replays
        torch.cuda.synchronize()
    say("first call captured: eager call and 2 replays bit-identical to an eager cache")


# ---- cache sets: one cache per (layer, denoising step), advanced by batched launches ----

def test_tiny_set_stream_full_parity():
    """Tiny f32 set of 3 members with a 2-frame reference each, every member with its own
    inputs, conv weights and reference: 27 history blocks then 20 AR steps; every output row
    of every member against that member's oracle each step; one append and one compress
    launch per step for all members; each member's ring, memory and reference bit-exact."""
    w = synth.workload("tiny_ref")
    sr = SetRunner(w, 3)
    worst = 0.0
    for s in range(w["history_blocks"] + w["steps"]):
        for r in sr.runs:
            assert_keys_match(r, 2)
        res = sr.step(2)
        outs = []
        for r, x in zip(sr.runs, res):
            err, dl = r.compare_attention(x)
            worst = max(worst, err)
            assert err <= ATTN_TOL[F32] and dl <= LSE_TOL[F32], (s, r.member, err, dl)
            assert_state_matches(r)
            outs.append(x["out"].float().cpu().numpy())
        assert not np.array_equal(outs[0], outs[1])    # the members hold different data
    st = sr.cache.state()
    assert st["ref_valid"] == 1 and st["staged_member"] == 2
    for r in sr.runs:
        assert_memory_bitexact(r)
        assert_ring_bitexact(r)
        assert_ref_bitexact(r)
    say(f"tiny set of 3: worst rel L2 {worst:.2e} over 47 steps x 3 members")


def test_fp8_set_step_parity():
    """FP8 set of 2 members with a 2-frame reference, 512x512 frames with 8 heads: 11
    blocks through the batched append (quantising per member) and compress (each member's
    weights and scales), every member's memory, ring and reference bit-exact; then a full
    step of each member on sampled rows of all heads against its oracle."""
    w = synth.workload("fp8_kv", ref_frames=2, heads=8)
    sr = SetRunner(w, 2)
    for n in synth.block_sizes(w, 11):
        sr.step(n, attend=False)
    for r in sr.runs:
        assert_state_matches(r)
        assert_memory_bitexact(r)
        assert_ring_bitexact(r)
        assert_ref_bitexact(r)
    sel = sample_rows(w, 8, seed=99, per_head=4)
    res = sr.step(8, sel=sel)
    for r, x in zip(sr.runs, res):
        err, _ = r.compare_attention(x)
        say(f"fp8 set member {r.member}: rel L2 {err:.3e}")
        assert err <= ATTN_TOL[FP8]
        assert_lse(r, x, FP8)


def test_s512_set_equals_independent_caches():
    """512x512 bf16: a set of 2 members gives bit-identical outputs, LSE and cache contents
    to two independent caches fed the same inputs and weights (12 steps, the last 2
    attended)."""
    w = synth.workload("s512_bf16")
    sr = SetRunner(w, 2, with_oracle=False)
    solo = [Runner(w, seed=m, with_oracle=False) for m in range(2)]
    sizes = synth.block_sizes(w, 12)
    for i, n in enumerate(sizes):
        attend = i >= len(sizes) - 2
        res = sr.step(n, attend=attend, sel=False)
        ref = [r.step(n, attend=attend, sel=False) for r in solo]
        if attend:
            for m in range(2):
                assert torch.equal(res[m]["out"], ref[m]["out"]), (i, m)
                assert torch.equal(res[m]["lse"], ref[m]["lse"]), (i, m)
    assert sr.cache.state()["version"] == solo[0].cache.state()["version"]
    lay, one = sr.cache.layout, solo[0].cache.layout
    for m in range(2):
        a = sr.cache.buf[m * lay.member_bytes: (m + 1) * lay.member_bytes]
        b = solo[m].cache.buf[: one.member_bytes]
        assert torch.equal(a, b), f"persistent state of member {m}"
    say("s512 set of 2 == 2 independent caches, bit for bit")
