"""Pins of the CPU oracle against things other than itself: closed forms, hand-worked
values, brute force, special cases and an independent library (torch's bf16/e4m3 casts).

Each pin is chosen so that a plausible slip in the oracle (dropped term, wrong sign or
index, transposed operand, wrong tie rule) fails it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth
from oracle.bookkeeping import Bookkeeping, OracleStateError, OracleCapacityError
from oracle.stream import OracleCache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ======================================================================================
# bf16
# ======================================================================================

def _all_bf16_values():
    codes = np.arange(65536, dtype=np.uint32)
    vals = (codes << 16).view(np.float32).astype(np.float64)
    return codes.astype(np.uint16), vals


def test_bf16_nearest_bruteforce():
    """Nearest of all 65536 codes (ties to the even code) equals the oracle encoder."""
    codes, vals = _all_bf16_values()
    finite = np.isfinite(vals)
    fc, fv = codes[finite], vals[finite]
    order = np.argsort(fv, kind="stable")
    fc, fv = fc[order], fv[order]
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(3000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        # exact midpoints between neighbouring bf16 values: ties
        ((codes[16000:16400].astype(np.uint32) << 16) + 0x8000).view(np.float32),
    ])
    got = O.bf16_encode(xs)
    for x, g in zip(xs.astype(np.float64), got):
        d = np.abs(fv - x)
        best = d.min()
        cands = fc[d == best]
        # the same value can have two codes only for zero
        if x == 0.0:
            want = 0x8000 if math.copysign(1.0, x) < 0 else 0
        elif len(set(fv[d == best])) == 1:
            want = cands[0] if len(cands) == 1 else [c for c in cands if (c & 0x8000) == (0x8000 if x < 0 else 0)][0]
        else:
            want = [c for c in cands if (c & 1) == 0][0]
        assert g == want, (x, hex(g), hex(want))


def test_bf16_matches_torch_rne():
    """torch's float32 -> bfloat16 cast rounds to nearest even: an independent encoder."""
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(200000), rng.standard_normal(20000) * 1e5]).astype(np.float32)
    ours = O.bf16_encode(xs)
    theirs = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_nan_and_exact():
    assert O.bf16_encode(np.array([np.nan], np.float32))[0] & 0x7FC0 == 0x7FC0
    exact = np.array([1.0, -2.5, 3.140625, 0.0], np.float32)
    assert np.array_equal(O.bf16_value(O.bf16_encode(exact)), exact)


# ======================================================================================
# e4m3
# ======================================================================================

def test_e4m3_decode_points():
    g = load("e4m3_points.json")
    for code, val in g["decode"]:
        v = O.e4m3_value(int(code, 16))
        assert v == val and math.copysign(1, v) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(O.e4m3_value(int(code, 16)))


def test_e4m3_decode_closed_form():
    """value = (-1)^s 2^(e-7) (1 + m/8), or m/8 2^-6 for e = 0."""
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert O.e4m3_value(c) == (-mag if s else mag)


def test_e4m3_encode_points():
    for x, code in load("e4m3_points.json")["encode"]:
        assert O.e4m3_encode(x) == int(code, 16), x


def test_e4m3_roundtrip_every_code():
    for c in range(256):
        v = O.e4m3_value(c)
        if math.isnan(v):
            continue
        assert O.e4m3_encode(v) == c


def test_e4m3_nearest_bruteforce():
    table = O.e4m3_table()
    finite = [c for c in range(256) if not math.isnan(table[c])]
    rng = np.random.default_rng(2)
    xs = np.concatenate([rng.standard_normal(3000) * 50, rng.standard_normal(500) * 0.01,
                         rng.uniform(440, 600, 200)]).astype(np.float32)
    for x in xs.astype(np.float64):
        sign = 0x80 if x < 0 else 0
        cands = [c for c in finite if (c & 0x80) == sign]
        d = [abs(table[c] - x) for c in cands]
        best = min(d)
        tied = [c for c, di in zip(cands, d) if di == best]
        want = tied[0] if len(tied) == 1 else [c for c in tied if (c & 1) == 0][0]
        assert O.e4m3_encode(x) == want, x


def test_e4m3_matches_torch_in_range():
    """torch's float8_e4m3fn cast is round-to-nearest-even below the saturation point."""
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(2000) * 0.02]).astype(np.float32)
    xs = xs[np.abs(xs) < 440]
    theirs = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([O.e4m3_encode(x) for x in xs], np.uint8)
    assert np.array_equal(ours, theirs)


def test_quant_rows_scale_and_error():
    """scale = amax/448 (f32); the largest element codes to +-448; dequantised values are
    within half an e4m3 step of the input."""
    D = 128
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, D)).astype(np.float32)
    x[3] *= 8
    x[5] = 0
    codes, scales = O.quant_e4m3_rows(x, D)
    for r in range(64):
        amax = np.float32(np.abs(x[r]).max())
        if amax == 0:
            assert scales[r] == 1.0 and np.all((codes[r] & 0x7F) == 0)
            continue
        assert scales[r] == np.float32(amax / np.float32(448.0))
        j = int(np.abs(x[r]).argmax())
        assert codes[r, j] & 0x7F == 0x7E
    deq = O.e4m3_stored_value(codes, scales, D)
    err = np.abs(deq - x)
    bound = np.abs(x) * 2.0 ** -4 + scales[:, None].astype(np.float64) * 2.0 ** -10 + 1e-12
    assert np.all(err <= bound * 1.0001)


# ======================================================================================
# compression
# ======================================================================================

def test_compress_hand_example():
    g = load("compress_small.json")
    x = np.array(g["x"], np.float32)            # [r][C] one token
    w = np.array(g["w"], np.float32)
    b = np.array(g["b"], np.float32)
    out = O.compress_chain_f32(x, w, b)
    assert out.tolist() == g["expected"]
    assert O.compress_exact(x, w, b).tolist() == g["expected"]


def _rand_group(r=5, T=6, C=12, seed=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((r, T * C)).astype(np.float32)
    w = (rng.standard_normal((C, r)) * 0.2).astype(np.float32)
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    return x, w, b


@pytest.mark.parametrize("k", range(5))
def test_compress_delta_is_subsampling(k):
    """A delta kernel at tap k reduces the 5:1 conv to picking frame r*g + k, bit-exact."""
    x, _, _ = _rand_group()
    C = 12
    w = np.zeros((C, 5), np.float32)
    w[:, k] = 1.0
    out = O.compress_chain_f32(x, w, np.zeros(C, np.float32))
    assert np.array_equal(out, x[k])


def test_compress_uniform_is_mean():
    """The uniform kernel 1/5 ('mean memory') gives the 5-frame average, within the chain's
    rounding and the rounding of 1/5 to f32."""
    x, _, _ = _rand_group()
    C = 12
    w = np.full((C, 5), np.float32(0.2), np.float32)
    out = O.compress_chain_f32(x, w, np.zeros(C, np.float32)).astype(np.float64)
    mean = x.astype(np.float64).mean(axis=0)
    bound = 7 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=0) / 5 + 1e-30
    assert np.all(np.abs(out - mean) <= bound)


def test_compress_zero_weights_broadcast_bias():
    x, _, b = _rand_group()
    C = 12
    out = O.compress_chain_f32(x, np.zeros((C, 5), np.float32), b)
    assert np.array_equal(out, np.tile(b, 6))


def test_compress_linear_and_channel_indexing():
    """Scaling x by 2 scales the output by 2 exactly (b = 0); each channel uses its own
    weight row (a weight changed in channel c moves only channel c)."""
    x, w, _ = _rand_group()
    C = 12
    zb = np.zeros(C, np.float32)
    o1 = O.compress_chain_f32(x, w, zb)
    o2 = O.compress_chain_f32(2 * x, w, zb)
    assert np.array_equal(o2, 2 * o1)
    w2 = w.copy()
    w2[7, 3] += 1.0
    o3 = O.compress_chain_f32(x, w2, zb).reshape(6, C)
    d = o3 - o1.reshape(6, C)
    assert np.all(d[:, [c for c in range(C) if c != 7]] == 0)
    assert np.allclose(d[:, 7], x[3].reshape(6, C)[:, 7], rtol=1e-5, atol=1e-6)


def test_compress_chain_within_exact_bound():
    x, w, b = _rand_group(T=50, C=40, seed=9)
    out = O.compress_chain_f32(x, w, b).astype(np.float64)
    ex = O.compress_exact(x, w, b)
    C = 40
    wr = np.tile(np.abs(w.astype(np.float64)).T[:, None, :], (1, 50, 1)).reshape(5, -1)
    mag = np.abs(np.tile(b, 50)).astype(np.float64) + (wr * np.abs(x)).sum(axis=0)
    assert np.all(np.abs(out - ex) <= 6 * 2.0 ** -24 * mag + 1e-30)


# ======================================================================================
# RoPE
# ======================================================================================

def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((16, 2, 128))
    y = O.rope_rotate(x, np.zeros(16), np.zeros(16), 3, (44, 42, 42), 16, 4)
    assert np.array_equal(x, y)
    y1 = O.rope_rotate(x[:1], [0], [0], 1, (128, 0, 0), 16, 4)
    assert np.array_equal(x[:1], y1)


def test_rope_closed_form_pair():
    """Unit vector on pair i at 1D position p turns by p * theta^(-2i/D)."""
    D = 64
    for i in (0, 1, 5, 31):
        x = np.zeros((1, 1, D))
        x[0, 0, 2 * i] = 1.0
        p_t, p_u, T = 3, 7, 16
        y = O.rope_rotate(x, [p_t], [p_u], 1, (D, 0, 0), T, 4)
        ang = (p_t * T + p_u) * 10000.0 ** (-2 * i / D)
        assert abs(y[0, 0, 2 * i] - math.cos(ang)) < 1e-13
        assert abs(y[0, 0, 2 * i + 1] - math.sin(ang)) < 1e-13
        assert np.count_nonzero(y) <= 2


def test_rope_3d_parts_use_their_axis():
    """3D split (44, 42, 42): t turns channels [0,44), the grid row [44,86), the grid column
    [86,128); each with its own part width in the frequency exponent."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 1, 128))
    gw = 8
    cases = [((5, 0), slice(0, 44)), ((0, 3 * gw), slice(44, 86)), ((0, 3), slice(86, 128))]
    for (t, u), changed in cases:
        y = O.rope_rotate(x, [t], [u], 3, (44, 42, 42), 64, gw)
        mask = np.zeros(128, bool)
        mask[changed] = True
        assert np.array_equal(y[0, 0, ~mask], x[0, 0, ~mask])
        assert not np.allclose(y[0, 0, mask], x[0, 0, mask])
    # frequency of the first pair of the column part: angle = w * theta^0 = w
    e = np.zeros((1, 1, 128))
    e[0, 0, 86] = 1
    y = O.rope_rotate(e, [0], [2], 3, (44, 42, 42), 64, gw)
    assert abs(y[0, 0, 86] - math.cos(2)) < 1e-13 and abs(y[0, 0, 87] - math.sin(2)) < 1e-13
    # second pair of the row part: angle = h * theta^(-2/42)
    e = np.zeros((1, 1, 128))
    e[0, 0, 46] = 1
    y = O.rope_rotate(e, [0], [3 * gw], 3, (44, 42, 42), 64, gw)
    a = 3 * 10000.0 ** (-2 / 42)
    assert abs(y[0, 0, 46] - math.cos(a)) < 1e-13 and abs(y[0, 0, 47] - math.sin(a)) < 1e-13


def test_rope_norm_and_relative_position():
    """Rotations keep each pair's norm; q.k after rotation depends on position differences
    only, so a common shift of every position changes no score."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((10, 1, 128))
    k = rng.standard_normal((10, 1, 128))
    tq, uq = rng.integers(0, 30, 10), rng.integers(0, 64, 10)
    tk, uk = rng.integers(0, 30, 10), rng.integers(0, 64, 10)
    for mode, split in ((3, (44, 42, 42)), (1, (128, 0, 0))):
        qr = O.rope_rotate(q, tq, uq, mode, split, 64, 8)
        kr = O.rope_rotate(k, tk, uk, mode, split, 64, 8)
        assert np.allclose((qr ** 2).reshape(10, 64, 2).sum(-1), (q ** 2).reshape(10, 64, 2).sum(-1))
        qs = O.rope_rotate(q, tq + 7, uq, mode, split, 64, 8)
        ks = O.rope_rotate(k, tk + 7, uk, mode, split, 64, 8)
        s0 = qr[:, 0] @ kr[:, 0].T
        s1 = qs[:, 0] @ ks[:, 0].T
        assert np.allclose(s0, s1, atol=1e-11)


# ======================================================================================
# attention
# ======================================================================================

def _tiny_attn_inputs(seed, n_frames, hist_frames, H=2, D=64, gh=2, gw=3, scale=1.0):
    T = gh * gw
    rng = np.random.default_rng(seed)
    Lq, Lh = n_frames * T, hist_frames * T
    q = (rng.standard_normal((Lq, H, D)) * scale).astype(np.float32)
    kc = rng.standard_normal((Lq, H, D)).astype(np.float32)
    vc = rng.standard_normal((Lq, H, D)).astype(np.float32)
    kh = rng.standard_normal((Lh, H, D)).astype(np.float32) if Lh else None
    vh = rng.standard_normal((Lh, H, D)).astype(np.float32) if Lh else None
    ht = np.repeat(np.arange(hist_frames), T).astype(np.int32)
    hu = np.tile(np.arange(T), hist_frames).astype(np.int32)
    ct = np.repeat(np.arange(n_frames) + hist_frames, T).astype(np.int32)
    cu = np.tile(np.arange(T), n_frames).astype(np.int32)
    return dict(q=q, k_cur=kc, v_cur=vc, k_hist=kh, v_hist=vh, hist_t=ht, hist_u=hu,
                cur_t=ct, cur_u=cu, T=T, grid_w=gw)


def _attn(inp, blocks, form, mode=3, split=(22, 22, 20), **kw):
    return O.attention(inp["q"], inp["k_cur"], inp["v_cur"], inp["k_hist"], inp["v_hist"],
                       inp["hist_t"], inp["hist_u"], inp["cur_t"], inp["cur_u"], blocks,
                       inp["T"], mode, split, inp["grid_w"], **kw)


@pytest.mark.parametrize("blocks", [[3], [1, 2], [1, 1, 1], [2, 1]])
def test_attention_bruteforce_equals_segments(blocks):
    inp = _tiny_attn_inputs(10, sum(blocks), 4)
    o0, l0, _, _ = _attn(inp, blocks, 0)
    o1, l1, _, _ = _attn(inp, blocks, 1)
    assert np.allclose(o0, o1, atol=1e-12, rtol=0)
    assert np.allclose(l0, l1, atol=1e-12, rtol=0)


def test_attention_single_key_returns_value():
    """One key (T = 1, one current frame, no history): O = v and LSE = the score."""
    inp = _tiny_attn_inputs(11, 1, 0, gh=1, gw=1)
    o, lse, _, _ = _attn(inp, [1], 1, mode=1, split=(64, 0, 0))
    v = inp["v_cur"][0].astype(np.float64)
    assert np.allclose(o, v, atol=1e-14)
    q, k = inp["q"][0].astype(np.float64), inp["k_cur"][0].astype(np.float64)
    # same position for q and k: the rotation cancels in the score
    assert np.allclose(lse, (q * k).sum(-1) / 8.0, atol=1e-12)


def test_attention_zero_query_is_mean_of_visible_values():
    blocks = [1, 2]
    inp = _tiny_attn_inputs(12, 3, 2, scale=0.0)
    o, lse, heads, rows = _attn(inp, blocks, 1)
    T = inp["T"]
    vh, vc = inp["v_hist"].astype(np.float64), inp["v_cur"].astype(np.float64)
    for n, (h, i) in enumerate(zip(heads, rows)):
        blk = 0 if i < T else 1
        vis = np.concatenate([vh[:, h], vc[: (1 if blk == 0 else 3) * T, h]])
        assert np.allclose(o[n], vis.mean(0), atol=1e-13)
        assert abs(lse[n] - math.log(len(vis))) < 1e-12


def test_attention_equal_keys_is_mean():
    inp = _tiny_attn_inputs(13, 2, 1)
    kk = inp["k_cur"][0:1].copy()
    inp["k_cur"][:] = kk
    inp["k_hist"][:] = kk
    # equal keys at equal positions: make every position 0 so rotations agree
    for key in ("hist_t", "hist_u", "cur_t", "cur_u"):
        inp[key][:] = 0
    o, _, heads, rows = _attn(inp, [2], 1)
    vall = np.concatenate([inp["v_hist"], inp["v_cur"]]).astype(np.float64)
    for n, h in enumerate(heads):
        assert np.allclose(o[n], vall[:, h].mean(0), atol=1e-12)


def test_attention_mask_equals_truncated_context():
    """Rows of block 0 of a 2-block call equal a 1-block call with only block 0 present:
    later blocks are invisible to them; the last block sees everything."""
    inp = _tiny_attn_inputs(14, 3, 2)
    T = inp["T"]
    o_full, l_full, heads, rows = _attn(inp, [1, 2], 0)
    sub = dict(inp)
    for key in ("q", "k_cur", "v_cur", "cur_t", "cur_u"):
        sub[key] = inp[key][:T]
    o_sub, l_sub, h2, r2 = _attn(sub, [1], 1)
    sel = rows < T
    assert np.array_equal(heads[sel], h2) and np.array_equal(rows[sel], r2)
    assert np.allclose(o_full[sel], o_sub, atol=1e-12)
    o_one, _, _, _ = _attn(inp, [3], 1)
    last = rows >= T
    assert np.allclose(o_full[last], o_one[last], atol=1e-12)
    assert not np.allclose(o_full[sel], o_one[sel], atol=1e-6)


def test_attention_permuting_history_frames():
    """Moving history frames around together with their positions changes nothing."""
    inp = _tiny_attn_inputs(15, 1, 4)
    T = inp["T"]
    o0, _, _, _ = _attn(inp, [1], 1)
    perm = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(p * T, (p + 1) * T) for p in perm])
    p = dict(inp)
    for key in ("k_hist", "v_hist", "hist_t", "hist_u"):
        p[key] = inp[key][idx]
    o1, _, _, _ = _attn(p, [1], 1)
    assert np.allclose(o0, o1, atol=1e-12)


def test_attention_two_key_hand_example():
    """D = 2, T = 1: one history key at position 0 and the current token at 1D position 1;
    scores by hand: s_hist = (R(1) q) . k_h / sqrt 2, s_cur = q . k_c / sqrt 2."""
    q = np.array([[[0.5, -1.0]]], np.float32)
    kc = np.array([[[1.0, 2.0]]], np.float32)
    vc = np.array([[[3.0, -1.0]]], np.float32)
    kh = np.array([[[-0.5, 1.5]]], np.float32)
    vh = np.array([[[0.25, 4.0]]], np.float32)
    o, lse, _, _ = O.attention(q, kc, vc, kh, vh, [0], [0], [1], [0], [1], 1, 1, (2, 0, 0), 1)
    c, s = math.cos(1.0), math.sin(1.0)
    rq = (0.5 * c + 1.0 * s, 0.5 * s - 1.0 * c)
    s_h = (rq[0] * -0.5 + rq[1] * 1.5) / math.sqrt(2)
    s_c = (0.5 * 1.0 + -1.0 * 2.0) / math.sqrt(2)
    m = max(s_h, s_c)
    eh, ec = math.exp(s_h - m), math.exp(s_c - m)
    want = [(eh * 0.25 + ec * 3.0) / (eh + ec), (eh * 4.0 + ec * -1.0) / (eh + ec)]
    assert np.allclose(o[0], want, atol=1e-14)
    assert abs(lse[0] - (m + math.log(eh + ec))) < 1e-14


def test_attention_lse_normalises():
    inp = _tiny_attn_inputs(16, 2, 2)
    o, lse, heads, rows = _attn(inp, [2], 1, mode=1, split=(64, 0, 0))
    T = inp["T"]
    qr = O.rope_rotate(inp["q"], inp["cur_t"], inp["cur_u"], 1, (64,), T, inp["grid_w"])
    kr = np.concatenate([
        O.rope_rotate(inp["k_hist"], inp["hist_t"], inp["hist_u"], 1, (64,), T, inp["grid_w"]),
        O.rope_rotate(inp["k_cur"], inp["cur_t"], inp["cur_u"], 1, (64,), T, inp["grid_w"])])
    for n, (h, i) in enumerate(zip(heads, rows)):
        s = kr[:, h] @ qr[i, h] / 8.0
        assert abs(np.exp(s - lse[n]).sum() - 1.0) < 1e-12


# ======================================================================================
# bookkeeping and streaming
# ======================================================================================

def _run_schedule(W, M, r, first, block, steps):
    bk = Bookkeeping(W, M, r, max(first, block))
    rows = []
    for s in range(1, steps + 1):
        n = first if s == 1 else block
        st = bk.state()
        keys = bk.keys(n)
        rows.append([s, st["F"], st["E"], st["G"], st["pending"], st["mem_len"], st["win_len"],
                     len(keys)])
        bk.append(n)
        rows[-1].append(len(bk.compress()))
    return rows


@pytest.mark.parametrize("name", ["s512", "s720", "tiny"])
def test_schedule_golden(name):
    g = load("schedule.json")["workloads"][name]
    want = {r[0]: r for r in g["rows"]}
    got = _run_schedule(g["W"], g["M"], g["r"], g["first_block"], g["block"], max(want))
    for row in got:
        if row[0] in want:
            assert row == want[row[0]], (row, want[row[0]])


def test_schedule_closed_form_1000_steps():
    """F, E = max(0, F - W), G = floor(E / r), pending = E mod r, mem = min(G, M): memory
    stays at M once full, key frames stay constant and reset positions stay < M + W + B."""
    W, M, r, B = 8, 16, 5, 8
    bk = Bookkeeping(W, M, r, B)
    pend = []
    for s in range(1, 1001):
        F = B * (s - 1)
        E = max(0, F - W)
        st = bk.state()
        assert (st["F"], st["E"], st["G"], st["pending"], st["mem_len"]) == \
            (F, E, E // r, E % r, min(E // r, M))
        keys = bk.keys(B)
        assert all(k["t_pos"] < M + W + B for k in keys)
        if s >= 12:
            assert len(keys) == 32 and st["mem_len"] == M
        live = list(range(r * bk.G, bk.F))
        slots = [bk.raw_slot(f) for f in live]
        assert len(set(slots)) == len(slots)      # no raw slot holds two live frames
        pend.append(st["pending"])
        bk.append(B)
        bk.compress()
        # the new block plus window plus pending never exceeds the raw ring
        assert bk.F - r * bk.G <= bk.R
    assert pend[1:7] == [0, 3, 1, 4, 2, 0]


def test_first_two_blocks_uncompressed():
    """W = B: blocks 1 and 2 see no memory; block 3 is the first with a memory slot."""
    bk = Bookkeeping(8, 16, 5, 8)
    mems = []
    for _ in range(4):
        mems.append(bk.mem_len)
        bk.append(8)
        bk.compress()
    assert mems == [0, 0, 1, 3]


def test_bookkeeping_errors():
    bk = Bookkeeping(4, 10, 5, 2)
    with pytest.raises(OracleCapacityError):
        bk.append(3)
    with pytest.raises(OracleCapacityError):
        bk.append(0)
    for _ in range(5):
        bk.append(2)          # F = 10, E = 6: one complete group waits
    with pytest.raises(OracleStateError):
        bk.append(2)
    assert bk.compress() == [0]
    bk.append(2)


def test_window_only_positions_are_absolute():
    """M = 0 (motion-frame overlap: keep the last frames, drop the rest): the window's
    reset positions are the absolute positions shifted by a constant, and by the relative
    property of RoPE the scores equal those at absolute positions."""
    bk = Bookkeeping(4, 0, 5, 2)
    for _ in range(9):
        bk.append(2)
        bk.compress()
    keys = bk.keys(2)
    shift = {k["id"] - k["t_pos"] for k in keys}
    assert len(shift) == 1


def _tag_stream(kernel_tap):
    cfg = synth.workload("tiny_f32")
    oc = OracleCache(cfg)
    T, C = cfg["tokens"], cfg["channels"]
    w = np.zeros((C, 5), np.float32)
    if kernel_tap is None:
        w[:] = np.float32(0.2)
    else:
        w[:, kernel_tap] = 1.0
    b = np.zeros(C, np.float32)
    rng = np.random.default_rng(0)
    for blk in range(40):
        k = rng.standard_normal((2, T * C)).astype(np.float32)
        for i in range(2):
            k[i, 0] = 2 * blk + i          # frame-id tag
        oc.append(k, k.copy())
        oc.compress(w, b, w, b)
    return oc


@pytest.mark.parametrize("tap", [0, 2, 4])
def test_stream_frame_id_tag_delta(tap):
    oc = _tag_stream(tap)
    for slot, (g, sk, _) in oc.mem.items():
        assert slot == g % 10
        assert sk[1][0] == 5 * g + tap


def test_stream_frame_id_tag_uniform():
    oc = _tag_stream(None)
    for slot, (g, sk, _) in oc.mem.items():
        assert abs(sk[1][0] - (5 * g + 2)) <= 1e-5 * (5 * g + 2)


def test_stream_at_state_equals_sequential_stream():
    """Building the cache state at frame F directly equals streaming to F block by block
    (non-recursive FIFO memory: each slot comes from its own r frames only)."""
    cfg = synth.workload("tiny_f32", pool_blocks=3)
    T, C = cfg["tokens"], cfg["channels"]
    wk, bk = synth.conv_weights(cfg, 0, synth.TENSOR_WK)
    wv, bv = synth.conv_weights(cfg, 0, synth.TENSOR_WV)

    def frame_kv(f):
        return (synth.frames(cfg, 0, synth.TENSOR_K, [f])[0], synth.frames(cfg, 0, synth.TENSOR_V, [f])[0])

    seq = OracleCache(cfg)
    for step in range(40):
        ks = np.stack([frame_kv(seq.bk.F + i)[0] for i in range(2)])
        vs = np.stack([frame_kv(seq.bk.F + i)[1] for i in range(2)])
        seq.append(ks, vs)
        seq.compress(wk, bk, wv, bv)
        if step in (3, 17, 39):
            ff = OracleCache.at_state(cfg, seq.bk.F, frame_kv, wk, bk, wv, bv)
            assert ff.bk.state() == {**seq.bk.state(), "version": ff.bk.version}
            assert sorted(ff.mem) == sorted(seq.mem)
            for slot in seq.mem:
                assert ff.mem[slot][0] == seq.mem[slot][0]
                assert np.array_equal(ff.mem[slot][1][1], seq.mem[slot][1][1])
                assert np.array_equal(ff.mem[slot][2][1], seq.mem[slot][2][1])
            for f in range(seq.bk.E, seq.bk.F):
                assert np.array_equal(ff.raw[f][0][1], seq.raw[f][0][1])


# ---- reference segment -------------------------------------------------------------------

def test_reference_keys_hand_table():
    """Reference segment of 2 frames, window 4, memory 10 at 5:1, blocks of 2: after 27
    blocks (54 frames appended, 50 evicted, groups 0..9 compressed) the key table of a
    2-frame block, written out by hand."""
    bk = Bookkeeping(4, 10, 5, 2, ref_frames=2)
    for _ in range(27):
        bk.append(2)
        bk.compress()
    got = [(k["segment"], k["slot"], k["id"], k["t_pos"]) for k in bk.keys(2)]
    want = ([(3, 0, 0, 0), (3, 1, 1, 1)] +
            [(0, g, g, 2 + g) for g in range(10)] +
            [(1, 0, 50, 12), (1, 1, 51, 13), (1, 2, 52, 14), (1, 3, 53, 15)] +   # R = 10 slots
            [(2, 0, 54, 16), (2, 1, 55, 17)])
    assert got == want


def test_reference_positions_fixed_and_bounded():
    """Over 1000 steps the reference frames keep positions 0 and 1, come first, and every
    position stays below ref + M + W + B_max."""
    bk = Bookkeeping(8, 16, 5, 8, ref_frames=2)
    for _ in range(1000):
        keys = bk.keys(8)
        assert [(k["segment"], k["t_pos"]) for k in keys[:2]] == [(3, 0), (3, 1)]
        assert all(k["segment"] != 3 for k in keys[2:])
        assert max(k["t_pos"] for k in keys) < 2 + 16 + 8 + 8
        bk.append(8)
        bk.compress()


def test_reference_zero_query_is_mean_of_visible_values():
    """Closed form with a reference segment: q = 0 makes every visible score equal, so each
    row's output is the plain mean of the V rows it sees -- both reference frames, the
    window and the block frames up to its own -- and its LSE is log(count).  Window-only
    memory (M = 0) keeps every stored value equal to its input."""
    w = synth.workload("tiny_f32", ref_frames=2, mem_slots=0, window_frames=3, max_block_frames=3)
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    oc = OracleCache(w)
    rng = np.random.default_rng(5)
    kr, vr = (rng.standard_normal((2, T * H * D)).astype(np.float32) for _ in range(2))
    oc.set_ref(kr, vr)
    frames_v = {}
    for f0 in (0, 2, 4):                      # 6 frames appended; window = frames 3..5
        k = rng.standard_normal((2, T * H * D)).astype(np.float32)
        v = rng.standard_normal((2, T * H * D)).astype(np.float32)
        for i in range(2):
            frames_v[f0 + i] = v[i]
        oc.append(k, v)
        zw, zb = np.zeros((H * D, 5), np.float32), np.zeros(H * D, np.float32)
        oc.compress(zw, zb, zw, zb)           # M = 0: evicted groups are dropped
    q = np.zeros((3 * T, H, D), np.float32)
    kc = rng.standard_normal((3 * T, H, D)).astype(np.float32)
    vc = rng.standard_normal((3 * T, H, D)).astype(np.float32)
    O_, LSE, heads, rows = oc.attention(q, kc, vc, block_frames=[1, 2])
    hist_v = np.concatenate([vr.reshape(2 * T, H, D)] +
                            [frames_v[f].reshape(T, H, D) for f in (3, 4, 5)])
    for blk, n_cur in ((0, 1), (1, 3)):
        visible = np.concatenate([hist_v, vc[: n_cur * T]]).astype(np.float64)
        mean = visible.mean(axis=0)                       # [H][D]
        sel = np.where((rows >= (0 if blk == 0 else T)) & (rows < (T if blk == 0 else 3 * T)))[0]
        for i in sel:
            np.testing.assert_allclose(O_[i], mean[heads[i]], rtol=0, atol=1e-12)
            assert abs(LSE[i] - math.log(visible.shape[0])) < 1e-12


# ---- the per-row size of the weighted terms (used by the per-row parity bounds) ---------

def test_attention_rms_closed_forms():
    """RMS = sqrt(sum_j w_j^2 |v_j|^2): one visible key gives |v|; a zero query gives
    uniform weights 1/N over the visible keys, so RMS = sqrt(sum |v_j|^2) / N; the two-key
    hand example gives sqrt(w_h^2 |v_h|^2 + w_c^2 |v_c|^2) with its hand-worked weights."""
    inp = _tiny_attn_inputs(11, 1, 0, gh=1, gw=1)
    _, _, _, _, rms = _attn(inp, [1], 1, mode=1, split=(64, 0, 0), want_rms=True)
    assert np.allclose(rms, np.linalg.norm(inp["v_cur"][0].astype(np.float64), axis=-1), rtol=1e-13)

    blocks = [1, 2]
    inp = _tiny_attn_inputs(12, 3, 2, scale=0.0)
    _, _, heads, rows, rms = _attn(inp, blocks, 0, want_rms=True)
    T = inp["T"]
    vh, vc = inp["v_hist"].astype(np.float64), inp["v_cur"].astype(np.float64)
    for n, (h, i) in enumerate(zip(heads, rows)):
        vis = np.concatenate([vh[:, h], vc[: (1 if i < T else 3) * T, h]])
        want = math.sqrt((vis ** 2).sum()) / len(vis)
        assert abs(rms[n] - want) <= 1e-13 * want

    q = np.array([[[0.5, -1.0]]], np.float32)
    kc = np.array([[[1.0, 2.0]]], np.float32)
    vc = np.array([[[3.0, -1.0]]], np.float32)
    kh = np.array([[[-0.5, 1.5]]], np.float32)
    vh = np.array([[[0.25, 4.0]]], np.float32)
    _, _, _, _, rms = O.attention(q, kc, vc, kh, vh, [0], [0], [1], [0], [1], 1, 1, (2, 0, 0), 1,
                                  want_rms=True)
    c, s_ = math.cos(1.0), math.sin(1.0)
    rq = (0.5 * c + 1.0 * s_, 0.5 * s_ - 1.0 * c)
    s_h = (rq[0] * -0.5 + rq[1] * 1.5) / math.sqrt(2)
    s_c = (0.5 * 1.0 + -1.0 * 2.0) / math.sqrt(2)
    eh, ec = math.exp(s_h), math.exp(s_c)
    wh, wc = eh / (eh + ec), ec / (eh + ec)
    want = math.sqrt(wh ** 2 * (0.25 ** 2 + 4.0 ** 2) + wc ** 2 * (3.0 ** 2 + 1.0))
    assert abs(rms[0] - want) < 1e-14 * want


def test_attention_rms_does_not_change_o_or_lse():
    inp = _tiny_attn_inputs(16, 2, 2)
    o1, l1, _, _ = _attn(inp, [1, 1], 1)
    o2, l2, _, _, _ = _attn(inp, [1, 1], 1, want_rms=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
