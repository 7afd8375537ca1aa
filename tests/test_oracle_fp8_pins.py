"""Pins of the oracle's FP8 storage path (the model card's FP8 KV cache: K and V kept as
e4m3 codes with one f32 scale per (token, head), dequantised on use).

What is pinned, each against something other than the function under test:
  * the dequantiser against the E4M3FN closed form times the row's scale, for every code
    and a spread of scales, with the scale indexed per row;
  * the attention's scale arguments: a call on (code values, scales) equals the call on
    the products when those are exact in f32 (power-of-two scales), with K, V, Q and the
    block's own scales all distinct, so a swapped or mis-indexed scale changes the result;
  * the FP8 compressor through the streaming cache (news summary, ConvKV Memory bullet:
    1D convolution at 5:1): a delta kernel at tap k stores exactly the codes of frame
    r*g + k and the scale the closed form below gives; the uniform kernel 1/5 stores the
    5-frame mean of the stored values within e4m3's rounding bound;
  * the FP8 cache's attention equals attention over the dequantised values.
"""
import math

import numpy as np
import pytest

import oracle as O
import synth
from oracle.stream import OracleCache


def e4m3_closed_form(code):
    """(-1)^s 2^(e-7) (1 + m/8), or (m/8) 2^-6 for e = 0; NaN for S.1111.111."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


CODE_VALUES = np.array([e4m3_closed_form(c) for c in range(256)])
FINITE_CODES = np.array([c for c in range(256) if not math.isnan(CODE_VALUES[c])], np.uint8)


# ======================================================================================
# dequantiser
# ======================================================================================

def test_dequant_every_code_times_its_row_scale():
    """Row r of every code (a different rotation of 0..255 in each row) times scales[r]:
    one exact product (a code value has 4 significant bits, a scale 24) rounded to f32."""
    D = 256
    scales = np.array([1.0, 2.0 ** -7, 0.013671875, 3.0e-3, 7.5, 1.0e-20, 448.0 / 3.0, 0.1],
                      np.float32)
    rows = scales.size
    codes = np.stack([np.roll(np.arange(256, dtype=np.uint8), 37 * r) for r in range(rows)])
    got = O.e4m3_dequant_f32(codes, scales, D)
    want = np.float32(CODE_VALUES[codes] * scales.astype(np.float64)[:, None])
    nan = np.isnan(CODE_VALUES[codes])
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # each row used its own scale: the ratio to the code value is that row's scale
    for r in range(rows):
        sel = (~nan[r]) & (CODE_VALUES[codes[r]] != 0)
        ratio = got[r, sel].astype(np.float64) / CODE_VALUES[codes[r, sel]]
        assert np.allclose(ratio, scales[r], rtol=2.0 ** -23, atol=0)


def test_dequant_inverts_the_row_quantiser():
    """Quantise rows (one scale per (token, head) row of D channels), dequantise: every
    element is within half an e4m3 step of its input, and the row's largest element comes
    back as fl32(448 * scale)."""
    D = 128
    rng = np.random.default_rng(20)
    x = rng.standard_normal((40, D)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 8
    x[7] *= 1e-3
    codes, scales = O.quant_e4m3_rows(x, D)
    deq = O.e4m3_dequant_f32(codes, scales, D).astype(np.float64)
    err = np.abs(deq - x)
    bound = np.abs(x) * 2.0 ** -4 + scales[:, None].astype(np.float64) * 2.0 ** -10
    assert np.all(err <= bound * (1 + 2.0 ** -20) + 1e-30)
    j = np.abs(x).argmax(axis=1)
    top = np.abs(deq[np.arange(40), j])
    assert np.array_equal(np.float32(top), np.float32(448.0 * scales.astype(np.float64)))


# ======================================================================================
# attention over scaled values
# ======================================================================================

def _scaled_inputs(seed, H=2, D=64, gh=2, gw=3, hist_frames=3, cur_frames=2):
    """e4m3 code values and distinct power-of-two scales per (token, head) for q, k_hist,
    v_hist, k_cur, v_cur; the products are exact in f32."""
    T = gh * gw
    rng = np.random.default_rng(seed)

    def codes(n):
        c = rng.choice(FINITE_CODES, size=(n, H, D))
        # keep magnitudes moderate (|value| <= 8) so scores stay in a useful range
        vals = CODE_VALUES[c]
        vals = np.where(np.abs(vals) > 8, np.sign(vals) * 1.5, vals)
        return vals.astype(np.float32)

    def scales(n, lo, hi):
        return np.float32(2.0 ** rng.integers(lo, hi, size=(n, H)))

    Lh, Lq = hist_frames * T, cur_frames * T
    d = dict(T=T, grid_w=gw)
    d["q"], d["q_s"] = codes(Lq), scales(Lq, -4, -1)
    d["k_hist"], d["k_hist_s"] = codes(Lh), scales(Lh, -5, -2)
    d["v_hist"], d["v_hist_s"] = codes(Lh), scales(Lh, -2, 3)
    d["k_cur"], d["k_cur_s"] = codes(Lq), scales(Lq, -3, 0)
    d["v_cur"], d["v_cur_s"] = codes(Lq), scales(Lq, 0, 4)
    d["hist_t"] = np.repeat(np.arange(hist_frames), T).astype(np.int32)
    d["hist_u"] = np.tile(np.arange(T), hist_frames).astype(np.int32)
    d["cur_t"] = np.repeat(np.arange(cur_frames) + hist_frames, T).astype(np.int32)
    d["cur_u"] = np.tile(np.arange(T), cur_frames).astype(np.int32)
    return d


def _call(d, scaled, blocks=(1, 1), **swap):
    names = ("q", "k_cur", "v_cur", "k_hist", "v_hist")
    if scaled:
        x = {n: d[n] for n in names}
        s = {n: d[swap.get(n, n) + "_s"] for n in names}
    else:
        x = {n: np.float32(d[n] * d[n + "_s"][..., None]) for n in names}
        s = {n: None for n in names}
    return O.attention(x["q"], x["k_cur"], x["v_cur"], x["k_hist"], x["v_hist"], d["hist_t"],
                       d["hist_u"], d["cur_t"], d["cur_u"], list(blocks), d["T"], 3, (22, 22, 20),
                       d["grid_w"], q_scale=s["q"], k_cur_scale=s["k_cur"],
                       v_cur_scale=s["v_cur"], k_hist_scale=s["k_hist"],
                       v_hist_scale=s["v_hist"])


@pytest.mark.parametrize("form", [0, 1])
def test_attention_scales_equal_premultiplied_values(form):
    """Both forms (explicit mask matrix, segments), two query blocks."""
    d = _scaled_inputs(21)
    o_s, l_s, h_s, r_s = _call_form(d, True, form)
    o_p, l_p, h_p, r_p = _call_form(d, False, form)
    assert np.array_equal(h_s, h_p) and np.array_equal(r_s, r_p)
    assert np.array_equal(o_s, o_p)
    assert np.array_equal(l_s, l_p)


def _call_form(d, scaled, form):
    names = ("q", "k_cur", "v_cur", "k_hist", "v_hist")
    x = {n: d[n] if scaled else np.float32(d[n] * d[n + "_s"][..., None]) for n in names}
    s = {n: d[n + "_s"] if scaled else None for n in names}
    return O.attention(x["q"], x["k_cur"], x["v_cur"], x["k_hist"], x["v_hist"], d["hist_t"],
                       d["hist_u"], d["cur_t"], d["cur_u"], [1, 1], d["T"], 3, (22, 22, 20),
                       d["grid_w"], form=form, q_scale=s["q"], k_cur_scale=s["k_cur"],
                       v_cur_scale=s["v_cur"], k_hist_scale=s["k_hist"],
                       v_hist_scale=s["v_hist"])


@pytest.mark.parametrize("a,b", [("k_hist", "v_hist"), ("k_cur", "v_cur"), ("q", "k_cur")])
def test_attention_swapped_scales_are_detected(a, b):
    """Giving one tensor's scales to another changes the output: the equality above is not
    an accident of equal scales."""
    d = _scaled_inputs(22)
    o_p, _, _, _ = _call(d, False)
    o_x, _, _, _ = _call(d, True, **{a: b, b: a})
    assert np.abs(o_x - o_p).max() > 1e-3


def test_attention_scales_non_power_of_two():
    """Arbitrary f32 scales: the scaled call equals the premultiplied one within the f32
    rounding of the products (the premultiplied values carry it, the scaled call does not)."""
    d = _scaled_inputs(23)
    rng = np.random.default_rng(24)
    for n in ("q", "k_hist", "v_hist", "k_cur", "v_cur"):
        d[n + "_s"] = np.float32(d[n + "_s"] * rng.uniform(1.0, 2.0, d[n + "_s"].shape))
    o_s, l_s, _, _ = _call(d, True)
    o_p, l_p, _, _ = _call(d, False)
    scale = np.abs(o_p).max()
    assert np.abs(o_s - o_p).max() <= 1e-5 * scale
    assert np.abs(l_s - l_p).max() <= 1e-5


# ======================================================================================
# the FP8 compressor through the streaming cache
# ======================================================================================

def _fp8_tiny(**over):
    return synth.workload("tiny_f32", kv_dtype=synth.FP8, q_dtype=synth.BF16, **over)


def _fp8_stream(w, blocks, weight_fn, seed=30):
    """Streams `blocks` blocks of 2 frames with outlier-laden K/V into an FP8 oracle cache;
    returns the cache and the stored (codes, scales) of every appended frame."""
    oc = OracleCache(w)
    T, C, D = w["tokens"], w["channels"], w["head_dim"]
    wk, wv = weight_fn(C)
    zb = np.zeros(C, np.float32)
    rng = np.random.default_rng(seed)
    stored = {}
    for _ in range(blocks):
        k = rng.standard_normal((2, T * C)).astype(np.float32)
        v = rng.standard_normal((2, T * C)).astype(np.float32)
        for x in (k, v):
            x[rng.random(x.shape) < 0.01] *= 8
        k[:, :D] *= 1e-2   # one row per frame far smaller than the rest
        placed = oc.append(k, v)
        for f, _slot in placed:
            sk, sv = oc.raw[f]
            assert sk[0] == "fp8" and sv[0] == "fp8"
            stored[f] = (sk[1].copy(), sk[2].copy(), sv[1].copy(), sv[2].copy())
        oc.compress(wk, zb, wv, zb)
    return oc, stored


def _requant_scale(s):
    """Scale the quantiser gives a row dequantised from scale s: its largest magnitude is
    fl32(448 s), so the new scale is fl32(fl32(448 s) / 448)."""
    s = np.asarray(s, np.float32)
    amax = np.float32(np.float32(448.0) * s)
    return np.float32(amax / np.float32(448.0))


@pytest.mark.parametrize("tap", [0, 3, 4])
def test_fp8_delta_kernel_keeps_codes(tap):
    w = _fp8_tiny()

    def weights(C):
        wt = np.zeros((C, 5), np.float32)
        wt[:, tap] = 1.0
        return wt, wt.copy()

    oc, stored = _fp8_stream(w, 40, weights)
    assert len(oc.mem) == 10
    for slot, (g, sk, sv) in oc.mem.items():
        assert slot == g % 10
        ck, sck, cv, scv = stored[5 * g + tap]
        assert np.array_equal(sk[1], ck) and np.array_equal(sv[1], cv)
        assert np.array_equal(sk[2], _requant_scale(sck))
        assert np.array_equal(sv[2], _requant_scale(scv))
        # the re-quantised scale is the frame's own scale or one of its f32 neighbours
        ulp = np.spacing(sck)
        assert np.all(np.abs(sk[2].astype(np.float64) - sck) <= ulp)


def test_fp8_uniform_kernel_is_mean_of_stored_values():
    """'Mean memory' (the uniform kernel 1/5): each slot holds the mean of the 5 frames'
    stored values, up to the chain's rounding, the rounding of 1/5 and e4m3's half step."""
    w = _fp8_tiny()
    D = w["head_dim"]

    def weights(C):
        wt = np.full((C, 5), np.float32(0.2), np.float32)
        return wt, wt.copy()

    oc, stored = _fp8_stream(w, 40, weights)
    tab = CODE_VALUES
    for slot, (g, sk, sv) in oc.mem.items():
        for which, s in ((0, sk), (2, sv)):
            frames = [stored[5 * g + k] for k in range(5)]
            vals = np.stack([tab[f[which]].reshape(-1, D) * f[which + 1].astype(np.float64)[:, None]
                             for f in frames])          # exact stored values [5][rows][D]
            mean = vals.mean(axis=0)
            got = tab[s[1]].reshape(-1, D) * s[2].astype(np.float64)[:, None]
            chain = 8 * 2.0 ** -24 * np.abs(vals).sum(axis=0) / 5
            e4m3 = np.abs(mean) * 2.0 ** -4 + s[2].astype(np.float64)[:, None] * 2.0 ** -10
            assert np.all(np.abs(got - mean) <= (chain + e4m3) * (1 + 1e-6) + 1e-30)


def test_fp8_cache_attention_equals_dequantised_values():
    """The FP8 cache's attention (code values + per-(token, head) scales in the oracle's
    attention) equals attention over the dequantised history passed as plain values."""
    w = _fp8_tiny(pool_blocks=3)
    T, H, D = w["tokens"], w["heads"], w["head_dim"]
    wk, bk = synth.conv_weights(w, 0, synth.TENSOR_WK)
    wv, bv = synth.conv_weights(w, 0, synth.TENSOR_WV)
    oc, _ = _fp8_stream(w, 30, lambda C: (wk, wv))
    rng = np.random.default_rng(31)
    q, kc, vc = (rng.standard_normal((2 * T, H, D)).astype(np.float32) for _ in range(3))
    o8, l8, heads, rows = oc.attention(q, kc, vc)
    kh, khs, vh, vhs, ht, hu = oc.history()
    assert khs.shape == kh.shape[:2] and vhs.shape == vh.shape[:2]
    kdeq = np.float32(kh.astype(np.float64) * khs[..., None])
    vdeq = np.float32(vh.astype(np.float64) * vhs[..., None])
    nh = len(oc.keys(0))
    cur_t = np.repeat(np.arange(2, dtype=np.int32) + nh, T)
    cur_u = np.tile(np.arange(T, dtype=np.int32), 2)
    c = oc.cfg
    op, lp, h2, r2 = O.attention(q, kc, vc, kdeq, vdeq, ht, hu, cur_t, cur_u, [2], T,
                                 c["rope_mode"], c["rope_split"], c["grid_w"], c["rope_theta"])
    assert np.array_equal(heads, h2) and np.array_equal(rows, r2)
    assert np.abs(o8 - op).max() <= 1e-5 * np.abs(op).max()
    assert np.abs(l8 - lp).max() <= 1e-5
