"""Long-run streaming on the GPU: 1000 consecutive AR steps at 512x512 shapes with rolling
eviction -> compression -> ring append.  Every step: the cache state and key-frame table
equal the oracle's bookkeeping bit for bit, reset positions stay below M + W + B_max, and
no device memory is allocated (the footprint is the one buffer).  At steps 1, 2, 3, 12,
13, 500 and 1000 the attention output is compared with the oracle on sampled rows."""
import numpy as np
import pytest
import torch

import compressed_kv_causal_amd as L
import synth
from oracle.bookkeeping import Bookkeeping
from oracle.stream import OracleCache
from stream_helpers import BF16, check_heads_and_rows, pair_norm_max, rel_l2, row_bounds, sample_rows

pytestmark = pytest.mark.gpu

CHECK_STEPS = {1, 2, 3, 12, 13, 500, 1000}


def test_long_run_1000_steps():
    w = synth.workload("long_run")
    T, H, D, B = w["tokens"], w["heads"], w["head_dim"], w["block"]
    pool_blocks = w["pool_blocks"]
    # the pool: block n of the stream uses pool block n mod 7 (frame ids f mod 56)
    pool = []
    host = []
    for blk in range(pool_blocks):
        ids = list(range(blk * B, (blk + 1) * B))
        trip_d, trip_h = [], []
        for tensor in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V):
            x = torch.from_numpy(synth.frames(w, 0, tensor, ids).reshape(B * T, H, D)).to(torch.bfloat16)
            trip_d.append(x.cuda())
            trip_h.append(x.float().numpy())
        pool.append(trip_d)
        host.append(trip_h)
    wk, bk = synth.conv_weights(w, 0, synth.TENSOR_WK)
    wv, bv = synth.conv_weights(w, 0, synth.TENSOR_WV)
    d_w = [torch.from_numpy(a).cuda() for a in (wk, bk, wv, bv)]

    def frame_kv(f):
        blk, i = (f // B) % pool_blocks, f % B
        return (host[blk][1].reshape(B, -1)[i], host[blk][2].reshape(B, -1)[i])

    cache = L.Cache(L.make_cfg(**w))
    footprint = cache.nbytes
    bkp = Bookkeeping(w["window_frames"], w["mem_slots"], w["ratio"], B)
    KF = w["mem_slots"] + w["window_frames"] + B
    out = torch.empty((B * T, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, B * T), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    allocated = torch.cuda.memory_allocated()
    errs = {}
    for step in range(1, 1001):
        q, k, v = pool[(step - 1) % pool_blocks]
        keys = cache.keys(B)
        want = bkp.keys(B)
        assert [(x["segment"], x["slot"], x["id"], x["t_pos"]) for x in keys] == \
               [(x["segment"], x["slot"], x["id"], x["t_pos"]) for x in want], step
        assert max(x["t_pos"] for x in keys) < KF
        if step >= 12:
            assert len(keys) == KF
        L.lact_rope_reset_apply(cache.h, q, k, v, B)
        L.lact_block_attention(cache.h, None, out, lse)
        if step in CHECK_STEPS:
            oc = OracleCache.at_state(w, bkp.F, frame_kv, wk, bk, wv, bv)
            qh, kh, vh = host[(step - 1) % pool_blocks]
            sel = sample_rows(w, B, seed=step, per_head=2)
            O, LSE, heads, rows, rms = oc.attention(qh, kh, vh, sel=sel, want_rms=True)
            got = out.float().cpu().numpy()[rows, heads]
            errs[step] = rel_l2(got, O)
            dl = float(np.abs(lse.cpu().numpy()[heads, rows] - LSE).max())
            kh_hist = oc.history()[0]
            kpair = pair_norm_max(kh) if kh_hist is None else \
                np.maximum(pair_norm_max(kh), pair_norm_max(kh_hist))
            qn = np.linalg.norm(qh[rows, heads].astype(np.float64), axis=1)
            b = row_bounds(O, rms, qn, kpair, heads, BF16, D)
            wh, wr = check_heads_and_rows(got, O, heads, BF16, b, label=f"long run step {step}")
            print(f"step {step}: rel L2 {errs[step]:.3e}, worst head {wh:.3e}, worst row / bound "
                  f"{wr:.3f}, max dLSE {dl:.2e}", flush=True)
            assert errs[step] <= 1e-2 and dl <= 2e-2
        L.lact_kv_ring_append(cache.h, k, v, B)
        L.lact_convkv_compress(cache.h, *d_w)
        bkp.append(B)
        bkp.compress()
        st = cache.state()
        ob = bkp.state()
        assert (st["F"], st["E"], st["G"], st["pending"], st["mem_len"], st["win_len"]) == \
               (ob["F"], ob["E"], ob["G"], ob["pending"], ob["mem_len"], ob["win_len"]), step
        if step % 100 == 0:
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated() == allocated
            print(f"step {step}: state F={st['F']} G={st['G']} mem {st['mem_len']}", flush=True)
    assert L.lact_cache_footprint(cache.cfg) == footprint
    assert set(errs) == CHECK_STEPS
