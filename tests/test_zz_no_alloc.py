"""The allocation-free attention entry point (lact_member_block_attention_static) against
lact_member_block_attention: same kernels, so the outputs and LSE must be bit-identical;
two calls in a row, the second with a smaller input, and its capacity refusal."""
import numpy as np
import pytest
import torch

import compressed_kv_causal_amd as L
import synth
from stream_helpers import Runner

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _filled(w, blocks):
    run = Runner(w, with_oracle=False)
    for _ in range(blocks):
        run.step(w["block"], attend=False)
    return run


def _both(run, n, blocks=None):
    """Stages n frames, then attention through both entry points; returns both results."""
    (q, _), (k, _), (v, _) = run.inputs(n)
    run.cache.rope_reset_apply(q, k, v, member=run.member)
    Lq = n * run.T
    lse_a = torch.empty((run.H, Lq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    a = run.cache.block_attention(blocks, lse=lse_a, member=run.member)
    b = run.cache.block_attention_static(blocks, lse=lse_b, member=run.member)
    torch.cuda.synchronize()
    return a, lse_a, b, lse_b


@pytest.mark.parametrize("name,over", [
    ("s512_bf16", dict(grid_h=16, grid_w=16, heads=8)),        # D = 128 kernel + its exact pass
    ("s512_bf16", dict(grid_h=16, grid_w=16, heads=8, head_dim=64, rope_split=(22, 22, 20))),
    ("fp8_kv", dict(grid_h=16, grid_w=16, heads=8)),
])
def test_static_queue_matches_cache_queue(name, over):
    w = synth.workload(name, **over)
    say(f"static-queue attention: {name} {over}")
    run = _filled(w, 11)
    for n, blocks in ((8, None), (3, [1, 2])):               # second call: a smaller input
        a, la, b, lb = _both(run, n, blocks)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), n
        assert torch.isfinite(a.float()).all()


def test_static_queue_refuses_oversized_calls():
    """heads x 256-row tiles beyond LACT_STATIC_QUEUE_MAX is refused before any launch."""
    w = synth.workload("s512_bf16", heads=64, head_dim=64, rope_split=(22, 22, 20), grid_h=32,
                       grid_w=32, window_frames=0, mem_slots=0, max_block_frames=65)
    say("static-queue attention: capacity refusal")
    run = Runner(w, with_oracle=False)
    g = torch.Generator(device="cuda").manual_seed(0)
    q, k, v = (torch.randn((65 * 1024, 64, 64), generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    run.cache.rope_reset_apply(q, k, v)
    items = 64 * ((65 * 1024 + 255) // 256)
    assert items > L.LACT_STATIC_QUEUE_MAX
    with pytest.raises(L.LactError) as ei:
        run.cache.block_attention_static()
    assert ei.value.status == 3 and "LACT_STATIC_QUEUE_MAX" in str(ei.value)
    st = run.cache.state()
    assert st["staged_valid"] == 1            # the refused call changed nothing
    torch.cuda.synchronize()
