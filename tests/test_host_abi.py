"""Host-side tests of liblact.so (no GPU needed): exported symbols, sizing, configuration
checks, the C++ planner against the oracle's bookkeeping (bit-exact over 1000 steps for
every workload's schedule), and the error paths of the C ABI that fail before anything is
enqueued."""
import ctypes
import os
import re

import pytest
import torch

import compressed_kv_causal_amd as L
import synth
from oracle.bookkeeping import Bookkeeping, OracleCapacityError, OracleStateError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_declared_symbol_is_exported():
    with open(os.path.join(ROOT, "include", "lact.h")) as f:
        text = f.read()
    declared = set(re.findall(r"\b(lact_\w+)\s*\(", text))
    assert len(declared) >= 17
    lib = L.lib()
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in lact.h but not exported"
    assert declared == set(L.EXPORTS)


def _cfg(name="s512_bf16", **kw):
    return L.make_cfg(**synth.workload(name, **kw))


def test_footprint_is_pure_and_matches_layout():
    for name in synth.WORKLOADS:
        c = _cfg(name)
        a, b = L.lact_cache_footprint(c), L.lact_cache_footprint(c)
        assert a == b
        lay = L.lact_cache_layout(c)
        assert lay.total == a
        w = synth.workload(name)
        R = w["window_frames"] + w["max_block_frames"] + w["ratio"] - 1
        assert lay.ring_slots == R
        ref = w.get("ref_frames", 0)
        assert lay.key_frames_max == ref + w["mem_slots"] + w["window_frames"] + w["max_block_frames"]
        esize = {0: 4, 1: 2, 2: 1}[w["kv_dtype"]]
        assert lay.frame_bytes == w["tokens"] * w["channels"] * esize
        fp8 = w["kv_dtype"] == 2
        # persistent regions first (one member), then the staging
        names = ("ring_k", "ring_v", "mem_k", "mem_v", "ref_k", "ref_v") + \
            (("ring_k_scale", "ring_v_scale", "mem_k_scale", "mem_v_scale", "ref_k_scale",
              "ref_v_scale") if fp8 else ()) + ("krot", "qrot", "vcur", "vcur_scale", "vscale",
                                                "rope_table", "attn_flags", "vmax")
        offs = [getattr(lay, n) for n in names]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert lay.members == 1 and lay.krot == lay.member_bytes
        fb, M, W = lay.frame_bytes, w["mem_slots"], w["window_frames"]
        assert lay.mem_k - lay.ring_v >= fb * R and lay.ref_k - lay.mem_v >= fb * M
        # staged keys and queries are in the q dtype, the block's V in the kv dtype; FP8
        # adds every key's V row scale per head and the heads' exponent bounds
        ob = w["tokens"] * w["channels"] * {0: 4, 1: 2}[w["q_dtype"]]
        KF = lay.key_frames_max
        assert lay.qrot - lay.krot >= ob * KF and lay.vcur - lay.qrot >= ob * w["max_block_frames"]
        assert lay.vcur_scale - lay.vcur >= fb * w["max_block_frames"]
        if fp8:
            assert lay.vscale - lay.vcur_scale >= w["tokens"] * w["heads"] * 4 * w["max_block_frames"]
            assert lay.rope_table - lay.vscale >= 3 * 4 * w["heads"] * (KF * w["tokens"] + 64)
            assert lay.total - lay.vmax >= 4 * 32 * w["heads"]
            sb = w["tokens"] * w["heads"] * 4
            assert lay.member_bytes - lay.ref_v_scale >= sb * ref
        else:
            assert lay.ring_k_scale == 0 and lay.vcur_scale == lay.vscale == lay.rope_table
            assert lay.vmax == lay.total
    # 512x512 bf16: 2R + 2M + KF + 2 B_max = 120 frames of 10 MiB, plus the small tables
    mib = L.lact_cache_footprint(_cfg("s512_bf16")) / 2 ** 20
    assert 1200 <= mib < 1201


def test_set_layout_and_footprint():
    """A set of n members: n copies of the persistent regions at a fixed stride, one
    staging area; a set of 1 is the single cache."""
    for name in ("s512_bf16", "fp8_kv", "tiny_ref", "s720_bf16"):
        c = _cfg(name)
        one = L.lact_cache_layout(c)
        s1 = L.lact_set_layout(c, 1)
        assert [getattr(one, f) for f, _ in L.lact_layout._fields_] == \
            [getattr(s1, f) for f, _ in L.lact_layout._fields_]
        for n in (2, 3, 120):
            lay = L.lact_set_layout(c, n)
            assert lay.members == n and lay.member_bytes == one.member_bytes
            assert lay.member_bytes % 256 == 0
            for f in ("ring_k", "ring_v", "mem_k", "mem_v", "ref_k", "ref_v", "ring_k_scale",
                      "mem_v_scale", "frame_bytes", "ring_slots", "key_frames_max"):
                assert getattr(lay, f) == getattr(one, f), f
            shift = (n - 1) * one.member_bytes
            for f in ("krot", "qrot", "vcur", "vscale", "rope_table", "attn_flags", "vmax", "vcur_scale", "total"):
                assert getattr(lay, f) == getattr(one, f) + shift, f
            assert L.lact_set_footprint(c, n) == lay.total
    # 40 layers x 3 denoising steps at 512x512 bf16: 120 x 720 MiB persistent + 480 MiB staging
    c = _cfg("s512_bf16")
    gib = L.lact_set_footprint(c, 120) / 2 ** 30
    assert 84.8 < gib < 84.9
    assert L.lact_set_footprint(c, 120) < 120 * L.lact_cache_footprint(c) * 0.62
    for n in (0, -1, L.LACT_MAX_MEMBERS + 1):
        with pytest.raises(L.LactError) as e:
            L.lact_set_footprint(c, n)
        assert e.value.status == 3


@pytest.mark.parametrize("kw, status", [
    (dict(head_dim=96), 2), (dict(heads=0), 2), (dict(ratio=0), 2), (dict(ratio=17), 2),
    (dict(max_block_frames=0), 2), (dict(mem_slots=-1), 2),
    (dict(mem_slots=200, window_frames=50, max_block_frames=8), 3),
    (dict(kv_dtype=0, q_dtype=1), 4), (dict(kv_dtype=2, q_dtype=0), 4),
    (dict(rope_split=(44, 42, 40)), 2), (dict(rope_split=(43, 43, 42)), 2), (dict(rope_mode=2), 2),
    (dict(rope_theta=0.5), 1), (dict(ref_frames=-1), 2),
    (dict(ref_frames=100, mem_slots=100, window_frames=50, max_block_frames=8), 3),
    (dict(grid_h=1024, grid_w=512), 3),
])
def test_config_validation(kw, status):
    with pytest.raises(L.LactError) as e:
        L.lact_cache_footprint(_cfg(**kw))
    assert e.value.status == status
    assert L.lib().lact_last_error().decode()


def _planner_matches_oracle(name, steps):
    w = synth.workload(name)
    cfg = L.make_cfg(**w)
    plan = L.Plan(cfg)
    bk = Bookkeeping(w["window_frames"], w["mem_slots"], w["ratio"], w["max_block_frames"],
                     w.get("ref_frames", 0))
    for s in range(steps):
        n = w["first_block"] if s == 0 else w["block"]
        got, want = plan.state(), bk.state()
        for key in ("F", "E", "G", "win_len", "mem_len", "pending", "ring_slots", "version"):
            assert got[key] == want[key], (name, s, key, got, want)
        gk, wk = plan.keys(n), bk.keys(n)
        assert [(k["segment"], k["slot"], k["id"], k["t_pos"]) for k in gk] == \
               [(k["segment"], k["slot"], k["id"], k["t_pos"]) for k in wk], (name, s)
        plan.append(n)
        bk.append(n)
        groups, written = plan.compress()
        want_groups = bk.compress()
        assert groups == want_groups, (name, s)
        assert written == min(len(want_groups), w["mem_slots"])


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_planner_bitexact_vs_oracle_1000_steps(name):
    _planner_matches_oracle(name, 1000)


@pytest.mark.parametrize("W, M, r, B", [(0, 4, 5, 3), (3, 1, 2, 7), (5, 0, 5, 8), (2, 7, 3, 1),
                                         (8, 16, 5, 8), (1, 1, 1, 1)])
def test_planner_bitexact_odd_shapes(W, M, r, B):
    """Odd sizes, including a memory of one slot (groups overwritten inside one call) and
    no window at all, with blocks of varying sizes."""
    w = synth.workload("tiny_f32", window_frames=W, mem_slots=M, ratio=r, max_block_frames=B)
    plan = L.Plan(L.make_cfg(**w))
    bk = Bookkeeping(W, M, r, B)
    for s in range(300):
        n = 1 + (s * 7) % B
        assert plan.state()["G"] == bk.G
        plan.append(n)
        bk.append(n)
        g1, written = plan.compress()
        g2 = bk.compress()
        assert g1 == g2 and written == min(len(g2), M)
        assert [(k["segment"], k["slot"], k["id"], k["t_pos"]) for k in plan.keys(n)] == \
               [(k["segment"], k["slot"], k["id"], k["t_pos"]) for k in bk.keys(n)]


def test_planner_errors_leave_state_unchanged():
    w = synth.workload("tiny_f32")
    plan = L.Plan(L.make_cfg(**w))
    bk = Bookkeeping(4, 10, 5, 2)
    with pytest.raises(L.LactError) as e:
        plan.append(3)
    assert e.value.status == 3
    with pytest.raises(OracleCapacityError):
        bk.append(3)
    for _ in range(5):
        plan.append(2)
        bk.append(2)
    before = plan.state()
    with pytest.raises(L.LactError) as e:
        plan.append(2)                    # a complete group is waiting
    assert e.value.status == 5
    with pytest.raises(OracleStateError):
        bk.append(2)
    assert plan.state() == before


class _HostOnlyCache:
    """A cache handle over a host address of the right alignment: lact_cache_init does no
    device work, and every call below fails its checks before anything is enqueued."""

    def __init__(self, name="tiny_f32", members=None, **kw):
        self.cfg = _cfg(name, **kw)
        if members is None:
            self.nbytes = L.lact_cache_footprint(self.cfg)
            self.h = L.lact_cache_init(self.cfg, 0x10000000, self.nbytes)
        else:
            self.nbytes = L.lact_set_footprint(self.cfg, members)
            self.h = L.lact_set_init(self.cfg, members, 0x10000000, self.nbytes)

    def close(self):
        L.lact_cache_destroy(self.h)


def _call(fn, *args):
    return fn(*args)


def test_abi_error_paths_before_enqueue():
    lib = L.lib()
    c = _HostOnlyCache()
    h = c.h
    vp = ctypes.c_void_p
    dev = vp(0x20000000)
    # attention before any RoPE pass at this state
    assert lib.lact_block_attention(h, None, 0, dev, None, None) == 5
    assert "rope" in lib.lact_last_error().decode().lower()
    # null / misaligned pointers
    assert lib.lact_rope_reset_apply(h, None, dev, dev, 2, None) == 1
    assert lib.lact_rope_reset_apply(h, vp(0x20000004), dev, dev, 2, None) == 1
    assert lib.lact_kv_ring_append(h, dev, None, 2, None) == 1
    assert lib.lact_convkv_compress(h, None, dev, dev, dev, None, None) == 1
    assert lib.lact_block_attention(h, None, 0, None, None, None) == 1
    # frame counts out of range
    assert lib.lact_rope_reset_apply(h, dev, dev, dev, 0, None) == 3
    assert lib.lact_rope_reset_apply(h, dev, dev, dev, 3, None) == 3
    assert lib.lact_kv_ring_append(h, dev, dev, 3, None) == 3
    assert lib.lact_kv_ring_append(h, dev, dev, 0, None) == 3
    # nothing changed
    st = L.lact_cache_state(h)
    assert (st["F"], st["G"], st["version"], st["staged_valid"]) == (0, 0, 0, 0)
    # keys of an empty cache: only the current frames, at positions 0..n-1
    keys = L.lact_cache_keys(h, 2)
    assert [(k["segment"], k["t_pos"]) for k in keys] == [(2, 0), (2, 1)]
    # compress with nothing ready enqueues nothing and succeeds
    n = ctypes.c_int32(-1)
    w = vp(0x30000000)
    assert lib.lact_convkv_compress(h, w, w, w, w, None, ctypes.byref(n)) == 0 and n.value == 0
    c.close()


def test_cache_init_checks():
    lib = L.lib()
    cfg = _cfg("tiny_f32")
    nbytes = L.lact_cache_footprint(cfg)
    out = ctypes.c_void_p()
    assert lib.lact_cache_init(ctypes.byref(cfg), ctypes.c_void_p(0x10000010), nbytes,
                               ctypes.byref(out)) == 1          # not 256-aligned
    assert lib.lact_cache_init(ctypes.byref(cfg), ctypes.c_void_p(0x10000000), nbytes - 1,
                               ctypes.byref(out)) == 3          # too small
    assert lib.lact_cache_init(ctypes.byref(cfg), None, nbytes, ctypes.byref(out)) == 1
    assert lib.lact_cache_destroy(None) == 0


def test_reference_segment_checks():
    """lact_ref_set: refused on a cache without a reference segment and for a wrong frame
    count; a cache with one refuses the RoPE pass until it is set; the key table starts with
    the reference frames at positions 0 .. ref_frames-1."""
    lib = L.lib()
    dev = ctypes.c_void_p(0x20000000)
    c = _HostOnlyCache("tiny_f32")
    assert lib.lact_ref_set(c.h, dev, dev, 2, None) == 5          # no reference segment
    c.close()
    c = _HostOnlyCache("tiny_ref")
    assert lib.lact_ref_set(c.h, dev, dev, 1, None) == 2          # ref_frames is 2
    assert lib.lact_ref_set(c.h, None, dev, 2, None) == 1
    assert lib.lact_rope_reset_apply(c.h, dev, dev, dev, 2, None) == 5
    assert "reference" in lib.lact_last_error().decode()
    assert L.lact_cache_state(c.h)["ref_valid"] == 0
    keys = L.lact_cache_keys(c.h, 2)
    assert [(k["segment"], k["t_pos"], k["slot"]) for k in keys] == \
        [(L.SEG_REF, 0, 0), (L.SEG_REF, 1, 1), (L.SEG_CURRENT, 2, 0),
         (L.SEG_CURRENT, 3, 1)]
    c.close()


def test_multiblock_argument_checks():
    lib = L.lib()
    c = _HostOnlyCache("tiny_f32", max_block_frames=6)
    dev = ctypes.c_void_p(0x20000000)
    blocks = (ctypes.c_int32 * 2)(1, 2)
    # still no RoPE pass: state error comes first
    assert lib.lact_block_attention(c.h, blocks, 2, dev, None, None) == 5
    c.close()


def test_set_member_checks():
    """A set refuses the single-cache forms of the per-member calls and member indexes out
    of range; attention asks for the member the staging holds; the buffer must hold every
    member; the reference is tracked per member; one bookkeeping for all members."""
    lib = L.lib()
    dev = ctypes.c_void_p(0x20000000)
    c = _HostOnlyCache("tiny_ref", members=3)
    assert lib.lact_rope_reset_apply(c.h, dev, dev, dev, 2, None) == 1
    assert "member" in lib.lact_last_error().decode()
    assert lib.lact_block_attention(c.h, None, 0, dev, None, None) == 1
    assert lib.lact_ref_set(c.h, dev, dev, 2, None) == 1
    for m in (-1, 3):
        assert lib.lact_member_rope_reset_apply(c.h, m, dev, dev, dev, 2, None) == 1
        assert lib.lact_member_block_attention(c.h, m, None, 0, dev, None, None) == 1
        assert lib.lact_member_ref_set(c.h, m, dev, dev, 2, None) == 1
    # no reference stored yet: the RoPE pass of any member is refused
    assert lib.lact_member_rope_reset_apply(c.h, 1, dev, dev, dev, 2, None) == 5
    assert lib.lact_member_block_attention(c.h, 1, None, 0, dev, None, None) == 5
    st = L.lact_cache_state(c.h)
    assert st["ref_valid"] == 0 and st["staged_member"] == 0 and st["F"] == 0
    c.close()
    # a set's buffer must hold all members
    cfg = _cfg("tiny_f32")
    need = L.lact_set_footprint(cfg, 4)
    with pytest.raises(L.LactError) as e:
        L.lact_set_init(cfg, 4, 0x10000000, need - 1)
    assert e.value.status == 3
    with pytest.raises(L.LactError) as e:
        L.lact_set_init(cfg, 0, 0x10000000, need)
    assert e.value.status == 3


def test_header_is_plain_c99():
    """include/lact.h compiles as strict C99 (no C++ or compiler extensions) with every
    warning an error; nothing is written (syntax check of a translation unit on stdin)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = ('#include "lact.h"\n'
           "int main(void) {\n"
           "  lact_cfg c; lact_layout l; lact_state s; lact_key_frame k;\n"
           "  (void)c; (void)l; (void)s; (void)k;\n"
           "  return LACT_MAX_KEY_FRAMES > 0 && LACT_MAX_MEMBERS > 0 ? 0 : 1;\n"
           "}\n")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    r = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-I", inc, "-x", "c", "-"], input=src, text=True, capture_output=True)
    assert r.returncode == 0, r.stderr


def test_binding_tensor_checks():
    """The binding's checks on tensors handed to kernels: exact shape, dtype and device,
    and whole frames; the C calls take bare pointers and trust them."""
    cpu = torch.device("cpu")
    t = torch.zeros((32, 2, 64), dtype=torch.bfloat16)
    L._expect(t, (32, 2, 64), torch.bfloat16, cpu, "q")
    for shape, dtype, dev in (((16, 2, 64), torch.bfloat16, cpu), ((32, 2, 64), torch.float32, cpu),
                              ((32, 2, 64), torch.bfloat16, torch.device("cuda", 0))):
        with pytest.raises(ValueError):
            L._expect(t, shape, dtype, dev, "q")
    with pytest.raises(TypeError):
        L._expect([0.0], (1,), torch.float32, cpu, "q")
    assert L._frames(t, 16, "q") == 2
    for bad, T in ((t, 24), (torch.zeros((0, 2, 64)), 16)):
        with pytest.raises(ValueError):
            L._frames(bad, T, "q")


def test_c_client_against_the_header():
    """A plain C program (tests/c_client/plan_client.c) built with gcc against
    include/lact.h and linked to liblact.so: the structs and calls as a C compiler sees
    them, on the host-only calls (sizing, layout, errors, 1000 planner steps against the
    schedule's closed form)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(L.LIB_PATH)
    out_dir = os.path.join(root, "_build", "c_client")       # git-ignored build folder
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "plan_client")
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    r = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                        "-I", os.path.join(root, "include"),
                        os.path.join(root, "tests", "c_client", "plan_client.c"),
                        "-L", libdir, "-llact", f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{rocm_lib}",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "1000 planner steps hold" in r.stdout


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for several (flag or a launcher's WORLD_SIZE) it
    exits non-zero with a message before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    bench = os.path.join(root, "bench.py")
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, bench] + args, capture_output=True, text=True,
                           timeout=120, env=dict(os.environ, **env))
        assert r.returncode == 2, (args, env, r.stderr)
        assert "one GPU" in r.stderr and r.stdout == ""


def test_missing_library_fails_loudly(monkeypatch):
    """Without liblact.so every entry of the binding raises (there is no CPU path)."""
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", os.path.join(os.path.dirname(L.LIB_PATH), "absent.so"))
    cfg = _cfg("tiny_f32")
    for call in (L.lib, lambda: L.lact_cache_footprint(cfg), lambda: L.Plan(cfg)):
        with pytest.raises(RuntimeError, match="missing"):
            call()
