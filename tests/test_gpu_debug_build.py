"""The bounds-checking build (liboscar_debug.so, OSCAR_DEBUG): kernels report
an index they clamp or skip through the cache's status word
(OSCAR_STATUS_DEBUG_BOUNDS) and otherwise behave as the release build.

Each case runs in a child process whose binding loads the debug library
(OSCAR_LIB): valid inputs on both INT2 kernels and with shared pages keep the
status word 0 and stay within the oracle bar; a history page id outside the
pool (which every kernel skips), a demotion entry with only one of its two
slots set (skipped) and a member of a shared segment whose history ends inside
the segment's pages set the bit, while the release build, given the same
inputs in this process, goes on without a word."""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DEBUG_LIB = os.path.join(ROOT, "int2_rotated_kv_amd", "liboscar_debug.so")

CHILD = textwrap.dedent(r"""
    import sys
    import numpy as np
    import torch
    sys.path.insert(0, {tests!r})
    sys.path.insert(0, {root!r})
    import synth
    import split_helpers as sh
    from int2_rotated_kv_amd import binding as ob
    assert ob.LIB_PATH.endswith("liboscar_debug.so"), ob.LIB_PATH
    MODE = {mode!r}
    segs = [(0, 30, 0, 3)]
    wl = synth.workload("tiny", B=3, Hkv=2, Hq=16, D=128, G=128, lengths=(2400, 2400, 900), steps=2, seed=901)
    inp = synth.share_history(synth.make_small(wl), segs)
    if MODE == "valid":
        ref = sh.oracle_step(inp, steps=2)
        for kernel, shared, fused in ((ob.INT2_VALU, None, False), (ob.INT2_MFMA, None, True),
                                      (ob.INT2_MFMA, segs, False)):
            run = sh.build_and_step(inp, steps=2, int2_kernel=kernel, shared=shared, fused=fused)
            assert run.status == 0, (kernel, shared, run.status)
            for b, r in ref.items():
                e = sh.row_rel_err(run.out[b].astype(np.float64), r["out"])
                assert np.all(e <= 2e-3), (kernel, b, e.max())
        print("debug build: valid inputs, status 0, within the bar")
    else:
        run = sh.build_and_step(inp, steps=1, int2_kernel=ob.INT2_MFMA,
                                shared=segs if MODE == "shared" else None)
        sc = run.sc
        assert sc.cache.read_status() == 0
        if MODE == "shared":
            # sequence 2's history made shorter than the 30 shared pages (480
            # tokens) that the cascade attends whole for it
            sc.hist_len[2] = 400
            args = sc.decode_args(int2_kernel=ob.INT2_MFMA, shared=segs)
            out = torch.zeros((wl.B, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
            ob.decode(sc.cache, args, sh.to_dev_bf16(inp.q[0]).view(torch.int16),
                      torch.from_numpy(inp.R_k).cuda(), torch.from_numpy(inp.R_v).cuda(), out)
        elif MODE == "page":
            # a history page id past the pool in sequence 1's table
            sc.hist_pages[1, 3] = int(sc.cache.int2.shape[0]) + 7
            args = sc.decode_args(int2_kernel=ob.INT2_MFMA)
            out = torch.zeros((wl.B, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
            ob.decode(sc.cache, args, sh.to_dev_bf16(inp.q[0]).view(torch.int16),
                      torch.from_numpy(inp.R_k).cuda(), torch.from_numpy(inp.R_v).cuda(), out)
        else:
            # a demotion entry with a source slot but no destination
            src = torch.tensor([5, -1, -1], dtype=torch.int32, device="cuda")
            dst = torch.tensor([-1, -1, -1], dtype=torch.int32, device="cuda")
            ob.demote_pack(sc.cache, src, dst, torch.from_numpy(inp.R_k).cuda(),
                           torch.from_numpy(inp.R_v).cuda(), torch.from_numpy(inp.clip_k).cuda(),
                           torch.from_numpy(inp.clip_v).cuda())
        torch.cuda.synchronize()
        st = sc.cache.read_status()
        print("status", st)
        assert st & ob.STATUS_DEBUG_BOUNDS, st
""")


def _child(mode):
    if not os.path.exists(DEBUG_LIB):
        pytest.skip("liboscar_debug.so is not built (python -m int2_rotated_kv_amd.build --debug)")
    env = dict(os.environ, OSCAR_LIB=DEBUG_LIB)
    src = CHILD.format(tests=HERE, root=ROOT, mode=mode)
    r = subprocess.run([sys.executable, "-u", "-c", src], env=env, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0, f"child failed ({mode})"


def test_debug_build_valid_inputs():
    _child("valid")


@pytest.mark.parametrize("mode", ["page", "demote", "shared"])
def test_debug_build_reports_skipped_indices(mode):
    _child(mode)
    # the release build skips the same inputs without a word (a member history
    # shorter than its shared pages: they are still attended whole for it)
    import torch
    import synth
    import split_helpers as sh
    from int2_rotated_kv_amd import binding as ob
    segs = [(0, 30, 0, 3)]
    wl = synth.workload("tiny", B=3, Hkv=2, Hq=16, D=128, G=128, lengths=(2400, 2400, 900), steps=1, seed=901)
    inp = synth.make_small(wl)
    if mode == "shared":
        inp = synth.share_history(inp, segs)
    run = sh.build_and_step(inp, steps=1, int2_kernel=ob.INT2_MFMA, shared=segs if mode == "shared" else None)
    sc = run.sc
    if mode == "shared":
        sc.hist_len[2] = 400
        args = sc.decode_args(int2_kernel=ob.INT2_MFMA, shared=segs)
        out = torch.zeros((wl.B, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
        ob.decode(sc.cache, args, sh.to_dev_bf16(inp.q[0]).view(torch.int16),
                  torch.from_numpy(inp.R_k).cuda(), torch.from_numpy(inp.R_v).cuda(), out)
        assert torch.isfinite(out).all()
    elif mode == "page":
        sc.hist_pages[1, 3] = int(sc.cache.int2.shape[0]) + 7
        args = sc.decode_args(int2_kernel=ob.INT2_MFMA)
        out = torch.zeros((wl.B, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
        ob.decode(sc.cache, args, sh.to_dev_bf16(inp.q[0]).view(torch.int16),
                  torch.from_numpy(inp.R_k).cuda(), torch.from_numpy(inp.R_v).cuda(), out)
        assert torch.isfinite(out).all()
    else:
        src = torch.tensor([5, -1, -1], dtype=torch.int32, device="cuda")
        dst = torch.tensor([-1, -1, -1], dtype=torch.int32, device="cuda")
        ob.demote_pack(sc.cache, src, dst, torch.from_numpy(inp.R_k).cuda(), torch.from_numpy(inp.R_v).cuda(),
                       torch.from_numpy(inp.clip_k).cuda(), torch.from_numpy(inp.clip_v).cuda())
    torch.cuda.synchronize()
    assert sc.cache.read_status() == 0
