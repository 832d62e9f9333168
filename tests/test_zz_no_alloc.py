"""GPU check of oscar_decode_step_noalloc (the decode step whose workspace is
the library's static device array) against oscar_decode_step with a
workspace the caller allocates: two steps on a larger batch, then two steps
on a smaller one in the same process (the static array then holds the larger
call's contents).  With the deterministic option the two entry points give
the same outputs, lse and pool bytes bit for bit; both are checked against
the oracle as well (page bytes exact, outputs within 2e-3)."""
import sys

import numpy as np
import pytest

import synth
import split_helpers as sh

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    # larger first: 4 sequences, 8 KV heads, g = 4
    dict(B=4, Hkv=8, Hq=32, D=128, G=64, lengths=(3000, 1500, 2200, 700), steps=2, seed=401,
         clip_set=synth.WIDE_CLIPS),
    # then smaller: 2 sequences, 2 KV heads, g = 8, group 128
    dict(B=2, Hkv=2, Hq=16, D=128, G=128, lengths=(900, 400), steps=2, seed=402),
]


@pytest.mark.parametrize("kernel", [2, 1])
def test_noalloc_step_matches_workspace_step(kernel):
    from int2_rotated_kv_amd import binding as ob
    for i, kw in enumerate(CASES):
        _say(f"case: noalloc step, kernel {kernel}, call {i}: {kw}")
        wl = synth.workload("tiny", **kw)
        inp = synth.make_small(wl, distinct_rv=True)
        common = dict(steps=wl.steps, int2_kernel=kernel, flags=ob.FLAG_DETERMINISTIC)
        ref_run = sh.build_and_step(inp, fused=True, **common)
        run = sh.build_and_step(inp, noalloc=True, **common)
        assert np.array_equal(run.out.view(np.uint32), ref_run.out.view(np.uint32)), "outputs differ"
        assert np.array_equal(run.lse.view(np.uint32), ref_run.lse.view(np.uint32)), "lse differ"
        assert np.array_equal(run.pool, ref_run.pool), "INT2 pools differ"
        assert np.array_equal(run.bf16_k, ref_run.bf16_k) and np.array_equal(run.bf16_v, ref_run.bf16_v)
        ref = sh.oracle_step(inp, steps=wl.steps)
        for b, r in ref.items():
            want = sh.oracle_records(r, wl.D, wl.G, wl.Hkv)
            got = run.pool[run.sc.hist_table_h[b, :want.shape[0]]]
            assert np.array_equal(got, want), f"seq {b}: page bytes differ from the oracle"
            e = sh.row_rel_err(run.out[b].astype(np.float64), r["out"])
            assert np.all(e <= 2e-3), f"seq {b}: row errors {np.sort(e)[-4:]}"
            assert np.abs(run.lse[b] - r["lse"]).max() < 1e-3
        _say(f"call {i}: bitwise equal to oscar_decode_step, within the oracle bar")
