"""GPU parity of shared history pages (a prompt prefix that several sequences'
page tables list), attended once for all their sequences, against the CPU
oracle, which attends every sequence's history on its own.

The member sequences' tokens are equal on the shared pages (synth.share_history)
and their page tables alias the first member's physical pages.  Page bytes must
be bit-exact, outputs within 2e-3 max relative error per row and lse within
1e-3, on both the separate calls and oscar_decode_step, over several steps (the
new tokens go to each sequence's own pages)."""
import sys

import numpy as np
import pytest

import synth
import split_helpers as sh

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(run, inp, ref):
    wl = inp.wl
    worst = 0.0
    for b, r in ref.items():
        want = sh.oracle_records(r, wl.D, wl.G, wl.Hkv)
        got = run.pool[run.sc.hist_table_h[b, :want.shape[0]]]
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"seq {b}: {len(bad)} byte mismatches, first {bad[:5].tolist()}"
        e = sh.row_rel_err(run.out[b].astype(np.float64), r["out"])
        worst = max(worst, float(e.max()))
        assert np.all(e <= TOL), f"seq {b}: row errors {np.sort(e)[-4:]}"
        assert np.abs(run.lse[b] - r["lse"]).max() < 1e-3, f"seq {b}: lse"
    return worst


CASES = {
    # 8 q heads per KV head, group = head_dim = 128 (the Qwen3-32B shape): a
    # prefix shared by 5 sequences (40 query rows per KV head), then two
    # different continuations shared by 3 and by 2 of them
    "d128_tree": (dict(B=5, Hkv=2, Hq=16, D=128, G=128, lengths=(2400, 2300, 2400, 2200, 900), seed=501),
                  [(0, 30, 0, 5), (30, 70, 0, 3), (30, 4, 3, 2)]),
    # 20 sequences x 8 q heads = 160 rows: two row groups of the cascade grid
    "d128_rows160": (dict(B=20, Hkv=2, Hq=16, D=128, G=128, lengths=tuple(600 + 7 * i for i in range(20)),
                          seed=502),
                     [(0, 16, 0, 20)]),
    # head_dim 64, group 64, 4 q heads per KV head; the whole prompt history
    # of two sequences is shared (their own pages: only the steps' tokens)
    "d64_all": (dict(B=3, Hkv=2, Hq=8, D=64, G=64, lengths=(1600, 1600, 1000), seed=503),
                [(0, 80, 0, 2), ]),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("fused", [False, True])
def test_shared_pages_match_oracle(case, fused):
    from int2_rotated_kv_amd import binding as ob
    kw, segs = CASES[case]
    _say(f"case: shared pages {case}, fused {fused}")
    wl = synth.workload("tiny", steps=3, clip_set=synth.WIDE_CLIPS, **kw)
    inp = synth.share_history(synth.make_small(wl, distinct_rv=True), segs)
    ref = sh.oracle_step(inp, steps=3)
    run = sh.build_and_step(inp, steps=3, int2_kernel=ob.INT2_AUTO, fused=fused, shared=segs)
    w = _check(run, inp, ref)
    # the same step with every sequence reading its pages on its own: also
    # within the bar (the two paths round their f16 weights against
    # different running maxima, so they agree only to the bar's order)
    plain = sh.build_and_step(inp, steps=3, int2_kernel=ob.INT2_AUTO, fused=fused)
    wp = _check(plain, inp, ref)
    e = sh.row_rel_err(run.out.astype(np.float64), plain.out.astype(np.float64)).max()
    _say(f"{case}: bytes exact, worst row rel err {w:.3e} (per-sequence reading {wp:.3e}, "
         f"between the two {e:.2e})")


def test_shared_pages_deterministic_and_vector_alu():
    """With the deterministic option the shared-page path is bitwise
    repeatable and the fused step equals the separate calls bit for bit; the
    vector-ALU kernel ignores the shared segments (every sequence reads its
    pages) and agrees within the bar."""
    from int2_rotated_kv_amd import binding as ob
    kw, segs = CASES["d128_tree"]
    _say("case: shared pages, deterministic option and vector-ALU kernel")
    wl = synth.workload("tiny", steps=2, **kw)
    inp = synth.share_history(synth.make_small(wl), segs)
    det = dict(steps=2, int2_kernel=ob.INT2_MFMA, flags=ob.FLAG_DETERMINISTIC, shared=segs)
    a = sh.build_and_step(inp, **det)
    b = sh.build_and_step(inp, **det)
    c = sh.build_and_step(inp, fused=True, **det)
    d = sh.build_and_step(inp, noalloc=True, **det)
    for other, what in ((b, "second run"), (c, "fused step"), (d, "allocation-free step")):
        assert np.array_equal(a.out.view(np.uint32), other.out.view(np.uint32)), f"{what}: outputs differ"
        assert np.array_equal(a.lse.view(np.uint32), other.lse.view(np.uint32)), f"{what}: lse differ"
    ref = sh.oracle_step(inp, steps=2)
    _check(a, inp, ref)
    v = sh.build_and_step(inp, steps=2, int2_kernel=ob.INT2_VALU, shared=segs)
    _check(v, inp, ref)


def test_shared_segments_rejected():
    """Segments that do not tile a sequence's first pages, or leave the batch or
    max_hist_len, are rejected before anything is launched."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    kw, segs = CASES["d128_tree"]
    wl = synth.workload("tiny", steps=1, **kw)
    inp = synth.share_history(synth.make_small(wl), segs)
    run = sh.build_and_step(inp, steps=1, int2_kernel=ob.INT2_AUTO, shared=segs)
    sc = run.sc
    for bad in ([(1, 29, 0, 5)],                     # does not start at page 0
                [(0, 30, 0, 5), (31, 69, 0, 3)],     # gap
                [(0, 30, 0, 5), (0, 30, 1, 2)],      # overlap
                [(0, 30, 0, 6)],                     # beyond the batch
                [(0, 30, 0, 1)],                     # a single sequence
                [(0, 400, 0, 2)]):                   # beyond max_hist_len
        args = sc.decode_args(shared=bad)
        with pytest.raises(ob.OscarError):
            ob.workspace_bytes(sc.cache, args)
    torch.cuda.synchronize()


def _random_tree(seed):
    """A seeded batch whose sequences share history pages as a prefix tree:
    contiguous groups of the batch share a root prefix, and contiguous
    subgroups of a group may share a continuation after it."""
    rng = np.random.default_rng(3000 + seed)
    D, G = [(128, 128), (64, 64)][seed % 2]
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([4, 8]))
    B = int(rng.integers(3, 9))
    lengths = [int(x) for x in rng.integers(900, 2600, B)]
    pages = [(L - 320) // 16 for L in lengths]
    segs = []
    b = 0
    while b < B:
        n = int(rng.integers(2, B - b + 1)) if B - b >= 2 else 1
        grp = list(range(b, b + n))
        b += n
        if n < 2:
            continue
        root = int(rng.integers(1, min(pages[i] for i in grp) + 1))
        segs.append((0, root, grp[0], n))
        if n >= 4:
            k = int(rng.integers(2, n - 1))
            for sub in (grp[:k], grp[k:]):
                left = min(pages[i] for i in sub) - root
                if len(sub) >= 2 and left > 0:
                    segs.append((root, int(rng.integers(1, left + 1)), sub[0], len(sub)))
    return dict(B=B, Hkv=Hkv, Hq=g * Hkv, D=D, G=G, lengths=tuple(lengths), seed=3100 + seed), segs


@pytest.mark.parametrize("seed", range(6))
def test_shared_pages_random_trees(seed):
    """Seeded random prefix trees (group sizes, prefix and continuation
    lengths, KV heads, 4 or 8 q heads per KV head, head_dim 64 or 128 with
    one group per token): bytes exact and outputs within the bar against the
    oracle, two steps through oscar_decode_step."""
    from int2_rotated_kv_amd import binding as ob
    kw, segs = _random_tree(seed)
    _say(f"case: random shared tree {seed}: {kw}, segments {segs}")
    if not segs:
        pytest.skip("no group of two or more sequences drawn")
    wl = synth.workload("tiny", steps=2, clip_set=synth.WIDE_CLIPS, **kw)
    inp = synth.share_history(synth.make_small(wl, distinct_rv=True), segs)
    ref = sh.oracle_step(inp, steps=2)
    run = sh.build_and_step(inp, steps=2, int2_kernel=ob.INT2_MFMA, fused=True, shared=segs)
    assert run.status == 0
    w = _check(run, inp, ref)
    _say(f"random tree {seed}: bytes exact, worst row rel err {w:.3e}")


def test_shared_pages_with_codebook():
    """A Lloyd-Max codebook cache with shared pages: the cascade has no
    codebook path, so every sequence reads its shared pages itself; bytes
    exact and outputs within the bar against the oracle (which uses the
    levels), through the separate calls and oscar_decode_step."""
    from int2_rotated_kv_amd import binding as ob
    kw, segs = CASES["d128_tree"]
    _say("case: shared pages with a codebook")
    wl = synth.workload("tiny", steps=2, **kw)
    inp = synth.share_history(synth.make_small(wl, distinct_rv=True), segs)
    cb = synth.make_codebook(wl.seed, wl.Hkv)
    ref = sh.oracle_step(inp, steps=2, codebook=cb)
    for fused in (False, True):
        run = sh.build_and_step(inp, steps=2, int2_kernel=ob.INT2_AUTO, fused=fused, shared=segs, codebook=cb)
        assert run.status == 0
        w = _check(run, inp, ref)
        _say(f"codebook with shared pages, fused {fused}: bytes exact, worst row rel err {w:.3e}")
