"""GPU parity of the split-cache decode path against the CPU oracle.

Bars: INT2 page bytes (codes, packing, bf16 scale/zero) bit-exact; attention
outputs within 2e-3 max relative error per row (max |err| / max |ref|)."""
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


def _check_bytes(run, inp, ref):
    wl = inp.wl
    for b, r in ref.items():
        want = sh.oracle_records(r, wl.D, wl.G, wl.Hkv)
        phys = run.sc.hist_table_h[b, :want.shape[0]]
        got = run.pool[phys]
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"seq {b}: {len(bad)} byte mismatches, first {bad[:5].tolist()}"


def _check_out(run, ref, tol=TOL):
    worst = 0.0
    for b, r in ref.items():
        e = sh.row_rel_err(run.out[b].astype(np.float64), r["out"])
        worst = max(worst, float(e.max()))
        assert np.all(e <= tol), f"seq {b}: row errors {np.sort(e)[-4:]}"
        lerr = np.abs(run.lse[b] - r["lse"]).max()
        assert lerr < 1e-3, f"seq {b}: lse error {lerr}"
    return worst


KERNELS = [1, 2]      # vector-ALU and matrix-core INT2 kernels


@pytest.mark.parametrize("kernel", KERNELS)
def test_tiny_one_step(kernel):
    _say("case: tiny one step, kernel", kernel)
    inp = synth.make_small(synth.workload("tiny"))
    run = sh.build_and_step(inp, steps=1, int2_kernel=kernel)
    ref = sh.oracle_step(inp, steps=1)
    _check_bytes(run, inp, ref)
    w = _check_out(run, ref)
    _say("tiny worst row rel err", w)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_tiny_splits_and_rotations(splits, kernel):
    """Different history chunkings, R_v != R_k, and R_v = identity."""
    _say("case: tiny splits", splits, "kernel", kernel)
    wl = synth.workload("tiny", B=2, lengths=(1024, 777), steps=2, seed=5)
    inp = synth.make_small(wl, distinct_rv=True)
    run = sh.build_and_step(inp, steps=2, int2_kernel=kernel, num_splits=splits)
    ref = sh.oracle_step(inp, steps=2)
    _check_bytes(run, inp, ref)
    _check_out(run, ref)
    run = sh.build_and_step(inp, steps=2, int2_kernel=kernel, num_splits=splits, R_v_none=True)
    ref = sh.oracle_step(inp, steps=2, R_v_none=True)
    _check_bytes(run, inp, ref)
    _check_out(run, ref)


@pytest.mark.parametrize("kernel", KERNELS)
def test_edge_lengths_and_head_map(kernel):
    """Sequences with no history, a partial sink, one history token; a
    non-contiguous GQA head map."""
    _say("case: edge lengths, kernel", kernel)
    wl = synth.workload("tiny", B=5, Hkv=2, Hq=8, lengths=(10, 64, 320, 321, 400), steps=1, seed=6)
    inp = synth.make_small(wl)
    hm = [1, 0, 1, 0, 0, 1, 1, 0]
    run = sh.build_and_step(inp, steps=1, int2_kernel=kernel, head_map=hm)
    ref = sh.oracle_step(inp, steps=1, head_map=hm)
    _check_bytes(run, inp, ref)
    _check_out(run, ref)


@pytest.mark.parametrize("kernel", KERNELS)
def test_qwen3_8b_32k_one_step(kernel):
    """Qwen3-8B-shaped layer at 32K context, every history page and output."""
    _say("case: qwen3-8b-32k, kernel", kernel)
    inp = synth.make_small(synth.workload("qwen3-8b-32k"))
    run = sh.build_and_step(inp, steps=1, int2_kernel=kernel)
    ref = sh.oracle_step(inp, steps=1)
    _check_bytes(run, inp, ref)
    w = _check_out(run, ref)
    _say("32k worst row rel err", w)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("D,G,Hq,Hkv", [(128, 128, 16, 2), (128, 32, 8, 2), (64, 64, 8, 1),
                                       (128, 64, 4, 2), (128, 64, 4, 4), (64, 32, 6, 3),
                                       (128, 32, 16, 2), (64, 32, 16, 2)])
def test_shapes(kernel, D, G, Hq, Hkv):
    """Other head_dim / group / GQA shapes: G = 128 with 8 q heads per KV head
    (Qwen3-32B-shaped), G = 32 at D = 128, G = 64 at D = 64; 2 and 1 q heads
    per KV head (partly empty head quads on the matrix-core kernel), and 3 KV
    heads with 2 q heads each; 8 q heads per KV head at G = 32 (at D = 128 the
    matrix-core kernel runs it with 8 waves per block); ragged history."""
    _say("case: shape", D, G, Hq, Hkv, "kernel", kernel)
    wl = synth.workload("tiny", B=2, Hkv=Hkv, Hq=Hq, D=D, G=G, lengths=(1500, 2077), steps=1, seed=11)
    inp = synth.make_small(wl)
    run = sh.build_and_step(inp, steps=1, int2_kernel=kernel, num_splits=2)
    ref = sh.oracle_step(inp, steps=1)
    _check_bytes(run, inp, ref)
    w = _check_out(run, ref)
    _say("worst row rel err", w)


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("shape", ["tiny", "edge", "d128g4", "d128g8"])
def test_bf16_history_comparison(shape, splits):
    """The comparison layout (whole history in BF16 pages, HISTORY_BF16) equals
    one softmax over all tokens of each sequence."""
    _say("case: BF16 history", shape, "splits", splits)
    if shape == "tiny":
        wl = synth.workload("tiny", B=2, lengths=(1024, 777), steps=1, seed=21)
    elif shape == "edge":
        wl = synth.workload("tiny", B=5, Hkv=2, Hq=8, lengths=(10, 64, 320, 321, 400), steps=1, seed=22)
    elif shape == "d128g4":
        wl = synth.workload("tiny", B=2, Hkv=2, Hq=8, D=128, G=64, lengths=(3000, 1700), steps=1, seed=23)
    else:
        wl = synth.workload("tiny", B=2, Hkv=2, Hq=16, D=128, G=128, lengths=(2500, 999), steps=1, seed=24)
    inp = synth.make_small(wl)
    out, lse = sh.build_bf16_history_and_attend(inp, num_splits=splits)
    ref = sh.oracle_plain(inp)
    for b, r in ref.items():
        e = sh.row_rel_err(out[b].astype(np.float64), r["out"])
        assert np.all(e <= TOL), f"seq {b}: row errors {np.sort(e)[-4:]}"
        assert np.abs(lse[b] - r["lse"]).max() < 1e-3


@pytest.mark.parametrize("shape", ["tiny", "edge", "d128g4", "d128g8", "b8"])
@pytest.mark.parametrize("kernel", KERNELS)
def test_fused_step_matches_separate_calls(shape, kernel):
    """oscar_decode_step over several steps gives the same INT2 and BF16 pool
    bytes, bit for bit, and the same outputs as demote_pack + write_bf16 +
    decode_attn + merge; and matches the oracle."""
    _say("case: fused step", shape, "kernel", kernel)
    if shape == "tiny":
        wl = synth.workload("tiny", B=2, lengths=(1024, 777), steps=3, seed=31)
    elif shape == "edge":
        wl = synth.workload("tiny", B=5, Hkv=2, Hq=8, lengths=(10, 64, 320, 321, 400), steps=3, seed=32)
    elif shape == "d128g4":
        wl = synth.workload("tiny", B=2, Hkv=2, Hq=8, D=128, G=64, lengths=(3000, 1700), steps=3, seed=33)
    elif shape == "d128g8":
        wl = synth.workload("tiny", B=2, Hkv=2, Hq=16, D=128, G=128, lengths=(2500, 999), steps=3, seed=34)
    else:
        # batch 8, mixed lengths: blocks of the INT2 kernel cover several sequences
        wl = synth.workload("tiny", B=8, Hkv=2, Hq=8, D=128, G=64,
                            lengths=(2000, 330, 500, 340, 900, 1200, 321, 700), steps=3, seed=35)
    inp = synth.make_small(wl, distinct_rv=True)
    sep = sh.build_and_step(inp, steps=3, int2_kernel=kernel)
    fus = sh.build_and_step(inp, steps=3, int2_kernel=kernel, fused=True)
    assert np.array_equal(sep.pool, fus.pool), "INT2 pools differ"
    assert np.array_equal(sep.bf16_k, fus.bf16_k) and np.array_equal(sep.bf16_v, fus.bf16_v), \
        "BF16 pools differ"
    # every kernel's work assignment is static: the same arithmetic in the
    # same order
    assert np.array_equal(sep.out.view(np.uint32), fus.out.view(np.uint32)), "outputs differ"
    assert np.array_equal(sep.lse.view(np.uint32), fus.lse.view(np.uint32)), "lse differ"
    ref = sh.oracle_step(inp, steps=3)
    _check_bytes(fus, inp, ref)
    _check_out(fus, ref)


@pytest.mark.parametrize("case", ["dominant_fallback", "dominant_balanced", "mixed_short", "batch_1025",
                                  "batch_512_8waves", "batch_513_8waves"])
def test_block_balancing(case):
    """The matrix-core kernel's block schedule: blocks take equal ranges of the
    histories laid end to end (a block may cover several short sequences, a
    long sequence many blocks); when one sequence would need more than
    2*num_splits + 2 partial slots it falls back to equal parts per sequence;
    batches above one sequence per thread of a block (1024, or 512 for the
    8-wave instances) always use parts."""
    _say("case: block balancing", case)
    if case.startswith("dominant"):
        wl = synth.workload("tiny", B=8, Hkv=2, Hq=8, D=128, G=64,
                            lengths=(6000, 400, 400, 400, 400, 400, 400, 400), steps=1, seed=41)
        splits = 1 if case == "dominant_fallback" else 0
    elif case == "mixed_short":
        wl = synth.workload("tiny", B=8, Hkv=2, Hq=8, D=128, G=64,
                            lengths=(2000, 330, 500, 340, 900, 1200, 321, 700), steps=1, seed=42)
        splits = 1
    elif case == "batch_1025":
        rng = np.random.default_rng(43)
        wl = synth.workload("tiny", B=1025, lengths=tuple(int(x) for x in rng.integers(300, 420, 1025)),
                            steps=1, seed=43)
        splits = 0
    else:
        # D = 128, G = 32, 8 q heads per KV head: the 8-wave instance
        n = 512 if case == "batch_512_8waves" else 513
        rng = np.random.default_rng(44)
        wl = synth.workload("tiny", B=n, Hkv=2, Hq=16, D=128, G=32,
                            lengths=tuple(int(x) for x in rng.integers(300, 420, n)), steps=1, seed=44)
        splits = 0
    inp = synth.make_small(wl)
    run = sh.build_and_step(inp, steps=1, int2_kernel=2, num_splits=splits)
    ref = sh.oracle_step(inp, steps=1)
    _check_bytes(run, inp, ref)
    _check_out(run, ref)


@pytest.mark.parametrize("Hkv,Hq,D,G", [(16, 64, 64, 32), (6, 24, 128, 64), (3, 24, 64, 64)])
def test_head_groups(Hkv, Hq, D, G):
    """KV-head counts other than 8 on the matrix-core kernel (blocks cover a
    pair of KV heads): 8 pairs per sequence (16 heads), 3 pairs (6 heads), and
    a last pair with a dead head (3 heads, 8 q heads per KV head); several
    sequences, so blocks are balanced across them; also through the fused
    decode step."""
    _say("case: head groups", Hkv, Hq, D, G)
    wl = synth.workload("tiny", B=3, Hkv=Hkv, Hq=Hq, D=D, G=G, lengths=(1300, 700, 2100), steps=2, seed=51)
    inp = synth.make_small(wl)
    ref = sh.oracle_step(inp, steps=2)
    for fused in (False, True):
        run = sh.build_and_step(inp, steps=2, int2_kernel=2, fused=fused)
        _check_bytes(run, inp, ref)
        _check_out(run, ref)


def test_bulk_quantise_order_and_splits():
    """oscar_demote_pack on many tokens: 4000 tokens of 8 KV heads in one call
    run the 16-token-block kernel, the 7-way split the one-token kernel, the
    2-way interleaved split the block kernel with pages completed by two
    calls (their V words take the AND/OR path).  The pool bytes do not depend
    on the order of the entries, on the split or on the kernel, and equal the
    oracle's records."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    from oracle import oscar_oracle as orc
    _say("case: bulk quantise order and splits")
    wl = synth.workload("tiny", B=1, Hkv=8, Hq=32, D=128, G=64, lengths=(4000,), steps=1, seed=61,
                        clip_set=synth.WIDE_CLIPS)
    inp = synth.make_small(wl)
    n, npg = 3992, 250                             # 249 full pages and one of 8 tokens
    K, V = inp.K[0][:n], inp.V[0][:n]              # [n][Hkv][D] bf16 bits
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    Rk, Rv = dev(inp.R_k), dev(inp.R_v)
    ck, cv = dev(inp.clip_k), dev(inp.clip_v)
    phys = synth.page_permutation(61, npg, extra=2)
    dst_all = (phys[np.arange(n) // 16].astype(np.int64) * 16 + np.arange(n) % 16).astype(np.int32)

    def run(order, chunks):
        cache = ob.Cache(wl.Hkv, wl.D, wl.G, npg + 2, npg + 1)
        kb = np.zeros((npg + 1, wl.Hkv, 16, wl.D), np.uint16)
        vb = np.zeros_like(kb)
        for t in range(n):
            kb[t // 16, :, t % 16] = K[t]
            vb[t // 16, :, t % 16] = V[t]
        cache.bf16_k.copy_(dev(kb.view(np.int16)))
        cache.bf16_v.copy_(dev(vb.view(np.int16)))
        src_all = np.arange(n, dtype=np.int32)
        for part in np.array_split(order, chunks):
            ob.demote_pack(cache, dev(src_all[part]), dev(dst_all[part]), Rk, Rv, ck, cv)
        torch.cuda.synchronize()
        return cache.int2.cpu().numpy()

    rng = np.random.default_rng(61)
    base = run(np.arange(n), 1)
    assert np.array_equal(run(rng.permutation(n), 1), base), "entry order changed the bytes"
    assert np.array_equal(run(np.arange(n), 7), base), "split calls changed the bytes"
    inter = np.concatenate([np.arange(0, n, 2), np.arange(1, n, 2)])
    assert np.array_equal(run(inter, 2), base), "interleaved calls changed the bytes"
    Kf, Vf = synth.bf16_bits_to_f64(K), synth.bf16_bits_to_f64(V)
    for j in range(wl.Hkv):
        kc, ks, kz = orc.quantize_tokens(Kf[:, j], inp.R_k[j], wl.G, float(inp.clip_k[j]))
        vc, vs, vz = orc.quantize_tokens(Vf[:, j], inp.R_v[j], wl.G, float(inp.clip_v[j]))
        for pg in (0, 31, 124, 249):
            a, e = pg * 16, min(n, pg * 16 + 16)
            pad = lambda x: np.concatenate([x[a:e], np.zeros((16 - (e - a),) + x.shape[1:], x.dtype)])
            want = orc.encode_record(pad(kc), pad(ks), pad(kz), pad(vc), pad(vs), pad(vz), wl.D, wl.G)
            assert np.array_equal(base[phys[pg], j], want), f"page {pg} head {j}"


@pytest.mark.parametrize("D,G,g,order", [(128, 32, 2, None), (128, 64, 4, None), (64, 64, 8, None),
                                         (128, 64, 2, (1, 0, 3, 2)), (64, 32, 4, (2, 3, 0, 1))])
def test_codebook_v_level_precision(D, G, g, order):
    """A codebook whose V levels each lie just under half an f16 unit in the
    last place from the nearest f16 value (the largest error a PV on f16
    levels could make, the same for every token with that code): outputs of
    the matrix-core kernel within a quarter of the bar against the oracle
    (which uses the levels as given), bytes exact.  The kernel writes the
    levels as Lmin + beta * h with integers 0 <= h <= 2047.  With `order` the
    V levels are given out of order (level k is the k-th of the ascending
    ones' permutation), so that the smallest and largest are not L0 and L3:
    the kernel's quantiser and the oracle's both count the midpoints below a
    value, so the bytes still agree."""
    from int2_rotated_kv_amd import binding as ob
    _say(f"case: codebook V level precision D{D} G{G} g{g} order {order}")
    wl = synth.workload("tiny", B=3, Hkv=2, Hq=2 * g, D=D, G=G, lengths=(2400, 1800, 2900), steps=1, seed=97 + g)
    inp = synth.make_small(wl, distinct_rv=True)
    cb = synth.make_codebook(wl.seed, wl.Hkv)
    for j in range(wl.Hkv):
        for k in range(4):
            x = np.float32(cb[j, 1, k])
            h = np.float16(x)
            up = np.nextafter(h, np.float16(np.inf))            # the f16 value above
            mid = (np.float64(h) + np.float64(up)) / 2
            cb[j, 1, k] = np.float32(mid - (np.float64(up) - np.float64(h)) * 0.01)
    assert np.all(np.diff(cb[:, 1], axis=-1) > 0)
    if order is not None:
        cb[:, 1] = cb[:, 1][:, list(order)]
    ref = sh.oracle_step(inp, steps=1, codebook=cb)
    run = sh.build_and_step(inp, steps=1, int2_kernel=ob.INT2_MFMA, codebook=cb)
    _check_bytes(run, inp, ref)
    worst = 0.0
    for b, r in ref.items():
        e = sh.row_rel_err(run.out[b].astype(np.float64), r["out"])
        worst = max(worst, float(e.max()))
    assert worst <= TOL / 4, f"worst row rel err {worst:.3e}"
    assert run.status == 0
    _say(f"codebook V level precision: worst row rel err {worst:.3e}")


@pytest.mark.parametrize("D,G,g", [(128, 64, 4), (64, 64, 8)])
def test_codebook_v_grid_hard_levels(D, G, g):
    """V levels (0.35, 1.6650913, 2.6494343, 2.6499999): the ratios
    (0.5718, 0.99975) on which a grid of integers 0..2047 measured from the
    smallest level errs most among 20000 random sets (2.4e-4 of the span;
    the oracle with its V levels replaced by that grid's errs by 1.86e-3 on
    these inputs, by 4.9e-7 with the kernel's grid).  Outputs of the
    matrix-core kernel within a quarter of the bar against the oracle,
    bytes exact."""
    from int2_rotated_kv_amd import binding as ob
    _say(f"case: codebook V grid hard levels D{D} G{G} g{g}")
    wl = synth.workload("tiny", B=3, Hkv=2, Hq=2 * g, D=D, G=G, lengths=(2300, 1900, 2700), steps=1,
                        seed=131 + g)
    inp = synth.make_small(wl, distinct_rv=True)
    cb = synth.make_codebook(wl.seed, wl.Hkv)
    cb[:, 1] = np.asarray([0.35, 1.6650913, 2.6494343, 2.6499999], dtype=np.float32)
    ref = sh.oracle_step(inp, steps=1, codebook=cb)
    run = sh.build_and_step(inp, steps=1, int2_kernel=ob.INT2_MFMA, codebook=cb)
    _check_bytes(run, inp, ref)
    worst = 0.0
    for b, r in ref.items():
        e = sh.row_rel_err(run.out[b].astype(np.float64), r["out"])
        worst = max(worst, float(e.max()))
    assert worst <= TOL / 4, f"worst row rel err {worst:.3e}"
    assert run.status == 0
    _say(f"codebook V grid hard levels: worst row rel err {worst:.3e}")


K_LEVEL_SETS = {
    "b0b1-dominant": (0.0, 0.1, 0.2, 3.0),      # cA = 0.1, cB = 0, cC = 2.7
    "b0-dominant": (0.0, 2.5, 0.05, 2.6),       # cB = 2.475, cC = -2.35
    "negative": (-1.5, -0.4, 0.45, 1.5),
    "out-of-order": (2.2, 0.3, 2.9, 0.8),
}


@pytest.mark.parametrize("levels", sorted(K_LEVEL_SETS))
@pytest.mark.parametrize("D,G,g", [(128, 64, 4), (128, 64, 8), (128, 128, 8), (64, 32, 8)])
def test_codebook_k_plane_weights(D, G, g, levels):
    """K codebooks whose plane weights cA = (L2 - L0)/2, cB = L1 - L0 - cA,
    cC = L3 - L2 - L1 + L0 differ widely (one plane dominant, negative
    levels, levels out of order), on instances where the matrix-core kernel
    takes the three planes in one accumulator with the weights in the query
    pieces (D128/G64 at 4 and 8 q heads per KV head, D64/G32 at 8) and one
    where each plane has its own (D128/G128 at 8): outputs within half the
    bar against the oracle (the f16 PV weights alone give up to ~4e-4 on
    these inputs, whatever the K levels), bytes exact, status 0."""
    from int2_rotated_kv_amd import binding as ob
    _say(f"case: codebook K plane weights D{D} G{G} g{g} {levels}")
    wl = synth.workload("tiny", B=3, Hkv=2, Hq=2 * g, D=D, G=G, lengths=(2100, 1700, 2600), steps=1,
                        seed=113 + g + D // 64)
    inp = synth.make_small(wl, distinct_rv=True)
    cb = synth.make_codebook(wl.seed, wl.Hkv)
    cb[0, 0] = np.asarray(K_LEVEL_SETS[levels], dtype=np.float32)
    ref = sh.oracle_step(inp, steps=1, codebook=cb)
    run = sh.build_and_step(inp, steps=1, int2_kernel=ob.INT2_MFMA, codebook=cb)
    _check_bytes(run, inp, ref)
    worst = 0.0
    for b, r in ref.items():
        e = sh.row_rel_err(run.out[b].astype(np.float64), r["out"])
        worst = max(worst, float(e.max()))
    assert worst <= TOL / 2, f"worst row rel err {worst:.3e}"
    assert run.status == 0
    _say(f"codebook K plane weights: worst row rel err {worst:.3e}")


@pytest.mark.parametrize("codebook", [False, True])
@pytest.mark.parametrize("D,G", [(64, 32), (64, 64), (128, 32), (128, 64), (128, 128)])
def test_bulk_quantise_every_shape(D, G, codebook):
    """oscar_demote_pack in bulk (2000 entries of 8 KV heads: the
    16-token-block kernel) for every head_dim and group size, with uniform
    codes and with a Lloyd-Max codebook: 1995 tokens into randomly placed
    pages, the last page partial (11 tokens), and 5 entries with both slots
    -1 (skipped) at random positions.  Every page's record bytes equal the
    oracle's (a partial page's unwritten token slots stay zero), and the
    status word stays 0."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    from oracle import oscar_oracle as orc
    _say(f"case: bulk quantise D{D} G{G} codebook {codebook}")
    seed = 71 + D + G + (1 if codebook else 0)
    wl = synth.workload("tiny", B=1, Hkv=8, Hq=32, D=D, G=G, lengths=(2100,), steps=1, seed=seed,
                        clip_set=synth.WIDE_CLIPS)
    inp = synth.make_small(wl)
    n, npg = 1995, 125                             # 124 full pages and one of 11 tokens
    K, V = inp.K[0][:n], inp.V[0][:n]              # [n][Hkv][D] bf16 bits
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    Rk, Rv = dev(inp.R_k), dev(inp.R_v)
    ck, cv = dev(inp.clip_k), dev(inp.clip_v)
    cb = synth.make_codebook(seed, wl.Hkv) if codebook else None
    phys = synth.page_permutation(seed, npg, extra=3)
    dst = (phys[np.arange(n) // 16].astype(np.int64) * 16 + np.arange(n) % 16).astype(np.int32)
    src = np.arange(n, dtype=np.int32)
    rng = np.random.default_rng(seed)
    at = np.sort(rng.choice(n, 5, replace=False))
    src = np.insert(src, at, -1)
    dst = np.insert(dst, at, -1)
    assert src.shape == (2000,) and ((2000 + 15) // 16) * wl.Hkv * 2 >= 1024   # the bulk kernel
    cache = ob.Cache(wl.Hkv, D, G, npg + 3, npg, codebook=dev(cb) if codebook else None)
    kb = np.zeros((npg, wl.Hkv, 16, D), np.uint16)
    vb = np.zeros_like(kb)
    for t in range(n):
        kb[t // 16, :, t % 16] = K[t]
        vb[t // 16, :, t % 16] = V[t]
    cache.bf16_k.copy_(dev(kb.view(np.int16)))
    cache.bf16_v.copy_(dev(vb.view(np.int16)))
    ob.demote_pack(cache, dev(src), dev(dst), Rk, Rv, ck, cv)
    torch.cuda.synchronize()
    pool = cache.int2.cpu().numpy()
    assert cache.read_status() == 0
    Kf, Vf = synth.bf16_bits_to_f64(K), synth.bf16_bits_to_f64(V)
    for j in range(wl.Hkv):
        if codebook:
            kc, ks, kz = orc.quantize_tokens_codebook(Kf[:, j], inp.R_k[j], G, float(inp.clip_k[j]), cb[j, 0])
            vc, vs, vz = orc.quantize_tokens_codebook(Vf[:, j], inp.R_v[j], G, float(inp.clip_v[j]), cb[j, 1])
        else:
            kc, ks, kz = orc.quantize_tokens(Kf[:, j], inp.R_k[j], G, float(inp.clip_k[j]))
            vc, vs, vz = orc.quantize_tokens(Vf[:, j], inp.R_v[j], G, float(inp.clip_v[j]))
        for pg in range(npg):
            a, e = pg * 16, min(n, pg * 16 + 16)
            pad = lambda x: np.concatenate([x[a:e], np.zeros((16 - (e - a),) + x.shape[1:], x.dtype)])
            want = orc.encode_record(pad(kc), pad(ks), pad(kz), pad(vc), pad(vs), pad(vz), D, G)
            assert np.array_equal(pool[phys[pg], j], want), f"page {pg} head {j}"
    unused = np.setdiff1d(np.arange(npg + 3), phys)
    assert not pool[unused].any(), "a page no entry names was written"


@pytest.mark.parametrize("shape", ["b8_mixed", "qwen3-8b-32k"])
def test_bitwise_repeatable(shape):
    """The matrix-core kernel's waves take fixed page batches (only their
    issue priority follows timing), so two runs on freshly built caches give
    bitwise the same outputs, the fused step gives bitwise the outputs of the
    separate calls, and OSCAR_FLAG_DETERMINISTIC (accepted, no effect)
    changes nothing; all within the oracle bar.  Batch 8 with mixed lengths
    puts several sequences in one block; the 32K layer gives each block long
    parts."""
    from int2_rotated_kv_amd import binding as ob
    _say("case: bitwise repeatable", shape)
    if shape == "b8_mixed":
        wl = synth.workload("tiny", B=8, Hkv=2, Hq=8, D=128, G=64,
                            lengths=(2000, 330, 500, 340, 900, 1200, 321, 700), steps=2, seed=61)
    else:
        wl = synth.workload("qwen3-8b-32k", steps=2)
    inp = synth.make_small(wl)
    a = sh.build_and_step(inp, steps=2, int2_kernel=2)
    b = sh.build_and_step(inp, steps=2, int2_kernel=2)
    c = sh.build_and_step(inp, steps=2, int2_kernel=2, fused=True)
    d = sh.build_and_step(inp, steps=2, int2_kernel=2, flags=ob.FLAG_DETERMINISTIC)
    for other, what in ((b, "second run"), (c, "fused step"), (d, "with the flag")):
        assert np.array_equal(a.out.view(np.uint32), other.out.view(np.uint32)), f"{what}: outputs differ"
        assert np.array_equal(a.lse.view(np.uint32), other.lse.view(np.uint32)), f"{what}: lse differ"
    ref = sh.oracle_step(inp, steps=2)
    _check_bytes(a, inp, ref)
    w = _check_out(a, ref)
    _say(f"bitwise repeatable, worst row rel err {w:.3e}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("shape", ["tiny", "d128g64", "d128g128", "d128g32", "d64g64g8", "d128g64sym",
                                   "d128g64mixed", "d128g32g8", "d128g64g8", "d64g32g8"])
def test_codebook_variant(shape, kernel):
    """Lloyd-Max codebook variant: the prompt history quantised in bulk, then
    two decode steps (one-token demotion, attention on either INT2 kernel),
    through the separate
    calls and through oscar_decode_step.  INT2 page bytes bit-exact against
    the oracle's nearest-level quantiser, outputs within the oracle bar, and
    the fused step bitwise equal to the separate calls.  "mixed": KV head 0
    has symmetric levels (the matrix-core kernel skips its third code plane),
    head 1 fitted ones."""
    from int2_rotated_kv_amd import binding as ob
    _say("case: codebook variant", shape, "kernel", kernel)
    if shape == "tiny":
        wl = synth.workload("tiny", B=2, lengths=(1024, 777), steps=2, seed=81)
    elif shape in ("d128g64", "d128g64sym", "d128g64mixed"):
        wl = synth.workload("tiny", B=2, Hkv=2, Hq=8, D=128, G=64, lengths=(3000, 1700), steps=2, seed=82)
    elif shape == "d128g128":
        wl = synth.workload("tiny", B=2, Hkv=2, Hq=16, D=128, G=128, lengths=(2500, 999), steps=2, seed=83)
    elif shape == "d128g32":
        wl = synth.workload("tiny", B=3, Hkv=2, Hq=8, D=128, G=32, lengths=(2000, 400, 1300), steps=2, seed=84)
    elif shape in ("d128g32g8", "d128g64g8", "d64g32g8"):
        # 8 q heads per KV head; the matrix-core kernel runs these with 8
        # waves per block
        D, G = {"d128g32g8": (128, 32), "d128g64g8": (128, 64), "d64g32g8": (64, 32)}[shape]
        wl = synth.workload("tiny", B=3, Hkv=2, Hq=16, D=D, G=G, lengths=(2200, 500, 1400), steps=2, seed=86)
    else:
        wl = synth.workload("tiny", B=2, Hkv=2, Hq=16, D=64, G=64, lengths=(1800, 700), steps=2, seed=85)
    inp = synth.make_small(wl, distinct_rv=True)
    # "sym": levels symmetric about the middle of the range, whose b0&b1 term
    # is exactly 0 (the matrix-core kernel then skips that code plane)
    cb = synth.make_codebook(wl.seed, wl.Hkv, symmetric=shape.endswith("sym"))
    if shape.endswith("sym"):
        assert np.all(((cb[..., 3] - cb[..., 2]) - cb[..., 1]) + cb[..., 0] == 0)
    mixed = shape.endswith("mixed")
    if mixed:
        cb[0] = synth.make_codebook(wl.seed, wl.Hkv, symmetric=True)[0]
        cterm = ((cb[..., 3] - cb[..., 2]) - cb[..., 1]) + cb[..., 0]
        assert np.all(cterm[0] == 0) and np.all(cterm[1] != 0)
    kw = dict(steps=2, int2_kernel=kernel, codebook=cb)
    sep = sh.build_and_step(inp, **kw)
    fus = sh.build_and_step(inp, fused=True, **kw)
    ref = sh.oracle_step(inp, steps=2, codebook=cb)
    _check_bytes(sep, inp, ref)
    _check_bytes(fus, inp, ref)
    w = _check_out(sep, ref)
    _check_out(fus, ref)
    assert np.array_equal(sep.out.view(np.uint32), fus.out.view(np.uint32)), "fused outputs differ"
    # the uniform quantiser would give other bytes: the codebook is really used
    uni = sh.oracle_step(inp, steps=2)
    assert not np.array_equal(sh.oracle_records(uni[0], wl.D, wl.G, wl.Hkv),
                              sh.oracle_records(ref[0], wl.D, wl.G, wl.Hkv))
    _say(f"codebook {shape} kernel {kernel}: bytes exact, worst row rel err {w:.3e}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_single_sequence_loose_length_bound(kernel):
    """One sequence whose max_hist_len is the page table's whole capacity,
    four times its history (the grid and the chunking are sized by the bound,
    the pages walked by the length): outputs and bytes match the oracle."""
    _say("case: single sequence, loose max_hist_len, kernel", kernel)
    wl = synth.workload("tiny", B=1, Hkv=2, Hq=8, D=128, G=64, lengths=(1500,), steps=2, seed=91)
    inp = synth.make_small(wl)
    extra = 3 * sh.hist_capacity_pages(1500, 2)              # table rows 4x the history
    bound = 16 * (sh.hist_capacity_pages(1500, 2) + extra)
    run = sh.build_and_step(inp, steps=2, int2_kernel=kernel, max_hist_len=bound, num_splits=40,
                            extra_pages=extra)
    ref = sh.oracle_step(inp, steps=2)
    _check_bytes(run, inp, ref)
    _check_out(run, ref)


def test_decode_step_in_hip_graph():
    """oscar_decode_step captured in a HIP graph (the library allocates,
    synchronises and memsets nothing, so a step can be captured) and replayed
    three times, with eager work and a synchronisation between replays:
    every replay equals the eager run of the same step bit for bit.  The step is re-run on the cache after it: its slot
    lists are planned again from the state before it, so each run demotes the
    token now in the freed slot (the new one) into the same history slot and
    stores the same new token, the same bytes every time."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    from int2_rotated_kv_amd.splitcache import SplitCache
    _say("case: decode step in a HIP graph")
    wl = synth.workload("tiny", B=3, Hkv=2, Hq=8, D=128, G=64, lengths=(2000, 700, 1300), steps=1, seed=95)
    inp = synth.make_small(wl)
    run = sh.build_and_step(inp, steps=1, int2_kernel=2, flags=ob.FLAG_DETERMINISTIC)
    sc = run.sc
    dev = "cuda"
    # plan the step build_and_step took again: the lengths and ring before it
    sc.hist_len_h -= np.array([1 if L >= 320 else 0 for L in wl.lengths])
    sc.bf16_len_h = np.minimum(np.array(wl.lengths), 320)
    sc.ring_head[:] = 0
    dsrc, ddst, wdst = (torch.from_numpy(x).to(dev) for x in sc.plan_step())
    sc.commit_step()
    sc.sync_lengths()
    args = sc.decode_args(int2_kernel=2, flags=ob.FLAG_DETERMINISTIC)
    B = wl.B
    kn = sh.to_dev_bf16(np.stack([inp.K[b][wl.lengths[b]] for b in range(B)])).view(torch.int16)
    vn = sh.to_dev_bf16(np.stack([inp.V[b][wl.lengths[b]] for b in range(B)])).view(torch.int16)
    q = sh.to_dev_bf16(inp.q[0]).view(torch.int16)
    Rk = torch.from_numpy(inp.R_k).to(dev)
    Rv = torch.from_numpy(inp.R_v).to(dev)
    ck = torch.from_numpy(inp.clip_k).to(dev)
    cv = torch.from_numpy(inp.clip_v).to(dev)
    ws = ob.alloc_workspace(sc.cache, args, device=dev)
    out = torch.zeros((B, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    lse = torch.zeros((B, wl.Hq), dtype=torch.float32, device=dev)

    def step():
        ob.decode_step(sc.cache, args, dsrc, ddst, ck, cv, wdst, kn, vn, q, Rk, Rv, ws, out, lse)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    pool0 = sc.cache.int2.clone()
    step()                                            # the eager step repeats itself
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32))
    assert torch.equal(sc.cache.int2, pool0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float(i + 1))                       # eager work between replays
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), f"replay {i}: outputs differ"
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), f"replay {i}: lse differ"
        assert torch.equal(sc.cache.int2, pool0), f"replay {i}: INT2 pool differs"
    _say("graph: 3 replays bitwise equal to the eager step")


def test_decode_steps_replayed_from_a_hip_graph():
    """Consecutive decode steps, each one replay of a HIP graph holding one
    oscar_decode_step (captured once; the step's slot lists, new token and
    query are copied into the captured buffers, the lengths into the cache,
    with eager work and a synchronisation between replays): every step's
    outputs within the oracle bar for that step, bitwise equal to the eager
    fused step at the same step, and the history bytes exact at the end."""
    _say("case: decode steps replayed from a HIP graph")
    wl = synth.workload("tiny", B=3, Hkv=2, Hq=8, D=128, G=64, lengths=(2000, 700, 1300), steps=4, seed=96)
    inp = synth.make_small(wl)
    got, eager = {}, {}
    run = sh.build_and_step(inp, steps=4, int2_kernel=2, graph=True,
                            on_step=lambda st, o, l: got.__setitem__(st, (o, l)))
    sh.build_and_step(inp, steps=4, int2_kernel=2, fused=True, max_hist_len=int(run.hist_len.max()),
                      on_step=lambda st, o, l: eager.__setitem__(st, (o, l)))
    worst = 0.0
    for st in range(4):
        ref = sh.oracle_step(inp, steps=st + 1)
        o, l = got[st]
        for b, r in ref.items():
            e = sh.row_rel_err(o[b].astype(np.float64), r["out"])
            worst = max(worst, float(e.max()))
            assert np.all(e <= TOL), f"step {st} seq {b}: row errors {np.sort(e)[-4:]}"
            assert np.abs(l[b] - r["lse"]).max() < 1e-3, f"step {st} seq {b}: lse"
        assert np.array_equal(o.view(np.uint32), eager[st][0].view(np.uint32)), f"step {st}: not the eager outputs"
    _check_bytes(run, inp, sh.oracle_step(inp, steps=4))
    assert run.status == 0
    _say(f"graph replays: 4 steps within the oracle bar (worst {worst:.3e}), bitwise the eager step")


def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([32, 64] if D == 64 else [32, 64, 128]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 7))
    lengths = tuple(int(x) for x in rng.integers(1, 3000, B))
    steps = int(rng.integers(1, 3))
    kernel = int(rng.choice([0, 1, 2]))
    codebook = bool(rng.integers(0, 2))
    det = bool(rng.integers(0, 2))
    clips = synth.WIDE_CLIPS if rng.integers(0, 2) else ()
    return dict(D=D, G=G, Hkv=Hkv, Hq=g * Hkv, B=B, lengths=lengths, steps=steps, seed=2000 + seed,
                clip_set=clips), kernel, codebook, det


@pytest.mark.parametrize("seed", list(range(12)) + [41, 48, 52])
def test_random_configurations(seed):
    """Seeded random configurations (head_dim, group, KV heads, q heads per KV
    head, batch, lengths from 1 to 3000 tokens, 1-2 steps, kernel choice,
    codebook or not, deterministic option or not, one clip ratio or per-head
    K != V ratios) against the oracle: page bytes exact, outputs within the
    bar, no status bit.  Seeds 41, 48 and 52 (codebook, matrix-core kernel,
    1 or 2 q heads per KV head) exceeded the bar (2.8e-3 to 5.6e-3) when PV
    took the V levels rounded to f16."""
    from int2_rotated_kv_amd import binding as ob
    kw, kernel, codebook, det = _random_case(seed)
    _say(f"case: random configuration {seed}: {kw}, kernel {kernel}, codebook {codebook}, det {det}")
    wl = synth.workload("tiny", **kw)
    inp = synth.make_small(wl, distinct_rv=bool(seed % 2))
    cb = synth.make_codebook(wl.seed, wl.Hkv) if codebook else None
    run = sh.build_and_step(inp, steps=wl.steps, int2_kernel=kernel, codebook=cb,
                            flags=ob.FLAG_DETERMINISTIC if det else 0)
    ref = sh.oracle_step(inp, steps=wl.steps, codebook=cb)
    _check_bytes(run, inp, ref)
    w = _check_out(run, ref)
    assert run.status == 0, f"status {run.status}"
    _say(f"random {seed}: bytes exact, worst row rel err {w:.3e}")
