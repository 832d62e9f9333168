"""GPU parity on the method's edge cases, against the CPU oracle.

* clip ratios that differ per KV head and between K and V (the clipping
  threshold is a per-layer, per-head calibration constant): a mixed-up head or
  K/V index would change page bytes;
* degenerate groups: all-zero tokens, and constant tokens under identity
  rotations (every rotated group constant), so that groups with scale 0 are
  written and read, with zero point 0 and with a non-zero zero point;
* V group scales just below the matrix-core kernel's f16 weight limit (correct
  on that kernel, no status bit) and above it (status bit set, the vector-ALU
  kernel correct);
* clip ratios outside (0, 1] and non-finite tokens, reported through the
  cache's status word.

Bars as in the other parity tests: page bytes bit-exact, outputs within 2e-3
max relative error per row, lse within 1e-3."""
import sys

import numpy as np
import pytest

import synth
import split_helpers as sh
from oracle import oscar_oracle as orc

pytestmark = pytest.mark.gpu
TOL = 2e-3
KERNELS = [1, 2]      # vector-ALU and matrix-core INT2 kernels


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


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("kernel", KERNELS)
def test_per_head_clips(kernel, fused):
    """Clip ratios from {1.0, 0.95, 0.8, 0.5}, different for K and V of
    every KV head; the prompt history through both demotion kernels (the
    first 1024 tokens of a sequence in one call: the 16-token-block kernel at
    8 KV heads; the rest: the one-token kernel), two decode steps through the
    separate calls or oscar_decode_step."""
    _say("case: per-head clips, kernel", kernel, "fused", fused)
    wl = synth.workload("tiny", B=2, Hkv=8, Hq=32, D=128, G=64, lengths=(1500, 1400), steps=2,
                        seed=301, clip_set=synth.WIDE_CLIPS)
    inp = synth.make_small(wl, distinct_rv=True)
    assert np.all(inp.clip_k != inp.clip_v)
    assert len(set(inp.clip_k.tolist())) > 1 and len(set(inp.clip_v.tolist())) > 1
    run = sh.build_and_step(inp, steps=2, int2_kernel=kernel, fused=fused)
    ref = sh.oracle_step(inp, steps=2)
    _check_bytes(run, inp, ref)
    w = _check_out(run, ref)
    assert run.status == 0, f"status {run.status}"
    # the case is sensitive to the clip indexing: with K and V swapped, or
    # head 0's ratios for every head, the oracle's bytes differ
    for ck, cv in ((inp.clip_v, inp.clip_k),
                   (np.full_like(inp.clip_k, inp.clip_k[0]), np.full_like(inp.clip_v, inp.clip_v[0]))):
        other = synth.SmallInputs(wl, inp.q, inp.K, inp.V, inp.R_k, inp.R_v, ck, cv, inp.out_k, inp.out_v)
        alt = sh.oracle_step(other, steps=2, seqs=[0])
        assert not np.array_equal(sh.oracle_records(alt[0], wl.D, wl.G, wl.Hkv),
                                  sh.oracle_records(ref[0], wl.D, wl.G, wl.Hkv))
    _say(f"per-head clips: bytes exact, worst row rel err {w:.3e}")


def _planted(identity: bool):
    """Two sequences with all-zero and constant tokens in the prompt history
    (one whole page of zeros; the first sequence's prompt history is written
    by both demotion kernels, the second's by the one-token kernel), as the
    first demoted token (the oldest recent one) and as the new token of step
    0."""
    wl = synth.workload("tiny", B=2, Hkv=8, Hq=32, D=128, G=64, lengths=(1400, 420), steps=2,
                        seed=311, clip_set=synth.WIDE_CLIPS)
    inp = synth.make_small(wl, distinct_rv=True)
    for b, L in enumerate(wl.lengths):
        s, h, r = synth.split_lengths(L)
        synth.plant_tokens(inp, b, [s + 3, s + h - 1] + list(range(s + 16, s + 32)), "zero")
        synth.plant_tokens(inp, b, [s + 7, s + 40], "const", value=1.5, which="k")
        synth.plant_tokens(inp, b, [s + 7, s + 41], "const", value=-2.25, which="v")
        synth.plant_tokens(inp, b, [s + h], "zero")              # first demoted token
        synth.plant_tokens(inp, b, [L], "const", value=0.75)     # new token of step 0
    if identity:
        inp.R_k = np.broadcast_to(np.eye(wl.D, dtype=np.float32), inp.R_k.shape).copy()
    return inp


@pytest.mark.parametrize("identity", [False, True])
@pytest.mark.parametrize("kernel", KERNELS)
def test_degenerate_groups(kernel, identity):
    """Groups whose bf16 scale is 0: all-zero tokens (zero point 0) and, with
    identity rotations (R_k = I, R_v = NULL), constant tokens (every group
    constant: zero point c * clip).  Written by the bulk path and by the
    per-step demotion, then attended; both must match the oracle exactly."""
    _say("case: degenerate groups, kernel", kernel, "identity rotations", identity)
    inp = _planted(identity)
    wl = inp.wl
    for fused in (False, True):
        run = sh.build_and_step(inp, steps=2, int2_kernel=kernel, R_v_none=identity, fused=fused)
        ref = sh.oracle_step(inp, steps=2, R_v_none=identity)
        _check_bytes(run, inp, ref)
        w = _check_out(run, ref)
        assert run.status == 0, f"status {run.status}"
    # the planted groups really have scale 0 (and, with identity rotations, a
    # non-zero zero point for the constant tokens)
    r = ref[0]
    s, h, _ = synth.split_lengths(wl.lengths[0])
    assert np.all(r["ks"][3] == 0) and np.all(r["vs"][3] == 0) and np.all(r["kz"][3] == 0)
    assert np.all(r["ks"][h] == 0) and np.all(r["vs"][h] == 0)      # the demoted token
    if identity:
        assert np.all(r["ks"][7] == 0) and np.all(r["kz"][7] != 0)
        assert np.all(r["vs"][7] == 0) and np.all(r["vz"][7] != 0)
    _say(f"degenerate groups: bytes exact, worst row rel err {w:.3e}")


def _v_range_inputs(v_range: float, seed: int):
    """Unrotated V (R_v = NULL) uniform in [-v_range, v_range], clip 0.95, so
    the largest V group scale is about 0.95 * 2 * v_range / 3."""
    wl = synth.workload("tiny", B=2, Hkv=8, Hq=32, D=128, G=64, lengths=(1500, 800), steps=1,
                        seed=seed, v_range=v_range)
    return synth.make_small(wl)


def _expected_v_flag(ref, codebook=None):
    """OSCAR_STATUS_MFMA_V_RANGE as the header defines it: some V group's bf16
    scale times c reaches OSCAR_MFMA_V_SCALE_LIMIT, c = 1 without a codebook
    and max(1, largest |V level|) / 16 with one (fp32), or a V level reaches
    16 times the limit."""
    from int2_rotated_kv_amd import binding as ob
    lim = np.float32(ob.MFMA_V_SCALE_LIMIT)
    flag = False
    for r in ref.values():
        for j in range(r["vs"].shape[1]):
            cm = np.float32(1.0)
            if codebook is not None:
                L = np.abs(codebook[j, 1].astype(np.float32))
                if np.any(L >= np.float32(16.0) * lim):
                    return True
                cm = max(np.float32(1.0), L.max()) * np.float32(1.0 / 16.0)
            prod = r["vs"][:, j].astype(np.float32) * np.float32(cm)
            flag |= bool(np.any(prod >= lim))
    return flag


@pytest.mark.parametrize("kernel", KERNELS)
def test_v_scales_below_mfma_limit(kernel):
    """V group scales up to ~900 (the matrix-core kernel's f16 weights then
    reach 64 * 900 = 57600 < 65504): no status bit, outputs within the bar
    on both kernels."""
    from int2_rotated_kv_amd import binding as ob
    _say("case: V scales below the MFMA limit, kernel", kernel)
    inp = _v_range_inputs(1420.0, 321)
    run = sh.build_and_step(inp, steps=1, int2_kernel=kernel, R_v_none=True)
    ref = sh.oracle_step(inp, steps=1, R_v_none=True)
    vmax = max(float(r["vs"].max()) for r in ref.values())
    assert 850.0 < vmax < ob.MFMA_V_SCALE_LIMIT, vmax
    assert not _expected_v_flag(ref)
    _check_bytes(run, inp, ref)
    w = _check_out(run, ref)
    assert run.status == 0, f"status {run.status}"
    _say(f"largest V scale {vmax}: status 0, worst row rel err {w:.3e}")


def test_v_scales_above_mfma_limit():
    """V group scales up to ~1260: the demotion sets OSCAR_STATUS_MFMA_V_RANGE
    (written both by the bulk path and the decode step's demotion), and the
    vector-ALU kernel, which the status word tells the caller to use, is
    within the bar.  With a Lloyd-Max codebook the matrix-core kernel's
    weights are p * scale_v (its levels below 2.7 are the f16 operand), so the
    same scales fit: no bit, and the matrix-core kernel is within the bar
    too."""
    from int2_rotated_kv_amd import binding as ob
    _say("case: V scales above the MFMA limit")
    inp = _v_range_inputs(2000.0, 322)
    for fused in (False, True):
        run = sh.build_and_step(inp, steps=1, int2_kernel=1, R_v_none=True, fused=fused)
        ref = sh.oracle_step(inp, steps=1, R_v_none=True)
        assert _expected_v_flag(ref)
        assert run.status == ob.STATUS_MFMA_V_RANGE, f"status {run.status}"
        _check_bytes(run, inp, ref)
        _check_out(run, ref)
    cb = synth.make_codebook(322, inp.wl.Hkv)
    ref = sh.oracle_step(inp, steps=1, R_v_none=True, codebook=cb)
    assert not _expected_v_flag(ref, cb)
    for kernel in KERNELS:
        run = sh.build_and_step(inp, steps=1, int2_kernel=kernel, R_v_none=True, codebook=cb)
        assert run.status == 0, f"codebook, kernel {kernel}: status {run.status}"
        _check_bytes(run, inp, ref)
        w = _check_out(run, ref)
        _say(f"codebook, kernel {kernel}: status 0, worst row rel err {w:.3e}")


@pytest.mark.parametrize("bad", [0.0, 1.5, float("nan"), -0.5])
def test_clip_out_of_range_rejected(bad):
    """A clip ratio outside (0, 1] for one KV head's K (and another head's V)
    sets OSCAR_STATUS_CLIP_RANGE and writes those groups as scale 0, zero 0,
    codes 0; every other part of the records is the oracle's.  Through the
    bulk path, the per-step demotion and oscar_decode_step."""
    from int2_rotated_kv_amd import binding as ob
    _say("case: clip out of range", bad)
    wl = synth.workload("tiny", B=1, Hkv=8, Hq=32, D=128, G=64, lengths=(1500,), steps=2, seed=331)
    inp = synth.make_small(wl)
    good = synth.make_small(wl)
    inp.clip_k = inp.clip_k.copy()
    inp.clip_v = inp.clip_v.copy()
    inp.clip_k[0] = np.float32(bad)
    inp.clip_v[5] = np.float32(bad)
    ref = sh.oracle_step(good, steps=2)[0]
    for part, j in (("k", 0), ("v", 5)):
        for key in ("c", "s", "z"):
            ref[part + key][:, j] = 0
    want = sh.oracle_records(ref, wl.D, wl.G, wl.Hkv)
    for fused in (False, True):
        run = sh.build_and_step(inp, steps=2, int2_kernel=1, fused=fused)
        assert run.status == ob.STATUS_CLIP_RANGE, f"status {run.status}"
        got = run.pool[run.sc.hist_table_h[0, :want.shape[0]]]
        bad_at = np.argwhere(got != want)
        assert bad_at.size == 0, f"{len(bad_at)} byte mismatches, first {bad_at[:5].tolist()}"


def test_nonfinite_token_flagged():
    """A token with an infinite channel sets OSCAR_STATUS_NONFINITE (the
    rotation spreads it over the token's groups); finite caches never set it."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    _say("case: non-finite token")
    wl = synth.workload("tiny", B=1, Hkv=8, Hq=32, D=128, G=64, lengths=(1400,), steps=1, seed=341)
    inp = synth.make_small(wl)
    s, h, _ = synth.split_lengths(1400)
    inp.K[0][s + 10, 1, 5] = np.uint16(0x7F80)                   # +inf in bf16
    dev = "cuda"
    cache = ob.Cache(wl.Hkv, wl.D, wl.G, 80, 80, device=dev)
    kb = np.zeros((80, wl.Hkv, 16, wl.D), np.uint16)
    vb = np.zeros_like(kb)
    for t in range(h):
        kb[t // 16, :, t % 16] = inp.K[0][s + t]
        vb[t // 16, :, t % 16] = inp.V[0][s + t]
    cache.bf16_k.copy_(torch.from_numpy(kb.view(np.int16)).to(dev))
    cache.bf16_v.copy_(torch.from_numpy(vb.view(np.int16)).to(dev))
    Rk, Rv = torch.from_numpy(inp.R_k).to(dev), torch.from_numpy(inp.R_v).to(dev)
    ck, cv = torch.from_numpy(inp.clip_k).to(dev), torch.from_numpy(inp.clip_v).to(dev)
    src = torch.arange(0, h, dtype=torch.int32, device=dev)
    ob.demote_pack(cache, src[:10], src[:10], Rk, Rv, ck, cv)     # finite tokens only
    assert cache.read_status() == 0
    ob.demote_pack(cache, src, src, Rk, Rv, ck, cv)               # 16-token-block kernel
    assert cache.read_status() == ob.STATUS_NONFINITE
    cache.clear_status()
    ob.demote_pack(cache, src[10:11], src[10:11], Rk, Rv, ck, cv)  # one-token path
    assert cache.read_status() == ob.STATUS_NONFINITE


@pytest.mark.parametrize("v_range,flag", [(8000.0, False), (12500.0, True)])
def test_v_scales_codebook_limit(v_range, flag):
    """With a codebook (levels below 2.7) the limit sits at V scales of about
    1023 * 16 / 2.7: scales up to ~5000 fit (no bit, the matrix-core kernel
    within the bar), scales up to ~7900 set OSCAR_STATUS_MFMA_V_RANGE (the
    vector-ALU kernel within the bar)."""
    from int2_rotated_kv_amd import binding as ob
    _say("case: codebook V scales, range", v_range)
    inp = _v_range_inputs(v_range, 323)
    cb = synth.make_codebook(323, inp.wl.Hkv)
    ref = sh.oracle_step(inp, steps=1, R_v_none=True, codebook=cb)
    assert _expected_v_flag(ref, cb) == flag
    kernel = 1 if flag else 2
    run = sh.build_and_step(inp, steps=1, int2_kernel=kernel, R_v_none=True, codebook=cb)
    assert run.status == (ob.STATUS_MFMA_V_RANGE if flag else 0), f"status {run.status}"
    _check_bytes(run, inp, ref)
    w = _check_out(run, ref)
    vmax = max(float(r["vs"].max()) for r in ref.values())
    _say(f"largest V scale {vmax}: status {run.status}, worst row rel err {w:.3e}")
