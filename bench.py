"""Decode-step benchmark of the split-cache INT2 path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--int2-kernel auto|valu|mfma]

One step = the whole hot path for every sequence of the batch, one
oscar_decode_step call: demote the oldest recent token into the INT2 history,
write the new token into the freed BF16 slot, attend both segments (query
rotation, BF16 segment, INT2 history chunks) and merge.  The same steps
through the four separate entry points (oscar_demote_pack, oscar_write_bf16,
oscar_decode_attn, oscar_merge) are timed alongside.  Inputs are synthetic and
already resident in HBM when timing starts.  Prints ONE JSON line.

The default workload is the Qwen3-8B-shaped batch-32 cache at ~100K context
(8 KV heads, 32 q heads, head_dim 128, INT2 group 64, lengths uniform in
[90000, 100000]): the largest 100K-context configuration on one GPU.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PAGE, SINK, RECENT = 16, 64, 256
HBM_PEAK_GBS = 8000.0


# --------------------------------------------------------------------------
# workload construction (device side, through the library)
# --------------------------------------------------------------------------

class BenchState:
    pass


def build_workload(name: str, total_steps: int, device="cuda", log=print, bf16_history=False,
                   codebook=False, group_size=0, q_heads=0):
    """Build the split cache of a 100K-class workload on the device and plan
    `total_steps` decode steps.  History pages are quantised by
    oscar_demote_pack from generated BF16 tokens.  With bf16_history, the same
    tokens are also laid out as the comparison cache: every history page kept
    in BF16 at its physical id (same page tables), the sink/recent pages after
    them.  With codebook ("fit" or "symmetric"), the cache uses the Lloyd-Max
    codebook variant (seeded levels from synth.make_codebook).  group_size /
    q_heads, when non-zero, replace the workload's G / Hq (the workload is then
    named with them appended)."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    from int2_rotated_kv_amd.splitcache import SplitCache

    ov = {}
    if group_size:
        ov["G"] = group_size
    if q_heads:
        ov["Hq"] = q_heads
    wl = synth.workload(name, steps=total_steps, **ov)
    if ov:
        wl = dataclasses.replace(wl, name=name + "".join(f"-{k}{v}" for k, v in sorted(ov.items())))
    gen = synth.LargeGen(wl, device=device)
    t0 = time.time()
    cb = synth.make_codebook(wl.seed, wl.Hkv, symmetric=codebook == "symmetric") if codebook else None
    sc = SplitCache(wl.B, wl.Hkv, wl.Hq, wl.D, wl.G, gen.hist_table, gen.n_unique,
                    staging_pages=synth.LargeGen.PAGES_PER_BLOCK, device=device,
                    codebook=None if cb is None else torch.from_numpy(cb).to(device))
    Rk = torch.from_numpy(gen.R_k).to(device)
    Rv = torch.from_numpy(gen.R_v).to(device)
    ck = torch.from_numpy(gen.clip_k).to(device)
    cv = torch.from_numpy(gen.clip_v).to(device)

    # unique pages that hold prompt history
    prompt = np.zeros(gen.n_unique, dtype=bool)
    for b in range(wl.B):
        npg = -(-int(gen.hist_len0[b]) // PAGE)
        prompt[gen.unique_of[b, :npg]] = True
    ppb = synth.LargeGen.PAGES_PER_BLOCK
    n_hist = sc.cache.num_int2_pages
    if bf16_history:
        shape = (n_hist + sc.cache.num_bf16_pages, wl.Hkv, PAGE, wl.D)
        bk = torch.zeros(shape, dtype=torch.int16, device=device)
        bv = torch.zeros(shape, dtype=torch.int16, device=device)
    for blk in range(-(-gen.n_unique // ppb)):
        us = np.arange(blk * ppb, min((blk + 1) * ppb, gen.n_unique))
        sel = us[prompt[us]]
        if sel.size == 0:
            continue
        k, v = gen.history_block(blk)
        k = k.view(ppb, PAGE, wl.Hkv, wl.D)[torch.from_numpy(sel - blk * ppb).to(device)]
        v = v.view(ppb, PAGE, wl.Hkv, wl.D)[torch.from_numpy(sel - blk * ppb).to(device)]
        sc.fill_history_pages(gen.phys_of_unique[sel], k.reshape(-1, wl.Hkv, wl.D),
                              v.reshape(-1, wl.Hkv, wl.D), Rk, Rv, ck, cv)
        if bf16_history:
            ph = torch.from_numpy(gen.phys_of_unique[sel].astype(np.int64)).to(device)
            bk[ph] = k.view(torch.int16).permute(0, 2, 1, 3)
            bv[ph] = v.view(torch.int16).permute(0, 2, 1, 3)
    for b in range(wl.B):
        k, v = gen.bf16_tokens(b)
        sc.load_bf16(b, k, v)
    sc.hist_len_h[:] = gen.hist_len0
    torch.cuda.synchronize()
    log(f"[bench] built {name}: {gen.n_unique} unique INT2 pages "
        f"({gen.n_unique * wl.Hkv * sc.cache.rec / 1e9:.2f} GB) in {time.time() - t0:.1f}s")
    status = sc.cache.read_status()
    if status:
        raise RuntimeError(f"demotion reported status bits {status:#x} on {name}")

    # plan every step on the host; upload the slot lists and lengths once
    T = total_steps
    dsrc = np.zeros((T, wl.B), np.int32)
    ddst = np.zeros((T, wl.B), np.int32)
    wdst = np.zeros((T, wl.B), np.int32)
    hl = np.zeros((T, wl.B), np.int32)
    bl = np.zeros((T, wl.B), np.int32)
    h0 = sc.hist_len_h.copy()
    b0 = sc.bf16_len_h.copy()
    r0 = sc.ring_head.copy()
    for s in range(T):
        a, d, w = sc.plan_step()
        sc.commit_step()
        dsrc[s], ddst[s], wdst[s] = a, d, w
        hl[s], bl[s] = sc.hist_len_h, sc.bf16_len_h
    sc.hist_len_h[:], sc.bf16_len_h[:], sc.ring_head[:] = h0, b0, r0
    st = BenchState()
    st.wl, st.gen, st.sc = wl, gen, sc
    # pages the page tables alias (a shared prompt prefix), as the caller's
    # prefix cache would report them
    st.shared = gen.shared_segments()
    st.codebook_h = cb
    st.Rk, st.Rv, st.ck, st.cv = Rk, Rv, ck, cv
    dev = lambda x: torch.from_numpy(x).to(device)
    st.dsrc, st.ddst, st.wdst, st.hl, st.bl = dev(dsrc), dev(ddst), dev(wdst), dev(hl), dev(bl)
    st.hl_h, st.bl_h = hl, bl
    toks = [gen.step_tokens(s) for s in range(T)]
    if bf16_history:
        # sink/recent pages after the history pages; window slot w -> n_hist*16 + w
        bk[n_hist:] = sc.cache.bf16_k
        bv[n_hist:] = sc.cache.bf16_v
        st.cmp_cache = ob.Cache(wl.Hkv, wl.D, wl.G, 0, bk.shape[0], device=device,
                                bf16_k=bk, bf16_v=bv)
        st.cmp_win_pages = sc.bf16_pages + n_hist
        st.cmp_off = n_hist * PAGE
        log(f"[bench] comparison cache: {bk.shape[0]} BF16 pages "
            f"({2 * bk.numel() * 2 / 1e9:.2f} GB)")
    st.knew = torch.stack([t[0] for t in toks]).view(torch.int16)
    st.vnew = torch.stack([t[1] for t in toks]).view(torch.int16)
    st.q = torch.stack([t[2] for t in toks]).view(torch.int16)
    return st


def step_args(st, s: int, int2_kernel: int, num_splits: int = 0):
    from int2_rotated_kv_amd import binding as ob
    return ob.DecodeArgs(st.wl.B, st.wl.Hq, st.sc.hist_pages, st.hl[s], st.sc.bf16_pages, st.bl[s],
                         int(st.hl_h[s].max()), int2_kernel=int2_kernel, num_splits=num_splits,
                         shared=st.shared)


def breakdown_steps(steps):
    """Extra steps run after the timed ones: as many through the separate
    entry points with nothing else on the stream, then as many again with an
    event between phases."""
    return 2 * min(steps, 20)


COLD_SCRATCH = 512 << 20   # bytes written between cold steps (> the 256 MB last-level cache)


def run_steps(st, steps, warmup, int2_kernel, keep_first_out=False, num_splits=0, cold_steps=0,
              prewarm_s=0.0):
    """Warmup steps, then `steps` timed steps through oscar_decode_step with
    nothing else on the stream; then min(steps, 20) steps through the separate
    entry points (demote_pack, write_bf16, decode_attn, merge), timed the same
    way, and as many again with events between the phases (decode_attn split
    into its QROT|BF16 and INT2 phases).  With cold_steps, that many more
    steps each preceded by a 512 MiB scratch write (nothing of the cache left
    in any cache level), timed by events around the step alone.  With
    prewarm_s, that many seconds of INT2-phase launches precede the warmup
    steps (clock ramp after the host-side set-up)."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    E2 = breakdown_steps(steps)
    E = E2 // 2
    T_hot = steps + warmup + E2
    T = T_hot + 2 * cold_steps
    args = [step_args(st, s, int2_kernel, num_splits) for s in range(T)]
    a_qb = [a.with_phases(ob.PHASE_QROT | ob.PHASE_BF16) for a in args]
    a_i2 = [a.with_phases(ob.PHASE_INT2) for a in args]
    # the chunk count (and with it the workspace) need not grow monotonically
    # with the history length: size the workspace for every planned step
    ws = torch.empty(max(ob.workspace_bytes(st.sc.cache, a) for a in args), dtype=torch.uint8,
                     device=st.q.device)
    wl = st.wl
    out = torch.zeros((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=st.q.device)
    lse = torch.zeros((wl.B, wl.Hq), dtype=torch.float32, device=st.q.device)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(E)]
    first_out = None
    cache = st.sc.cache

    def one(s):
        ob.decode_step(cache, args[s], st.dsrc[s], st.ddst[s], st.ck, st.cv, st.wdst[s],
                       st.knew[s], st.vnew[s], st.q[s], st.Rk, st.Rv, ws, out, lse)

    def one_separate(s):
        ob.demote_pack(cache, st.dsrc[s], st.ddst[s], st.Rk, st.Rv, st.ck, st.cv)
        ob.write_bf16(cache, st.wdst[s], st.knew[s], st.vnew[s])
        ob.decode_attn(cache, args[s], st.q[s], st.Rk, ws)
        ob.merge(cache, args[s], ws, st.Rv, out, lse)

    def one_phased(s, e):
        e[0].record()
        ob.demote_pack(cache, st.dsrc[s], st.ddst[s], st.Rk, st.Rv, st.ck, st.cv)
        ob.write_bf16(cache, st.wdst[s], st.knew[s], st.vnew[s])
        e[1].record()
        ob.decode_attn(cache, a_qb[s], st.q[s], st.Rk, ws)
        e[2].record()
        ob.decode_attn(cache, a_i2[s], st.q[s], st.Rk, ws)
        e[3].record()
        ob.merge(cache, args[s], ws, st.Rv, out, lse)
        e[4].record()

    # the GPU idles while the host builds caches and plans steps; a few
    # hundred ms of back-to-back INT2 launches (they only rewrite workspace
    # partials) bring its clocks up before the warmup steps
    if prewarm_s > 0:
        ob.decode_attn(cache, a_qb[0], st.q[0], st.Rk, ws)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < prewarm_s:
            for _ in range(10):
                ob.decode_attn(cache, a_i2[0], st.q[0], st.Rk, ws)
            torch.cuda.synchronize()
    for s in range(warmup):
        one(s)
        if s == 0 and keep_first_out:
            torch.cuda.synchronize()
            first_out = (out.cpu().numpy().copy(), lse.cpu().numpy().copy())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(E):
        one_separate(warmup + steps + i)
    torch.cuda.synchronize()
    wall_sep = time.perf_counter() - t0
    for i in range(E):
        one_phased(warmup + steps + E + i, ev[i])
    torch.cuda.synchronize()
    seg = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(4)] for e in ev]).reshape(E, 4)  # ms
    # the INT2 kernel alone: back-to-back launches of the last step's INT2 phase
    # (it only rewrites the workspace partials) between two events on the
    # stream it is launched on
    n_i2 = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_i2):
        ob.decode_attn(cache, a_i2[T_hot - 1], st.q[T_hot - 1], st.Rk, ws)
    e1.record()
    torch.cuda.synchronize()
    int2_only_ms = e0.elapsed_time(e1) / n_i2
    res = dict(wall_s=wall, seg_ms=seg, first_out=first_out, out=out, args=args,
               int2_only_ms=int2_only_ms, int2_only_step=T_hot - 1,
               ms_separate=1000.0 * wall_sep / E if E else float("nan"))
    if steps:
        res["graph"] = time_graph(one, T_hot - 1, steps, out)
    if cold_steps:
        # two cache-cold protocols, cold_steps steps each: 512 MiB of scratch
        # read (clean eviction, as other layers' caches and weights do) or
        # written (dirty eviction) on the stream before every step
        scratch = torch.ones(COLD_SCRATCH // 4, dtype=torch.int32, device=st.q.device)
        flush = {"read": lambda i: scratch.sum(), "write": lambda i: scratch.fill_(i)}
        for k, (name, fl) in enumerate(flush.items()):
            base = T_hot + k * cold_steps
            ec = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(cold_steps)]
            for i in range(cold_steps):
                fl(i)
                ec[i][0].record()
                one(base + i)
                ec[i][1].record()
            torch.cuda.synchronize()
            last = base + cold_steps - 1
            ci = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(10)]
            for i in range(10):
                fl(i)
                ci[i][0].record()
                ob.decode_attn(cache, a_i2[last], st.q[last], st.Rk, ws)
                ci[i][1].record()
            torch.cuda.synchronize()
            res[f"cold_{name}"] = dict(
                ms=float(np.mean([a.elapsed_time(b) for a, b in ec])),
                int2_ms=float(np.mean([a.elapsed_time(b) for a, b in ci])),
                int2_step=last, steps=range(base, base + cold_steps))
    return res


def time_graph(one, s, replays, out):
    """The decode step `s` (already run once) captured in a HIP graph and
    replayed: each replay repeats the same step (the demotion rewrites the
    same bytes, the store the same token).  Three replays, each followed by a
    synchronisation, are checked against an eager run of the step first
    (every kernel's work assignment is static, so they must agree bit for
    bit); then `replays` replays are timed back to back."""
    import torch
    try:
        one(s)
        torch.cuda.synchronize()
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one(s)
        worst = 0.0
        for _ in range(3):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            den = ref.abs().amax(dim=-1).clamp_min(1e-30)
            worst = max(worst, float(((out - ref).abs().amax(dim=-1) / den).max()))
        t0 = time.perf_counter()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize()
        ms = 1000.0 * (time.perf_counter() - t0) / replays
        return dict(ms_per_step=ms, replay_vs_eager_max_rel=worst, ok=worst == 0.0)
    except Exception as e:  # a capture failure is reported, not fatal
        return dict(ms_per_step=None, error=str(e)[:200], ok=False)


def measure_bulk_quantize(st, n_calls=10):
    """Throughput of the bulk path of oscar_demote_pack (prompt histories):
    the BF16 staging pages of the cache (the last block of generated history
    tokens) quantised into a scratch INT2 pool, 4096 tokens per call."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    wl, sc = st.wl, st.sc
    n = sc.staging_pages * PAGE
    scratch = ob.Cache(wl.Hkv, wl.D, wl.G, sc.staging_pages, sc.cache.num_bf16_pages,
                       device=st.q.device, bf16_k=sc.cache.bf16_k, bf16_v=sc.cache.bf16_v)
    base = sc.staging_base * PAGE
    src = torch.arange(base, base + n, dtype=torch.int32, device=st.q.device)
    dst = torch.arange(0, n, dtype=torch.int32, device=st.q.device)
    ob.demote_pack(scratch, src, dst, st.Rk, st.Rv, st.ck, st.cv)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_calls):
        ob.demote_pack(scratch, src, dst, st.Rk, st.Rv, st.ck, st.cv)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_calls
    return {"kernel": "k_demote_bulk", "tokens_per_call": n, "ms_per_call": ms,
            "token_heads_per_s": n * wl.Hkv / (ms * 1e-3),
            "fp64_fma_per_token_head": 2 * wl.D * wl.D}


def run_steps_bf16(st, steps, warmup):
    """The same decode steps on the comparison cache (history in BF16 pages):
    copy the oldest recent token into its history slot, write the new token
    into the freed window slot, attend (BF16 window + BF16 history) and merge.
    Returns the timed wall seconds and the per-launch time of the history
    kernel alone."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    wl, cache = st.wl, st.cmp_cache
    T = steps + warmup
    args = [ob.DecodeArgs(wl.B, wl.Hq, st.sc.hist_pages, st.hl[s], st.cmp_win_pages, st.bl[s],
                          int(st.hl_h[s].max()), int2_kernel=ob.HISTORY_BF16) for s in range(T)]
    a_h = [a.with_phases(ob.PHASE_INT2) for a in args]
    ws = torch.empty(max(ob.workspace_bytes(cache, a) for a in args), dtype=torch.uint8,
                     device=st.q.device)
    out = torch.zeros((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=st.q.device)
    lse = torch.zeros((wl.B, wl.Hq), dtype=torch.float32, device=st.q.device)
    src = (st.dsrc.long() + st.cmp_off)
    wdst = st.wdst + st.cmp_off
    kp, vp = cache.bf16_k, cache.bf16_v

    def one(s):
        sp, so = src[s] // PAGE, src[s] % PAGE
        kd, vd = kp[sp, :, so, :], vp[sp, :, so, :]       # [B, Hkv, D]
        ob.write_bf16(cache, st.ddst[s], kd, vd)
        ob.write_bf16(cache, wdst[s], st.knew[s], st.vnew[s])
        ob.decode_attn(cache, args[s], st.q[s], None, ws)
        ob.merge(cache, args[s], ws, None, out, lse)

    for s in range(warmup):
        one(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        ob.decode_attn(cache, a_h[T - 1], st.q[T - 1], None, ws)
    e1.record()
    torch.cuda.synchronize()
    return dict(wall_s=wall, hist_ms=e0.elapsed_time(e1) / n, out=out, lse=lse)


# --------------------------------------------------------------------------
# byte accounting (algorithmic: what the method must move)
# --------------------------------------------------------------------------

def hist_bytes_per_token_head(D, G):
    return 2 * (D // 4) + 2 * (D // G) * 4


def int2_alg_bytes(wl, hl_row, splits):
    units = int(hl_row.sum()) * wl.Hkv
    pages = int(sum(-(-int(h) // PAGE) for h in hl_row))
    return (units * hist_bytes_per_token_head(wl.D, wl.G) + pages * 4
            + wl.B * wl.Hq * wl.D * 4 + wl.B * wl.Hq * splits * (wl.D + 2) * 4), units


def step_alg_bytes(wl, hl_row, bl_row, splits):
    i2, _ = int2_alg_bytes(wl, hl_row, splits)
    bf = int(bl_row.sum()) * wl.Hkv * wl.D * 2 * 2
    demote = wl.B * wl.Hkv * 2 * (wl.D * 2 + wl.D // 4 + (wl.D // wl.G) * 4)
    write = wl.B * wl.Hkv * 2 * wl.D * 2 * 2
    merge = wl.B * wl.Hq * (splits * (wl.D + 2) * 4 + (wl.D + 2) * 4 + wl.D * 4)
    q = wl.B * wl.Hq * wl.D * 2 * 2
    return i2 + bf + demote + write + merge + q


# --------------------------------------------------------------------------
# CPU baseline: the oracle, timed on this host
# --------------------------------------------------------------------------

def oracle_step0(st, b, timed=True):
    """The oracle's view of sequence b after the first decode step: it quantises
    the sequence's history from the generated BF16 tokens and encodes its own
    page records (set-up), then - the part that is timed - unpacks and
    dequantises every record, quantises the demoted token and attends all q
    heads over the split cache.  Returns (out [Hq][D], lse [Hq], records
    {kv_head: [pages] uint8 records}, seconds timed, KV-token-heads)."""
    import torch
    from oracle import oscar_oracle as orc

    wl, gen = st.wl, st.gen
    D, G, Hkv, g = wl.D, wl.G, wl.Hkv, wl.g
    ppb = synth.LargeGen.PAGES_PER_BLOCK
    knew0, vnew0, q0 = gen.step_tokens(0)
    hl0 = int(gen.hist_len0[b])
    npg = -(-hl0 // PAGE)
    us = gen.unique_of[b, :npg]
    blocks = {}
    kh = np.empty((npg * PAGE, Hkv, D), np.uint16)
    vh = np.empty_like(kh)
    for i, u in enumerate(us):
        blk = int(u) // ppb
        if blk not in blocks:
            blocks.clear()
            k, v = gen.history_block(blk)
            blocks[blk] = (k.view(torch.int16).cpu().numpy().view(np.uint16),
                           v.view(torch.int16).cpu().numpy().view(np.uint16))
        k, v = blocks[blk]
        o = (int(u) % ppb) * PAGE
        kh[i * PAGE:(i + 1) * PAGE] = k[o:o + PAGE]
        vh[i * PAGE:(i + 1) * PAGE] = v[o:o + PAGE]
    kh, vh = kh[:hl0], vh[:hl0]
    kb, vb = gen.bf16_tokens(b)
    kb = kb.view(torch.int16).cpu().numpy().view(np.uint16)
    vb = vb.view(torch.int16).cpu().numpy().view(np.uint16)
    # after step 0: token 64 (the oldest recent) is demoted, the new token appended
    dem_k, dem_v = kb[SINK], vb[SINK]
    u16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    bf_k = np.concatenate([kb[:SINK], kb[SINK + 1:], u16(knew0[b:b + 1])])
    bf_v = np.concatenate([vb[:SINK], vb[SINK + 1:], u16(vnew0[b:b + 1])])
    q = synth.bf16_bits_to_f64(u16(q0[b]))
    out_ref = np.zeros((wl.Hq, D))
    lse_ref = np.zeros(wl.Hq)
    records = {}
    spent = 0.0
    cb = getattr(st, "codebook_h", None)
    for j in range(Hkv):
        # the uniform quantiser, or the Lloyd-Max codebook variant
        if cb is None:
            quant = lambda x, R, clip, kv: orc.quantize_tokens(x, R, G, clip)
            deq = lambda c, s, z, kv: orc.dequant(c, s, z, G)
        else:
            quant = lambda x, R, clip, kv: orc.quantize_tokens_codebook(x, R, G, clip, cb[j, kv])
            deq = lambda c, s, z, kv: orc.dequant_codebook(c, s, z, G, cb[j, kv])
        K = synth.bf16_bits_to_f64(kh[:, j])
        V = synth.bf16_bits_to_f64(vh[:, j])
        kc, ks, kz = quant(K, gen.R_k[j], float(gen.clip_k[j]), 0)
        vc, vs, vz = quant(V, gen.R_v[j], float(gen.clip_v[j]), 1)
        recs = []
        for pg in range(npg):
            a_, e_ = pg * PAGE, min(hl0, pg * PAGE + PAGE)
            pad = lambda x, w: np.concatenate([x[a_:e_], np.zeros((PAGE - (e_ - a_), w), x.dtype)])
            recs.append(orc.encode_record(pad(kc, D), pad(ks, D // G), pad(kz, D // G),
                                          pad(vc, D), pad(vs, D // G), pad(vz, D // G), D, G))
        records[j] = recs
        heads = [h for h in range(wl.Hq) if h // g == j]
        t0 = time.perf_counter()
        dk = quant(synth.bf16_bits_to_f64(dem_k[j])[None], gen.R_k[j], float(gen.clip_k[j]), 0)
        dv = quant(synth.bf16_bits_to_f64(dem_v[j])[None], gen.R_v[j], float(gen.clip_v[j]), 1)
        parts = [orc.decode_record(r, D, G) for r in recs]
        khat = np.concatenate([deq(p_[0], p_[1], p_[2], 0) for p_ in parts])[:hl0]
        vhat = np.concatenate([deq(p_[3], p_[4], p_[5], 1) for p_ in parts])[:hl0]
        khat = np.concatenate([khat, deq(*dk, 0)])
        vhat = np.concatenate([vhat, deq(*dv, 1)])
        o, l = orc.decode_attention(q[heads], np.zeros(len(heads), int),
                                    synth.bf16_bits_to_f64(bf_k[:, j])[:, None],
                                    synth.bf16_bits_to_f64(bf_v[:, j])[:, None],
                                    khat[:, None], vhat[:, None], gen.R_k[j:j + 1], gen.R_v[j:j + 1])
        spent += time.perf_counter() - t0
        out_ref[heads] = o
        lse_ref[heads] = l
    return out_ref, lse_ref, records, spent, (hl0 + 1 + SINK + RECENT) * Hkv


def cpu_baseline(st, first_out, budget_s=12.0, max_seqs=4, log=print):
    """Time the CPU oracle on the first decode step of a few sequences (see
    oracle_step0: the timed part unpacks and dequantises every INT2 record,
    quantises the demoted token and attends all q heads over the split cache).
    Returns the baseline dict and the oracle-vs-GPU error of the sampled
    sequences."""
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    wl = st.wl
    timed, units, worst, seqs = 0.0, 0, 0.0, 0
    for b in range(wl.B):
        if seqs >= max_seqs or (seqs > 0 and timed >= budget_s):
            break
        out_ref, _, _, spent, u = oracle_step0(st, b)
        timed += spent
        units += u
        seqs += 1
        if first_out is not None:
            got = first_out[0][b].astype(np.float64)
            den = np.maximum(np.abs(out_ref).max(axis=1), 1e-30)
            worst = max(worst, float((np.abs(got - out_ref).max(axis=1) / den).max()))
        log(f"[bench] cpu oracle: sequence {b} done, {timed:.1f}s timed so far")
    return dict(value=units / timed, unit="KV-token-heads/s", cores=int(blas_threads), kind="oracle",
                sample=f"first decode step of {seqs} of {wl.B} sequences (all {wl.Hkv} KV heads, "
                       f"{wl.Hq} q heads): unpack + dequantise every INT2 record, quantise the "
                       f"demoted token, fp64 attention; {timed:.1f}s timed",
                seconds=timed), worst


# --------------------------------------------------------------------------

def traffic_from_profile(kernel_name: str, workload: str):
    """HBM bytes per dispatch of `kernel_name` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the counter reads for a plain 1 GiB copy), or None when there is none or it
    was taken on a different version of the kernel's source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.split("(")[0].split()
    first = lambda k: kv.get(k, [""])[0] if kv.get(k) else ""
    # the sources the kernel is built from, hashed in the order listed
    srcs = [os.path.join(ROOT, "int2_rotated_kv_amd", "csrc", f) for f in kv.get("source", [])]
    if first("workload") != workload or not srcs or not all(os.path.isfile(f) for f in srcs):
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    if h.hexdigest()[:16] != first("source_sha256_16"):
        return None
    try:
        return float(first("hbm_bytes_per_dispatch"))
    except (KeyError, ValueError):
        return None


def batch1_leg(steps, warmup, cold_steps, log, compare=True):
    """The 102400-token single sequence (Qwen3-8B shape; 100K context at
    batch 1) in the same process: hot steps, the two cold protocols, the INT2
    launch alone, and the same steps on a BF16 history (the pages' batch-1
    comparison).  Returns the JSON object of the leg."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    T = steps + warmup + breakdown_steps(steps) + 2 * cold_steps
    st = build_workload("qwen3-8b-100k-b1", T, log=log, bf16_history=compare)
    wl = st.wl
    r = run_steps(st, steps, warmup, ob.INT2_AUTO, cold_steps=cold_steps, prewarm_s=0.2)
    timed = range(warmup, warmup + steps)
    ms = 1000.0 * r["wall_s"] / steps
    kvth = np.mean([int(st.hl_h[s].sum() + st.bl_h[s].sum()) * wl.Hkv for s in timed])
    splits, _, _, kind = ob.decode_plan(st.sc.cache, r["args"][warmup])
    i2 = int2_alg_bytes(wl, st.hl_h[r["int2_only_step"]], splits)[0]
    seg = r["seg_ms"]
    leg = {
        "workload": wl.name, "batch": wl.B, "context": int(wl.lengths[0]), "steps": steps,
        "ms_per_step": ms, "value": kvth / (ms * 1e-3), "unit": "KV-token-heads/s",
        "ms_per_step_separate_calls": r["ms_separate"],
        "ms_per_step_graph": r.get("graph", {}).get("ms_per_step"),
        "step_ms_breakdown": {"demote+write": float(seg[:, 0].mean()), "qrot+bf16": float(seg[:, 1].mean()),
                              "int2": float(seg[:, 2].mean()), "merge": float(seg[:, 3].mean())},
        "int2_hot": {"launch_ms": r["int2_only_ms"], "alg_bytes": i2,
                     "frac": i2 / (r["int2_only_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    for name in ("read", "write"):
        c = r.get(f"cold_{name}")
        if c is None:
            continue
        i2c = int2_alg_bytes(wl, st.hl_h[c["int2_step"]], splits)[0]
        leg[f"cold_{name}"] = {
            "ms_per_step": c["ms"], "int2_launch_ms": c["int2_ms"],
            "int2_frac": i2c / (c["int2_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "protocol": f"512 MiB scratch {name} on the stream before each step / launch",
        }
    if compare:
        rb = run_steps_bf16(st, steps, warmup)
        ms_b = 1000.0 * rb["wall_s"] / steps
        leg["bf16_history"] = {"ms_per_step": ms_b, "int2_speedup": ms_b / ms,
                               "hist_kernel_ms": rb["hist_ms"]}
    log(f"[bench] batch 1: {ms:.4f} ms/step hot, INT2 {r['int2_only_ms'] * 1000:.1f} us hot"
        + (f", {leg['cold_read']['ms_per_step'] * 1000:.1f} us/step read-cold" if "cold_read" in leg else ""))
    del st
    torch.cuda.empty_cache()
    return leg


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3-8b-b32-100k")
    ap.add_argument("--int2-kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0,
                    help="history chunks per (sequence, KV head); 0 = the library's choice")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--cold", action="store_true",
                    help="also time --steps steps each preceded by a 512 MiB scratch read, and "
                         "as many preceded by a 512 MiB scratch write (cache-cold protocols for "
                         "caches that fit the last-level cache)")
    ap.add_argument("--no-bf16-compare", action="store_true",
                    help="skip the comparison run over the same tokens with the whole "
                         "history kept in BF16 pages")
    ap.add_argument("--codebook", nargs="?", const="fit", default=None, choices=["fit", "symmetric"],
                    help="use the Lloyd-Max codebook variant of the INT2 history (seeded levels; "
                         "'symmetric': levels symmetric about the middle of the range, whose "
                         "third code plane the matrix-core kernel skips)")
    ap.add_argument("--group-size", type=int, default=0, metavar="G",
                    help="replace the workload's quantisation group size (32, 64 or 128)")
    ap.add_argument("--q-heads", type=int, default=0, metavar="HQ",
                    help="replace the workload's number of q heads (a multiple of its KV heads)")
    ap.add_argument("--no-shared", action="store_true",
                    help="do not pass the shared-prefix pages to the library (every sequence then "
                         "reads its aliased pages on its own)")
    ap.add_argument("--no-batch1", action="store_true",
                    help="skip the 102400-token batch-1 leg that the default run adds")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device-to-device copies of BYTES bytes (the "
                         "reference for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE) and exit")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {a.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch
    from int2_rotated_kv_amd import binding as ob

    log = lambda m: print(m, file=sys.stderr, flush=True)
    if a.calibrate_copy:
        src = torch.ones(a.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {a.calibrate_copy} bytes 5 times")
        return
    kern = {"auto": ob.INT2_AUTO, "valu": ob.INT2_VALU, "mfma": ob.INT2_MFMA}[a.int2_kernel]
    torch.cuda.set_device(0)
    cold_steps = a.steps if a.cold else 0
    st = build_workload(a.workload, a.steps + a.warmup + breakdown_steps(a.steps) + 2 * cold_steps,
                        log=log, bf16_history=not a.no_bf16_compare, codebook=a.codebook,
                        group_size=a.group_size, q_heads=a.q_heads)
    wl = st.wl
    if a.no_shared:
        st.shared = []
    r = run_steps(st, a.steps, a.warmup, kern, keep_first_out=not a.no_cpu_baseline,
                  num_splits=a.splits, cold_steps=cold_steps, prewarm_s=0.3)
    log(f"[bench] timed {a.steps} steps in {r['wall_s']:.3f}s")

    # per-step quantities over the timed steps
    timed = range(a.warmup, a.warmup + a.steps)
    ms_step = 1000.0 * r["wall_s"] / a.steps
    kvth = np.mean([int(st.hl_h[s].sum() + st.bl_h[s].sum()) * wl.Hkv for s in timed])
    splits, _, _, kind = ob.decode_plan(st.sc.cache, r["args"][a.warmup])
    step_bytes = np.mean([step_alg_bytes(wl, st.hl_h[s], st.bl_h[s], splits) for s in timed])
    seg = r["seg_ms"]
    int2_ms = float(seg[:, 2].mean())
    i2_last = int2_alg_bytes(wl, st.hl_h[r["int2_only_step"]], splits)[0]
    achieved = i2_last / (r["int2_only_ms"] * 1e-3) / 1e9
    kname = "k_int2_mfma" if kind == ob.INT2_MFMA else "k_int2_valu"
    # the committed counter summaries are taken with uniform codes
    tr = None if a.codebook else traffic_from_profile(kname, wl.name)
    out = {
        "metric": "decode attention: KV-tokens·heads/s and achieved HBM TB/s (% of peak) at 100K ctx",
        "value": kvth / (ms_step * 1e-3),
        "unit": "KV-token-heads/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32-accum (int8 QK pieces, f16 PV weights)",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "kv_heads": wl.Hkv, "q_heads": wl.Hq,
                   "head_dim": wl.D, "group": wl.G, "mean_context": float(np.mean(wl.lengths)),
                   "sink": SINK, "recent": RECENT, "page": PAGE, "int2_kernel": kname,
                   "splits": splits,
                   "codebook": {"fit": "lloyd-max", "symmetric": "lloyd-max-symmetric"}.get(a.codebook, "uniform"),
                   "shared_pages": [list(x) for x in st.shared],
                   "parallelism": "single-gpu"},
        "hbm_tbps": step_bytes / (ms_step * 1e-3) / 1e12,
        "hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "ms_per_step_separate_calls": r["ms_separate"],
        "ms_per_step_graph": r.get("graph", {}).get("ms_per_step"),
        "graph": r.get("graph"),
        "step_ms_breakdown": {"demote+write": float(seg[:, 0].mean()), "qrot+bf16": float(seg[:, 1].mean()),
                              "int2": int2_ms, "merge": float(seg[:, 3].mean())},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": tr, "kernel": kname,
                     "alg_bytes_per_launch": i2_last, "launch_ms": r["int2_only_ms"]},
    }
    if cold_steps:
        for name in ("read", "write"):
            c = r[f"cold_{name}"]
            i2c = int2_alg_bytes(wl, st.hl_h[c["int2_step"]], splits)[0]
            kv_c = np.mean([int(st.hl_h[s].sum() + st.bl_h[s].sum()) * wl.Hkv for s in c["steps"]])
            out[f"cold_{name}"] = {
                "ms_per_step": c["ms"], "value": kv_c / (c["ms"] * 1e-3),
                "int2_kernel_ms": c["int2_ms"],
                "int2_achieved_GBs": i2c / (c["int2_ms"] * 1e-3) / 1e9,
                "int2_frac": i2c / (c["int2_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "protocol": f"each step (and each INT2 launch) preceded by a 512 MiB scratch {name} "
                            "on the stream; HIP events around the step (launch) alone",
            }
            log(f"[bench] cold ({name}): {c['ms']:.4f} ms/step, INT2 {c['int2_ms'] * 1000:.1f} us")
    out["bulk_quantize"] = measure_bulk_quantize(st)
    if not a.no_bf16_compare:
        rb = run_steps_bf16(st, a.steps, a.warmup)
        ms_b = 1000.0 * rb["wall_s"] / a.steps
        hist_b = np.mean([int(st.hl_h[s].sum()) for s in timed]) * wl.Hkv * 2 * wl.D * 2
        hl_last = st.hl_h[a.steps + a.warmup - 1]
        out["bf16_history"] = {
            "ms_per_step": ms_b, "value": kvth / (ms_b * 1e-3), "unit": "KV-token-heads/s",
            "int2_speedup": ms_b / ms_step,
            "hist_kernel": "k_bf16_hist", "hist_kernel_ms": rb["hist_ms"],
            "hist_kernel_GBs": float(hl_last.sum()) * wl.Hkv * 2 * wl.D * 2 / (rb["hist_ms"] * 1e-3) / 1e9,
            "hist_bytes_per_step": hist_b,
            "what": "same steps, same tokens, whole history in BF16 pages (no rotation or "
                    "quantisation): copy the demoted token into the BF16 history, write the "
                    "new token, BF16 window + BF16 history attention, merge",
        }
        log(f"[bench] BF16-history comparison: {ms_b:.4f} ms/step, INT2 speed-up "
            f"{ms_b / ms_step:.2f}x")
    if not a.no_cpu_baseline:
        cb, worst = cpu_baseline(st, r["first_out"], budget_s=a.cpu_budget, log=log)
        out["cpu_baseline"] = cb
        out["sampled_parity_max_rel_err"] = worst
    if a.workload != "qwen3-8b-100k-b1" and not a.no_batch1 and not a.codebook:
        # the other 100K-context configuration: one sequence, batch 1
        st.cmp_cache = None
        del st, r
        torch.cuda.empty_cache()
        out["batch1_100k"] = batch1_leg(min(a.steps, 100), max(a.warmup, 10), min(a.steps, 50), log)
    print(json.dumps(out), flush=True)
    # release device memory before the interpreter's own teardown
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
