"""GPU parity at full size: the large caches (the batch-32 Qwen3-8B-shaped cache
at ~96K context that bench.py measures, a single 102400-token sequence, and the
Qwen3-32B-shaped shared-prefix batch), built and run in the configuration
bench.py times (automatic kernel choice and chunking), one decode step.
Checked against the oracle on sampled outputs:

* every q head of eight sequences spread over the batch of 32 (of the one
  sequence of the 102400-token cache, of every sequence in the shared-prefix
  batch): outputs within 2e-3 row relative error, lse within 1e-3 (the
  oracle quantises the sequence's history from the same generated tokens, in
  fp64, and attends it);
* the bytes of 48 sampled history pages of those sequences (all KV heads)
  equal the oracle's encoded records, and so do the written token rows of the
  page that received the step's demoted token."""
import sys
import time

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3
PAGE, SINK = 16, 64


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _u16(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _history_tokens(gen, b, hl0):
    """BF16 history tokens [hl0][Hkv][D] of sequence b as generated."""
    ppb = synth.LargeGen.PAGES_PER_BLOCK
    npg = -(-hl0 // PAGE)
    us = gen.unique_of[b, :npg]
    kh = np.empty((npg * PAGE, gen.wl.Hkv, gen.wl.D), np.uint16)
    vh = np.empty_like(kh)
    cur, kv = -1, None
    for i, u in enumerate(us):
        blk = int(u) // ppb
        if blk != cur:
            k, v = gen.history_block(blk)
            kv, cur = (_u16(k), _u16(v)), blk
        o = (int(u) % ppb) * PAGE
        kh[i * PAGE:(i + 1) * PAGE] = kv[0][o:o + PAGE]
        vh[i * PAGE:(i + 1) * PAGE] = kv[1][o:o + PAGE]
    return kh[:hl0], vh[:hl0]


def _check_sequences(st, first_out, pool, seqs, rng, codebook=None):
    """Oracle check of step 0 for the sequences `seqs`: every q head's output
    and lse, the bytes of 48 sampled prompt pages and of the page that
    received the demoted token.  Prompt-history pages are quantised once per
    unique page (sequences that share a prefix or a whole prompt alias the
    same pages), one KV head at a time."""
    from oracle import oscar_oracle as orc
    wl, gen = st.wl, st.gen
    D, G, Hkv, g = wl.D, wl.G, wl.Hkv, wl.g
    f64 = synth.bf16_bits_to_f64
    ppb = synth.LargeGen.PAGES_PER_BLOCK
    hl0 = {b: int(gen.hist_len0[b]) for b in seqs}
    npg = {b: -(-hl0[b] // PAGE) for b in seqs}
    us = np.unique(np.concatenate([gen.unique_of[b, :npg[b]] for b in seqs]))
    # prompt-history tokens of those unique pages, rows 16*i + t for us[i]
    kh = np.empty((us.size * PAGE, Hkv, D), np.uint16)
    vh = np.empty_like(kh)
    for blk in np.unique(us // ppb):
        sel = np.nonzero(us // ppb == blk)[0]
        k, v = gen.history_block(int(blk))
        k, v = _u16(k).reshape(ppb, PAGE, Hkv, D), _u16(v).reshape(ppb, PAGE, Hkv, D)
        kh.reshape(-1, PAGE, Hkv, D)[sel] = k[us[sel] % ppb]
        vh.reshape(-1, PAGE, Hkv, D)[sel] = v[us[sel] % ppb]
    rows = {b: (np.searchsorted(us, gen.unique_of[b, :npg[b]])[:, None] * PAGE
                + np.arange(PAGE)[None, :]).reshape(-1)[:hl0[b]] for b in seqs}
    knew, vnew, q0 = gen.step_tokens(0)
    knew, vnew, q0 = _u16(knew), _u16(vnew), _u16(q0)
    win = {}
    for b in seqs:
        kb, vb = gen.bf16_tokens(b)
        win[b] = (_u16(kb), _u16(vb))
    if codebook is None:
        quant = lambda x, R, clip, j, kv: orc.quantize_tokens(x, R, G, clip)
        deq = lambda c, s, z, j, kv: orc.dequant(c, s, z, G)
    else:
        quant = lambda x, R, clip, j, kv: orc.quantize_tokens_codebook(x, R, G, clip, codebook[j, kv])
        deq = lambda c, s, z, j, kv: orc.dequant_codebook(c, s, z, G, codebook[j, kv])
    out_ref = {b: np.zeros((wl.Hq, D)) for b in seqs}
    lse_ref = {b: np.zeros(wl.Hq) for b in seqs}
    sample = {b: np.sort(rng.choice(npg[b] - 1, size=min(48, npg[b] - 1), replace=False)) for b in seqs}
    for j in range(Hkv):
        qk = quant(f64(kh[:, j]), gen.R_k[j], float(gen.clip_k[j]), j, 0)
        qv = quant(f64(vh[:, j]), gen.R_v[j], float(gen.clip_v[j]), j, 1)
        xk, xv = deq(*qk, j, 0), deq(*qv, j, 1)
        heads = [h for h in range(wl.Hq) if h // g == j]
        for b in seqs:
            kb, vb = win[b]
            # step 0: the oldest recent token (window position 64) is demoted
            # to history position hl0, the new token appended to the window
            dk = quant(f64(kb[SINK:SINK + 1, j]), gen.R_k[j], float(gen.clip_k[j]), j, 0)
            dv = quant(f64(vb[SINK:SINK + 1, j]), gen.R_v[j], float(gen.clip_v[j]), j, 1)
            r = rows[b]
            hk = [np.concatenate([a[r], d]) for a, d in zip(qk, dk)]
            hv = [np.concatenate([a[r], d]) for a, d in zip(qv, dv)]
            for pg in sample[b]:
                sl = slice(pg * PAGE, (pg + 1) * PAGE)
                want = orc.encode_record(*(a[sl] for a in hk), *(a[sl] for a in hv), D, G)
                ph = gen.hist_table[b, pg]
                assert np.array_equal(pool[ph, j], want), \
                    f"seq {b} page {pg} (physical {ph}) head {j}: bytes differ"
            pg = hl0[b] // PAGE                   # the page that received the demoted token
            n = hl0[b] + 1 - pg * PAGE
            got = orc.decode_record(pool[gen.hist_table[b, pg], j], D, G)
            for a, w in zip(got, (*hk, *hv)):
                assert np.array_equal(a[:n], w[pg * PAGE:pg * PAGE + n]), \
                    f"seq {b} page {pg} head {j}: demoted token's page differs"
            bf_k = np.concatenate([kb[:SINK], kb[SINK + 1:], knew[b:b + 1]])[:, j]
            bf_v = np.concatenate([vb[:SINK], vb[SINK + 1:], vnew[b:b + 1]])[:, j]
            xhk = np.concatenate([xk[r], deq(*dk, j, 0)])
            xhv = np.concatenate([xv[r], deq(*dv, j, 1)])
            o, l = orc.decode_attention(f64(q0[b][heads]), np.zeros(len(heads), int),
                                        f64(bf_k)[:, None], f64(bf_v)[:, None],
                                        xhk[:, None], xhv[:, None], gen.R_k[j:j + 1], gen.R_v[j:j + 1])
            out_ref[b][heads], lse_ref[b][heads] = o, l
    worst = 0.0
    for b in seqs:
        got = first_out[0][b].astype(np.float64)
        den = np.maximum(np.abs(out_ref[b]).max(axis=1), 1e-30)
        err = np.abs(got - out_ref[b]).max(axis=1) / den
        assert np.all(err <= TOL), f"seq {b}: row errors {np.sort(err)[-4:]}"
        lerr = np.abs(first_out[1][b] - lse_ref[b]).max()
        assert lerr < 1e-3, f"seq {b}: lse error {lerr}"
        worst = max(worst, float(err.max()))
    return worst


@pytest.mark.parametrize("workload,codebook", [("qwen3-8b-b32-100k", False), ("qwen3-8b-100k-b1", False),
                                               ("qwen3-32b-b16-128k", False), ("qwen3-8b-100k-b1", True)])
def test_full_size_sampled(workload, codebook):
    """Batch-32 ~96K (the benchmark workload), one 102400-token sequence, and
    the Qwen3-32B-shaped batch 16 x 131072 with a shared 32768-token prefix
    (8 q heads per KV head, group 128); and the 102400-token sequence with the
    Lloyd-Max codebook variant (bench.py --codebook)."""
    import bench
    from int2_rotated_kv_amd import binding as ob
    t0 = time.time()
    _say(f"case: {workload}{' with codebook' if codebook else ''}, one decode step (bench configuration)")
    st = bench.build_workload(workload, 1, log=_say, codebook=codebook)
    r = bench.run_steps(st, 0, 1, ob.INT2_AUTO, keep_first_out=True)
    plan = ob.decode_plan(st.sc.cache, r["args"][0])
    assert st.sc.cache.read_status() == 0, f"cache status {st.sc.cache.read_status()}"
    _say(f"step done: chunks {plan[0]}, kernel {plan[3]}, {time.time() - t0:.1f}s")
    pool = st.sc.cache.int2.cpu().numpy()
    rng = np.random.default_rng(0)
    # every sequence of the shared-prefix batch (its pages are quantised once);
    # of the batch of 32, eight spread over the batch (the balanced schedule
    # splits most sequences across two or three blocks, at different offsets)
    if st.wl.shared_prefix:
        seqs = list(range(st.wl.B))
    else:
        seqs = sorted({int(round(i * (st.wl.B - 1) / 7)) for i in range(8)})
    w = _check_sequences(st, r["first_out"], pool, seqs, rng, codebook=st.codebook_h)
    _say(f"sequences {seqs}: bytes of sampled and demoted-token pages exact, worst row rel err "
         f"{w:.3e} ({time.time() - t0:.1f}s)")


CHECK_STEPS = (0, 1, 499, 999)


def test_long_decode_1000_steps():
    """The single 102400-token sequence over 1000 decode steps, each one
    oscar_decode_step (demote the oldest recent token, store the new one,
    attend, merge), in the configuration bench.py times.  At steps 0, 1, 499
    and 999 every q head is checked against the oracle, which replays the same
    steps: the token demoted at step s is the s-th of the window's tokens in
    arrival order (the 256 prompt tokens of the recent window, then the new
    tokens of steps 0, 1, ...), so after step s the history is the prompt
    history followed by the first s+1 of them, and the BF16 segment is the sink
    plus the next 256.  After the last step, the bytes of every page that the
    steps filled, and of 16 sampled prompt pages, equal the oracle's records."""
    import torch
    import bench
    from oracle import oscar_oracle as orc
    from int2_rotated_kv_amd import binding as ob
    t0 = time.time()
    T = CHECK_STEPS[-1] + 1
    _say(f"case: qwen3-8b-100k-b1, {T} decode steps, checks at {CHECK_STEPS}")
    st = bench.build_workload("qwen3-8b-100k-b1", T, log=_say)
    wl, gen, cache = st.wl, st.gen, st.sc.cache
    D, G, Hkv, g = wl.D, wl.G, wl.Hkv, wl.g
    args = [bench.step_args(st, s, ob.INT2_AUTO) for s in range(T)]
    ws = torch.empty(max(ob.workspace_bytes(cache, a) for a in args), dtype=torch.uint8,
                     device=st.q.device)
    out = torch.zeros((wl.B, wl.Hq, D), dtype=torch.float32, device=st.q.device)
    lse = torch.zeros((wl.B, wl.Hq), dtype=torch.float32, device=st.q.device)
    got = {}
    for s in range(T):
        ob.decode_step(cache, args[s], st.dsrc[s], st.ddst[s], st.ck, st.cv, st.wdst[s],
                       st.knew[s], st.vnew[s], st.q[s], st.Rk, st.Rv, ws, out, lse)
        if s in CHECK_STEPS:
            torch.cuda.synchronize()
            got[s] = (out[0].cpu().numpy().astype(np.float64), lse[0].cpu().numpy().copy())
    torch.cuda.synchronize()
    _say(f"{T} steps done ({time.time() - t0:.1f}s)")

    hl0 = int(gen.hist_len0[0])
    kh, vh = _history_tokens(gen, 0, hl0)
    kb, vb = gen.bf16_tokens(0)
    kb, vb = _u16(kb), _u16(vb)
    knew, vnew, qs = _u16(st.knew[:, 0]), _u16(st.vnew[:, 0]), _u16(st.q[:, 0])
    # window tokens in arrival order: the prompt's recent window, then the new tokens
    arr_k = np.concatenate([kb[SINK:], knew])
    arr_v = np.concatenate([vb[SINK:], vnew])
    f64 = synth.bf16_bits_to_f64
    quant = {}
    for j in range(Hkv):
        K = f64(np.concatenate([kh[:, j], arr_k[:T, j]]))
        V = f64(np.concatenate([vh[:, j], arr_v[:T, j]]))
        quant[j] = (orc.quantize_tokens(K, gen.R_k[j], G, float(gen.clip_k[j])),
                    orc.quantize_tokens(V, gen.R_v[j], G, float(gen.clip_v[j])))
    worst = 0.0
    for s in CHECK_STEPS:
        nh = hl0 + s + 1                          # history tokens after step s
        bf_k = np.concatenate([kb[:SINK], arr_k[s + 1:s + 1 + 256]])
        bf_v = np.concatenate([vb[:SINK], arr_v[s + 1:s + 1 + 256]])
        q = f64(qs[s])
        out_ref = np.zeros((wl.Hq, D))
        lse_ref = np.zeros(wl.Hq)
        for j in range(Hkv):
            (kc, ks, kz), (vc, vs, vz) = quant[j]
            heads = [h for h in range(wl.Hq) if h // g == j]
            o, l = orc.decode_attention(q[heads], np.zeros(len(heads), int),
                                        f64(bf_k[:, j])[:, None], f64(bf_v[:, j])[:, None],
                                        orc.dequant(kc[:nh], ks[:nh], kz[:nh], G)[:, None],
                                        orc.dequant(vc[:nh], vs[:nh], vz[:nh], G)[:, None],
                                        gen.R_k[j:j + 1], gen.R_v[j:j + 1])
            out_ref[heads], lse_ref[heads] = o, l
        o_gpu, l_gpu = got[s]
        den = np.maximum(np.abs(out_ref).max(axis=1), 1e-30)
        err = np.abs(o_gpu - out_ref).max(axis=1) / den
        assert np.all(err <= TOL), f"step {s}: row errors {np.sort(err)[-4:]}"
        lerr = np.abs(l_gpu - lse_ref).max()
        assert lerr < 1e-3, f"step {s}: lse error {lerr}"
        worst = max(worst, float(err.max()))
        _say(f"step {s}: {nh} history tokens, worst row rel err {err.max():.3e}, "
             f"lse err {lerr:.2e} ({time.time() - t0:.1f}s)")

    # page bytes after the last step: the pages the steps filled (the last one
    # partially: its written token rows are compared) and sampled prompt pages
    pool = cache.int2.cpu().numpy()
    nh = hl0 + T
    rng = np.random.default_rng(1)
    pages = list(range(hl0 // PAGE, -(-nh // PAGE)))
    pages += sorted(rng.choice(hl0 // PAGE, size=16, replace=False).tolist())
    for pg in pages:
        ph = int(st.sc.hist_table_h[0, pg])
        ntok = min(PAGE, nh - pg * PAGE)
        sl = slice(pg * PAGE, pg * PAGE + ntok)
        for j in range(Hkv):
            (kc, ks, kz), (vc, vs, vz) = quant[j]
            if ntok == PAGE:
                want = orc.encode_record(kc[sl], ks[sl], kz[sl], vc[sl], vs[sl], vz[sl], D, G)
                assert np.array_equal(pool[ph, j], want), f"page {pg} head {j}: bytes differ"
            else:
                dk = orc.decode_record(pool[ph, j], D, G)
                for a, w in zip(dk, (kc[sl], ks[sl], kz[sl], vc[sl], vs[sl], vz[sl])):
                    assert np.array_equal(a[:ntok], w), f"page {pg} head {j}: partial page differs"
    _say(f"bytes of {len(pages)} pages x {Hkv} heads exact; worst row rel err {worst:.3e} "
         f"({time.time() - t0:.1f}s)")
