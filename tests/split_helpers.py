"""Shared helpers of the GPU parity tests: build a split cache on the device
through the library, and compute the same step with the CPU oracle.

Inputs come only from synth; expected values only from oracle.  The two sides
meet here and nowhere else."""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

import synth
from oracle import oscar_oracle as orc

PAGE, SINK, RECENT = 16, 64, 256


def to_dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


@dataclass
class DeviceRun:
    sc: object            # SplitCache
    out: np.ndarray       # [B][Hq][D] float32
    lse: np.ndarray       # [B][Hq]
    pool: np.ndarray      # INT2 pool bytes [pages][Hkv][rec]
    hist_len: np.ndarray  # per sequence after the steps
    bf16_k: np.ndarray = None   # BF16 pools after the steps
    bf16_v: np.ndarray = None
    status: int = 0             # the cache's sticky OSCAR_STATUS_* word


def hist_capacity_pages(L: int, steps: int) -> int:
    s, h, r = synth.split_lengths(L)
    return max(1, -(-(h + steps) // PAGE))


def build_and_step(inp: synth.SmallInputs, steps: int = 1, int2_kernel=1, num_splits=0,
                   R_v_none=False, head_map=None, device="cuda", seed_perm=None, fused=False,
                   flags=0, codebook=None, max_hist_len=None, extra_pages=0, noalloc=False,
                   shared=None, graph=False, on_step=None):
    """Build the initial split cache of every sequence, run `steps` decode steps
    (demote oldest recent -> write new token -> attend -> merge; with fused,
    through the single oscar_decode_step call, with noalloc through
    oscar_decode_step_noalloc), return the outputs of the last step and the
    INT2 pool.  shared: [(first_page, num_pages, seq_begin, num_seqs)], whose
    member sequences' page tables then list seq_begin's physical pages there
    (their tokens must be equal: synth.share_history); passed to the decode
    calls as oscar_shared_pages.  graph: every step is one replay of a HIP
    graph holding one oscar_decode_step, captured at the first step (its
    arguments planned for max_hist_len or the lengths after the last step);
    each step copies its slot lists, new token and query into the captured
    buffers and the lengths into the cache first (every sequence must demote
    at every step, so that the call's shape stays the same).  on_step(st,
    out, lse) is called after each step with host copies."""
    import torch
    from int2_rotated_kv_amd import binding as ob
    from int2_rotated_kv_amd.splitcache import SplitCache

    wl = inp.wl
    B = wl.B
    caps = [hist_capacity_pages(L, steps) + extra_pages for L in wl.lengths]
    stride = max(caps)
    n_int2 = sum(caps)
    perm = synth.page_permutation(wl.seed if seed_perm is None else seed_perm, n_int2, extra=3)
    table = np.zeros((B, stride), dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :caps[b]] = perm[o:o + caps[b]]
        o += caps[b]
    for (first, num, s0, n) in (shared or []):
        for b in range(s0 + 1, s0 + n):
            table[b, first:first + num] = table[s0, first:first + num]
    cb = None if codebook is None else torch.from_numpy(np.asarray(codebook, np.float32)).to(device)
    sc = SplitCache(B, wl.Hkv, wl.Hq, wl.D, wl.G, table, n_int2 + 3, staging_pages=64, device=device,
                    codebook=cb)
    Rk = torch.from_numpy(inp.R_k).to(device)
    Rv = None if R_v_none else torch.from_numpy(inp.R_v).to(device)
    ck = torch.from_numpy(inp.clip_k).to(device)
    cv = torch.from_numpy(inp.clip_v).to(device)
    entries = []
    for b in range(B):
        L = wl.lengths[b]
        s, h, r = synth.split_lengths(L)
        K, V = inp.K[b], inp.V[b]
        bidx = list(range(0, s)) + list(range(s + h, L))
        sc.load_bf16(b, to_dev_bf16(K[bidx]), to_dev_bf16(V[bidx]))
        if h:
            entries.append((b, 0, to_dev_bf16(K[s:s + h]), to_dev_bf16(V[s:s + h])))
    sc.fill_history(entries, Rk, Rv, ck, cv)

    out = torch.zeros((B, wl.Hq, wl.D), dtype=torch.float32, device=device)
    lse = torch.zeros((B, wl.Hq), dtype=torch.float32, device=device)
    if graph:
        assert all(L >= 320 for L in wl.lengths), "every sequence demotes at every step"
        mh = int(sc.hist_len_h.max()) + steps if max_hist_len is None else max_hist_len
        args = sc.decode_args(max_hist_len=mh, kv_head_of_q=head_map, num_splits=num_splits,
                              int2_kernel=int2_kernel, flags=flags, shared=shared)
        ws = ob.alloc_workspace(sc.cache, args, device=device)
        bufs = None
        g = None
        for st in range(steps):
            dsrc, ddst, wdst = sc.plan_step()
            newk = np.stack([inp.K[b][wl.lengths[b] + st] for b in range(B)])
            newv = np.stack([inp.V[b][wl.lengths[b] + st] for b in range(B)])
            vals = [torch.from_numpy(x).to(device) for x in (dsrc, ddst, wdst)]
            vals += [to_dev_bf16(newk).view(torch.int16), to_dev_bf16(newv).view(torch.int16),
                     to_dev_bf16(inp.q[st]).view(torch.int16)]
            if bufs is None:
                bufs = [v.clone() for v in vals]
            else:
                for dst, v in zip(bufs, vals):
                    dst.copy_(v)
            sc.commit_step()
            sc.sync_lengths()
            d_src, d_dst, d_w, kn, vn, q = bufs
            if g is None:
                ob.decode(sc.cache, args, q, Rk, Rv, out, lse)      # warm-up, reads only
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    ob.decode_step(sc.cache, args, d_src, d_dst, ck, cv, d_w, kn, vn, q, Rk, Rv, ws, out, lse)
                torch.cuda.synchronize()
            out.fill_(float(st + 1))                                 # eager work between replays
            lse.zero_()
            g.replay()
            torch.cuda.synchronize()
            if on_step is not None:
                on_step(st, out.cpu().numpy(), lse.cpu().numpy())
        return DeviceRun(sc, out.cpu().numpy(), lse.cpu().numpy(), sc.cache.int2.cpu().numpy(),
                         sc.hist_len_h.copy(), sc.cache.bf16_k.cpu().numpy(), sc.cache.bf16_v.cpu().numpy(),
                         sc.cache.read_status())
    for st in range(steps):
        dsrc, ddst, wdst = sc.plan_step()
        newk = np.stack([inp.K[b][wl.lengths[b] + st] for b in range(B)])
        newv = np.stack([inp.V[b][wl.lengths[b] + st] for b in range(B)])
        kn, vn = to_dev_bf16(newk).view(torch.int16), to_dev_bf16(newv).view(torch.int16)
        d_src, d_dst, d_w = (torch.from_numpy(x).to(device) for x in (dsrc, ddst, wdst))
        q = to_dev_bf16(inp.q[st]).view(torch.int16)
        if noalloc:
            sc.commit_step()
            sc.sync_lengths()
            args = sc.decode_args(max_hist_len=max_hist_len, kv_head_of_q=head_map, num_splits=num_splits,
                                  int2_kernel=int2_kernel, flags=flags, shared=shared)
            ob.decode_step_noalloc(sc.cache, args, d_src, d_dst, ck, cv, d_w, kn, vn, q, Rk, Rv, out, lse)
            continue
        if not fused:
            ob.demote_pack(sc.cache, d_src, d_dst, Rk, Rv, ck, cv)
            ob.write_bf16(sc.cache, d_w, kn, vn)
        sc.commit_step()
        sc.sync_lengths()
        args = sc.decode_args(max_hist_len=max_hist_len, kv_head_of_q=head_map, num_splits=num_splits,
                              int2_kernel=int2_kernel, flags=flags, shared=shared)
        if fused:
            ws = ob.alloc_workspace(sc.cache, args, device=q.device)
            ob.decode_step(sc.cache, args, d_src, d_dst, ck, cv, d_w, kn, vn, q, Rk, Rv, ws, out, lse)
        else:
            ob.decode(sc.cache, args, q, Rk, Rv, out, lse)
        if on_step is not None:
            torch.cuda.synchronize()
            on_step(st, out.cpu().numpy(), lse.cpu().numpy())
    torch.cuda.synchronize()
    return DeviceRun(sc, out.cpu().numpy(), lse.cpu().numpy(), sc.cache.int2.cpu().numpy(),
                     sc.hist_len_h.copy(), sc.cache.bf16_k.cpu().numpy(), sc.cache.bf16_v.cpu().numpy(),
                     sc.cache.read_status())


def oracle_step(inp: synth.SmallInputs, steps: int = 1, R_v_none=False, head_map=None,
                seqs=None, heads=None, codebook=None):
    """Oracle view after `steps` decode steps: history quantised from the
    original tokens (with codebook [Hkv][2][4]: the Lloyd-Max variant), BF16 =
    sink + current recent window.  Returns per sequence (out [Hq][D], lse [Hq],
    quantised history dict)."""
    wl = inp.wl
    D, G = wl.D, wl.G
    hm = np.array(head_map) if head_map is not None else orc.default_head_map(wl.Hq, wl.Hkv)
    res = {}
    for b in (range(wl.B) if seqs is None else seqs):
        L = wl.lengths[b] + steps
        s, h, r = synth.split_lengths(L)
        K = synth.bf16_bits_to_f64(inp.K[b][:L])
        V = synth.bf16_bits_to_f64(inp.V[b][:L])
        kc = np.zeros((h, wl.Hkv, D), np.uint8); vc = np.zeros_like(kc)
        ks = np.zeros((h, wl.Hkv, D // G)); kz = np.zeros_like(ks); vs = np.zeros_like(ks); vz = np.zeros_like(ks)
        khat = np.zeros((h, wl.Hkv, D)); vhat = np.zeros_like(khat)
        for j in range(wl.Hkv):
            if h == 0:
                break
            Rv = np.eye(D) if R_v_none else inp.R_v[j]
            if codebook is None:
                c1, s1, z1 = orc.quantize_tokens(K[s:s + h, j], inp.R_k[j], G, float(inp.clip_k[j]))
                c2, s2, z2 = orc.quantize_tokens(V[s:s + h, j], Rv, G, float(inp.clip_v[j]))
                khat[:, j] = orc.dequant(c1, s1, z1, G)
                vhat[:, j] = orc.dequant(c2, s2, z2, G)
            else:
                lk, lv = codebook[j, 0], codebook[j, 1]
                c1, s1, z1 = orc.quantize_tokens_codebook(K[s:s + h, j], inp.R_k[j], G,
                                                          float(inp.clip_k[j]), lk)
                c2, s2, z2 = orc.quantize_tokens_codebook(V[s:s + h, j], Rv, G, float(inp.clip_v[j]), lv)
                khat[:, j] = orc.dequant_codebook(c1, s1, z1, G, lk)
                vhat[:, j] = orc.dequant_codebook(c2, s2, z2, G, lv)
            kc[:, j], ks[:, j], kz[:, j] = c1, s1, z1
            vc[:, j], vs[:, j], vz[:, j] = c2, s2, z2
        bidx = list(range(0, s)) + list(range(s + h, L))
        q = synth.bf16_bits_to_f64(inp.q[steps - 1][b])
        out, lse = orc.decode_attention(q, hm, K[bidx], V[bidx], khat, vhat, inp.R_k,
                                        None if R_v_none else inp.R_v)
        res[b] = dict(out=out, lse=lse, h=h, kc=kc, ks=ks, kz=kz, vc=vc, vs=vs, vz=vz)
    return res


def oracle_records(r, D, G, Hkv):
    """Expected bytes of every history page of one sequence: [pages][Hkv][rec]."""
    h = r["h"]
    npg = -(-h // PAGE)
    rec = orc.record_bytes(D, G)
    out = np.zeros((npg, Hkv, rec), np.uint8)
    for p in range(npg):
        a, e = p * PAGE, min(h, p * PAGE + PAGE)
        n = e - a
        for j in range(Hkv):
            def pad(x, fill_shape):
                y = np.zeros(fill_shape, dtype=x.dtype)
                y[:n] = x[a:e, j]
                return y
            kc = pad(r["kc"], (PAGE, D)); vc = pad(r["vc"], (PAGE, D))
            ks = pad(r["ks"], (PAGE, D // G)); kz = pad(r["kz"], (PAGE, D // G))
            vs = pad(r["vs"], (PAGE, D // G)); vz = pad(r["vz"], (PAGE, D // G))
            out[p, j] = orc.encode_record(kc, ks, kz, vc, vs, vz, D, G)
    return out


def row_rel_err(got, ref):
    """max_c |got - ref| / max_c |ref| per row (the last axis)."""
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return np.abs(got - ref).max(axis=-1) / den


def build_bf16_history_and_attend(inp: synth.SmallInputs, num_splits=0, device="cuda"):
    """The comparison layout: every sequence's history kept as BF16 pages of
    the BF16 pool (no rotation, no quantisation), sink + recent in BF16 pages
    of the same pool, every page at a seeded random physical id.  One
    decode_attn (history kind HISTORY_BF16) + merge; returns (out, lse)."""
    import torch
    from int2_rotated_kv_amd import binding as ob

    wl = inp.wl
    B, Hkv, D = wl.B, wl.Hkv, wl.D
    spl = [synth.split_lengths(L) for L in wl.lengths]
    hp = [-(-h // PAGE) for (_, h, _) in spl]
    wp = [-(-(s + r) // PAGE) for (s, _, r) in spl]
    n = sum(hp) + sum(wp)
    perm = synth.page_permutation(wl.seed + 11, n, extra=2)
    kpool = np.zeros((n + 2, Hkv, PAGE, D), np.uint16)
    vpool = np.zeros_like(kpool)
    hstride, wstride = max(1, max(hp)), max(1, max(wp))
    htab = np.zeros((B, hstride), np.int32)
    wtab = np.zeros((B, wstride), np.int32)
    o = 0
    for b in range(B):
        s, h, r = spl[b]
        K, V = inp.K[b], inp.V[b]
        for tab, idx, npg, col in ((htab, list(range(s, s + h)), hp[b], 0),
                                   (wtab, list(range(0, s)) + list(range(s + h, wl.lengths[b])), wp[b], 0)):
            for pgi in range(npg):
                ph = perm[o]; o += 1
                tab[b, pgi] = ph
                tok = idx[pgi * PAGE:(pgi + 1) * PAGE]
                kpool[ph, :, :len(tok)] = K[tok].transpose(1, 0, 2)
                vpool[ph, :, :len(tok)] = V[tok].transpose(1, 0, 2)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(device)
    cache = ob.Cache(Hkv, D, wl.G, 0, n + 2, device=device,
                     bf16_k=dev(kpool.view(np.int16)), bf16_v=dev(vpool.view(np.int16)))
    hl = np.array([h for (_, h, _) in spl], np.int32)
    bl = np.array([s + r for (s, _, r) in spl], np.int32)
    args = ob.DecodeArgs(B, wl.Hq, dev(htab), dev(hl), dev(wtab), dev(bl), int(hl.max()),
                         num_splits=num_splits, int2_kernel=ob.HISTORY_BF16)
    out = torch.zeros((B, wl.Hq, D), dtype=torch.float32, device=device)
    lse = torch.zeros((B, wl.Hq), dtype=torch.float32, device=device)
    q = to_dev_bf16(inp.q[0])
    ob.decode(cache, args, q.view(torch.int16), None, None, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_plain(inp: synth.SmallInputs):
    """Oracle attention of q (step 0) over every token of each sequence, all
    BF16 (the comparison layout): the split form with an unquantised history
    and identity rotations."""
    wl = inp.wl
    hm = orc.default_head_map(wl.Hq, wl.Hkv)
    eye = np.broadcast_to(np.eye(wl.D), (wl.Hkv, wl.D, wl.D))
    res = {}
    for b in range(wl.B):
        L = wl.lengths[b]
        s, h, r = synth.split_lengths(L)
        K = synth.bf16_bits_to_f64(inp.K[b][:L])
        V = synth.bf16_bits_to_f64(inp.V[b][:L])
        bidx = list(range(0, s)) + list(range(s + h, L))
        q = synth.bf16_bits_to_f64(inp.q[0][b])
        out, lse = orc.decode_attention(q, hm, K[bidx], V[bidx], K[s:s + h], V[s:s + h], eye, None)
        res[b] = dict(out=out, lse=lse)
    return res
