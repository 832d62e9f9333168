"""Host-side bookkeeping of the split cache for a batch of sequences.

The library is stateless: page allocation, page tables, lengths and the
recent-window ring are the caller's.  This module is that caller-side state for
tests, the benchmark and users: it owns the page tables (torch int32 tensors on
the device) and issues the library calls of one decode step:

    demote the oldest recent token of every full sequence into its INT2 history
    -> write the new token into the freed BF16 slot -> attend -> merge

Layout of one sequence's BF16 pages: 4 sink pages (slots 0..63) then 16
recent pages (slots 64..319).  The recent window is a ring: ring_head[b] is the
position (0..255) of the oldest recent token inside slots 64..319.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import binding as ob

PAGE = ob.PAGE
SINK, RECENT, MAXB = ob.SINK, ob.RECENT, ob.MAX_BF16
BF16_PAGES_PER_SEQ = MAXB // PAGE


class SplitCache:
    def __init__(self, B: int, Hkv: int, Hq: int, D: int, G: int, hist_table: np.ndarray,
                 num_int2_pages: int, staging_pages: int = 256, device="cuda", codebook=None):
        """hist_table: int32 [B][stride] physical INT2 page of each logical history
        page (entries beyond a sequence's capacity are ignored); codebook: float32
        [Hkv][2][4] device tensor of Lloyd-Max code levels, or None (uniform)."""
        import torch
        self.torch = torch
        self.B, self.Hkv, self.Hq, self.D, self.G = B, Hkv, Hq, D, G
        self.device = device
        self.staging_base = B * BF16_PAGES_PER_SEQ
        self.staging_pages = staging_pages
        self.cache = ob.Cache(Hkv, D, G, num_int2_pages, self.staging_base + staging_pages, device,
                              codebook=codebook)
        bf = np.arange(B * BF16_PAGES_PER_SEQ, dtype=np.int32).reshape(B, BF16_PAGES_PER_SEQ)
        self.bf16_pages_h = bf
        self.bf16_pages = torch.from_numpy(bf).to(device)
        self.hist_table_h = np.ascontiguousarray(hist_table, dtype=np.int32)
        self.hist_pages = torch.from_numpy(self.hist_table_h).to(device)
        self.hist_len_h = np.zeros(B, dtype=np.int64)
        self.bf16_len_h = np.zeros(B, dtype=np.int64)
        self.ring_head = np.zeros(B, dtype=np.int64)
        self.hist_len = torch.zeros(B, dtype=torch.int32, device=device)
        self.bf16_len = torch.zeros(B, dtype=torch.int32, device=device)

    # ------------------------------------------------------------------ slots
    def bf16_slot(self, b: int, pos: int) -> int:
        """Physical BF16 slot of table position pos (0..319) of sequence b."""
        return int(self.bf16_pages_h[b, pos // PAGE]) * PAGE + pos % PAGE

    def int2_slot(self, b: int, hpos: int) -> int:
        return int(self.hist_table_h[b, hpos // PAGE]) * PAGE + hpos % PAGE

    def sync_lengths(self):
        t = self.torch
        self.hist_len.copy_(t.from_numpy(self.hist_len_h.astype(np.int32)))
        self.bf16_len.copy_(t.from_numpy(self.bf16_len_h.astype(np.int32)))

    # ------------------------------------------------------------------ fill
    def load_bf16(self, b: int, k, v):
        """Initial sink + recent tokens of sequence b ([n][Hkv][D] bf16 tensors,
        n <= 320, token order: sink first, then the recent window oldest first)."""
        t = self.torch
        n = int(k.shape[0])
        assert n <= MAXB
        slots = t.tensor([self.bf16_slot(b, i) for i in range(n)], dtype=t.int32, device=self.device)
        ob.write_bf16(self.cache, slots, k.contiguous().view(t.int16), v.contiguous().view(t.int16))
        self.bf16_len_h[b] = n
        self.ring_head[b] = 0

    def fill_history(self, entries, R_k, R_v, clip_k, clip_v):
        """Quantise history tokens into INT2 slots through the staging BF16 pages.

        entries: iterable of (b, hpos0, k, v) with k, v [n][Hkv][D] bf16 device
        tensors holding history positions hpos0 .. hpos0+n-1 of sequence b.
        Demotion goes through oscar_demote_pack, the same call a decode step uses.
        """
        t = self.torch
        cap = self.staging_pages * PAGE
        base = self.staging_base * PAGE
        for (b, h0, k, v) in entries:
            n = int(k.shape[0])
            for a in range(0, n, cap):
                m = min(cap, n - a)
                src = t.arange(base, base + m, dtype=t.int32, device=self.device)
                ob.write_bf16(self.cache, src, k[a:a + m].contiguous().view(t.int16),
                              v[a:a + m].contiguous().view(t.int16))
                hp = np.arange(h0 + a, h0 + a + m)
                dst = (self.hist_table_h[b, hp // PAGE].astype(np.int64) * PAGE + hp % PAGE).astype(np.int32)
                ob.demote_pack(self.cache, src, t.from_numpy(dst).to(self.device), R_k, R_v, clip_k, clip_v)
            self.hist_len_h[b] = max(self.hist_len_h[b], h0 + n)

    def fill_history_pages(self, phys_pages: np.ndarray, k, v, R_k, R_v, clip_k, clip_v):
        """Quantise whole pages: k, v [len(phys_pages)*16][Hkv][D] go to the 16
        slots of each listed physical INT2 page (used for aliased prefix pages)."""
        t = self.torch
        cap = self.staging_pages
        base = self.staging_base * PAGE
        for a in range(0, len(phys_pages), cap):
            pp = np.asarray(phys_pages[a:a + cap], dtype=np.int64)
            m = len(pp) * PAGE
            src = t.arange(base, base + m, dtype=t.int32, device=self.device)
            ob.write_bf16(self.cache, src, k[a * PAGE:a * PAGE + m].contiguous().view(t.int16),
                          v[a * PAGE:a * PAGE + m].contiguous().view(t.int16))
            dst = (pp[:, None] * PAGE + np.arange(PAGE)[None, :]).reshape(-1).astype(np.int32)
            ob.demote_pack(self.cache, src, t.from_numpy(dst).to(self.device), R_k, R_v, clip_k, clip_v)

    # ------------------------------------------------------------------ step
    def plan_step(self):
        """Host plan of one decode step: (demote src, demote dst, write dst) slot
        lists.  Sequences whose BF16 window is not full only append."""
        dsrc, ddst, wdst = [], [], []
        for b in range(self.B):
            if self.bf16_len_h[b] >= MAXB:
                pos = SINK + int(self.ring_head[b])
                s = self.bf16_slot(b, pos)
                dsrc.append(s)
                ddst.append(self.int2_slot(b, int(self.hist_len_h[b])))
                wdst.append(s)
            else:
                wdst.append(self.bf16_slot(b, int(self.bf16_len_h[b])))
                dsrc.append(-1)
                ddst.append(-1)
        return (np.array(dsrc, np.int32), np.array(ddst, np.int32), np.array(wdst, np.int32))

    def commit_step(self):
        """Advance host lengths / ring after plan_step's calls were enqueued."""
        for b in range(self.B):
            if self.bf16_len_h[b] >= MAXB:
                self.hist_len_h[b] += 1
                self.ring_head[b] = (self.ring_head[b] + 1) % RECENT
            else:
                self.bf16_len_h[b] += 1

    def decode_args(self, max_hist_len: Optional[int] = None, **kw) -> ob.DecodeArgs:
        mh = int(self.hist_len_h.max()) if max_hist_len is None else int(max_hist_len)
        return ob.DecodeArgs(self.B, self.Hq, self.hist_pages, self.hist_len, self.bf16_pages,
                             self.bf16_len, mh, **kw)
