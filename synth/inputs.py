"""Seeded synthetic inputs for the split-cache decode path.

Every workload here is synthetic: Gaussian K/V with a few scaled outlier
channels per KV head (the pages explain INT2's difficulty by such channel-wise
outliers), Gaussian queries, and one random orthogonal rotation per KV head
built the way the pages compose it (an eigenbasis of a random SPD matrix times a
normalised Walsh-Hadamard matrix times a bit-reversal permutation).  Real model
activations, calibrated rotations and the pages' evaluation suites are not
available; these inputs stand in for their shapes, sizes and outlier structure.

This module draws random numbers and arranges them; it performs none of the
method's arithmetic on cache entries (no rotation of K/V, no quantisation, no
packing, no attention).  Building the rotation matrix itself is part of the
input recipe because calibration is not part of the hot path.

Two generators:
  * ``make_small``  numpy PCG64, host arrays; for workloads the oracle can
    evaluate in full (tiny, Qwen3-8B-shaped 32K).
  * ``LargeGen``    torch's device generator, block-seeded so that any page can
    be regenerated on demand; for the 100K-class workloads where the oracle only
    checks sampled rows and pages.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional

import numpy as np

SINK = 64          # BF16 attention-sink tokens at the start of each sequence
RECENT = 256       # BF16 recent-window tokens at the end of each sequence
PAGE = 16          # tokens per page, INT2 and BF16 pools alike


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hkv: int
    Hq: int
    D: int
    G: int
    lengths: tuple          # context length per sequence before the first step
    seed: int
    clip: float = 0.95
    n_outliers: int = 8
    outlier_scale: float = 30.0
    steps: int = 1
    shared_prefix: int = 0  # tokens of prefix whose history pages every sequence aliases
    distinct_frac: float = 0.0  # fraction of sequences with their own suffix (rest share one)
    clip_set: tuple = ()    # per-KV-head clip ratios drawn from this set, K != V per head;
                            # empty: `clip` for every head, K and V alike
    v_range: float = 0.0    # > 0: V tokens uniform in [-v_range, v_range], no outliers

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv


def _lengths_uniform(seed: int, B: int, lo: int, hi: int) -> tuple:
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=B))


# Clip ratios of the model-shaped workloads: one per (KV head, K|V), seeded,
# from a set near 1 (the ratio is a per-layer, per-head calibration constant;
# the tiny workload keeps the single 0.95 it is specified with).  The library
# and the oracle both read the float32 nearest to each value.
MODEL_CLIPS = (1.0, 0.95, 0.9, 0.85)
# A wider set for parity cases, so that a mixed-up head or K/V index changes
# bytes everywhere.
WIDE_CLIPS = (1.0, 0.8, 0.5, 0.95)

WORKLOADS: Dict[str, Workload] = {
    # 64 sink + 704 history + 256 recent, one decode step
    "tiny": Workload("tiny", B=1, Hkv=1, Hq=4, D=64, G=32, lengths=(1024,), seed=0,
                     n_outliers=4, outlier_scale=20.0),
    "qwen3-8b-32k": Workload("qwen3-8b-32k", B=1, Hkv=8, Hq=32, D=128, G=64,
                             lengths=(32768,), seed=1, clip_set=MODEL_CLIPS),
    "qwen3-8b-100k-b1": Workload("qwen3-8b-100k-b1", B=1, Hkv=8, Hq=32, D=128, G=64,
                                 lengths=(102400,), seed=2, steps=1000, clip_set=MODEL_CLIPS),
    "qwen3-8b-b32-100k": Workload("qwen3-8b-b32-100k", B=32, Hkv=8, Hq=32, D=128, G=64,
                                  lengths=_lengths_uniform(3, 32, 90000, 100000), seed=3,
                                  clip_set=MODEL_CLIPS),
    "qwen3-32b-b16-128k": Workload("qwen3-32b-b16-128k", B=16, Hkv=8, Hq=64, D=128, G=128,
                                   lengths=(131072,) * 16, seed=4, shared_prefix=32768,
                                   distinct_frac=0.2, clip_set=MODEL_CLIPS),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return dataclasses.replace(w, **overrides) if overrides else w


def split_lengths(L: int):
    """(sink, history, recent) token counts for a sequence of L tokens."""
    if L <= SINK + RECENT:
        return min(L, SINK), 0, max(0, L - SINK)
    return SINK, L - SINK - RECENT, RECENT


# ----------------------------------------------------------------------------
# rotation recipe (input construction; calibration itself is out of scope)
# ----------------------------------------------------------------------------

def _sylvester(D: int) -> np.ndarray:
    h = np.ones((1, 1))
    while h.shape[0] < D:
        h = np.block([[h, h], [h, -h]])
    return h


def _bitrev(i: int, nbits: int) -> int:
    r = 0
    for _ in range(nbits):
        r = (r << 1) | (i & 1)
        i >>= 1
    return r


def make_rotation(rng: np.random.Generator, D: int) -> np.ndarray:
    """One D x D orthogonal rotation, returned as float32 (row-vector convention x = k @ R).

    U: eigenvectors of S = A^T A / (2D), A ~ N(0,1)^{2D x D}, ordered by descending
    eigenvalue, each column's largest-magnitude entry made positive.
    R = U @ (H_D / sqrt(D)) @ P with P[i, bitrev(i)] = 1.
    """
    A = rng.standard_normal((2 * D, D))
    S = A.T @ A / (2 * D)
    w, V = np.linalg.eigh(S)
    V = V[:, np.argsort(-w, kind="stable")]
    idx = np.argmax(np.abs(V), axis=0)
    V = V * np.sign(V[idx, np.arange(D)])
    H = _sylvester(D) / math.sqrt(D)
    nb = int(round(math.log2(D)))
    P = np.zeros((D, D))
    for i in range(D):
        P[i, _bitrev(i, nb)] = 1.0
    return (V @ H @ P).astype(np.float32)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _outliers(rng: np.random.Generator, Hkv: int, D: int, n: int) -> np.ndarray:
    return np.stack([np.sort(rng.choice(D, size=n, replace=False)) for _ in range(Hkv)])


def _gaussian_kv(rng, n, Hkv, D, out_idx, scale):
    x = rng.standard_normal((n, Hkv, D), dtype=np.float32)
    for j in range(Hkv):
        x[:, j, out_idx[j]] *= np.float32(scale)
    return _f32_to_bf16_bits(x)


# ----------------------------------------------------------------------------
# small workloads: everything on the host
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class SmallInputs:
    wl: Workload
    q: np.ndarray            # uint16 bf16 bits [steps][B][Hq][D]
    K: List[np.ndarray]      # per sequence uint16 [L_b + steps][Hkv][D]  (token order)
    V: List[np.ndarray]
    R_k: np.ndarray          # float32 [Hkv][D][D]
    R_v: np.ndarray          # float32 [Hkv][D][D]
    clip_k: np.ndarray       # float32 [Hkv]
    clip_v: np.ndarray
    out_k: np.ndarray        # outlier channel indices [Hkv][n]
    out_v: np.ndarray


def clip_ratios(wl: Workload):
    """float32 [Hkv] clip ratios for K and for V.  With wl.clip_set: per KV
    head a seeded pair of distinct values of the set (K != V); otherwise
    wl.clip everywhere.  Drawn from their own generator, so the token streams
    do not depend on it."""
    if not wl.clip_set:
        c = np.full(wl.Hkv, wl.clip, dtype=np.float32)
        return c, c.copy()
    rng = np.random.Generator(np.random.PCG64(wl.seed + 31337))
    vals = np.array(wl.clip_set, dtype=np.float64)
    ck, cv = np.empty(wl.Hkv), np.empty(wl.Hkv)
    for j in range(wl.Hkv):
        a, b = rng.choice(len(vals), size=2, replace=False)
        ck[j], cv[j] = vals[a], vals[b]
    return ck.astype(np.float32), cv.astype(np.float32)


def make_small(wl: Workload, distinct_rv: bool = False) -> SmallInputs:
    """All inputs of a small workload.  Token t of sequence b is K[b][t]; tokens
    L_b .. L_b+steps-1 are the new tokens appended by the decode steps."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    R_k = np.stack([make_rotation(rng, wl.D) for _ in range(wl.Hkv)])
    R_v = np.stack([make_rotation(rng, wl.D) for _ in range(wl.Hkv)]) if distinct_rv else R_k.copy()
    out_k = _outliers(rng, wl.Hkv, wl.D, wl.n_outliers)
    out_v = _outliers(rng, wl.Hkv, wl.D, wl.n_outliers)
    K, V = [], []
    for b in range(wl.B):
        n = wl.lengths[b] + wl.steps
        K.append(_gaussian_kv(rng, n, wl.Hkv, wl.D, out_k, wl.outlier_scale))
        if wl.v_range > 0:
            u = rng.uniform(-wl.v_range, wl.v_range, (n, wl.Hkv, wl.D)).astype(np.float32)
            V.append(_f32_to_bf16_bits(u))
        else:
            V.append(_gaussian_kv(rng, n, wl.Hkv, wl.D, out_v, wl.outlier_scale))
    q = _f32_to_bf16_bits(rng.standard_normal((wl.steps, wl.B, wl.Hq, wl.D), dtype=np.float32))
    clip_k, clip_v = clip_ratios(wl)
    return SmallInputs(wl, q, K, V, R_k, R_v, clip_k, clip_v, out_k, out_v)


def share_history(inp: SmallInputs, segments) -> SmallInputs:
    """Make sequences share history pages, as a prefix cache does for a
    common prompt prefix: for each (first_page, num_pages, seq_begin,
    num_seqs), the history tokens of pages first_page .. +num_pages-1 (token
    positions 64 + 16*page ..) of sequences seq_begin+1 .. are overwritten (in
    place) with those of sequence seq_begin."""
    for (first, num, s0, n) in segments:
        a, e = SINK + PAGE * first, SINK + PAGE * (first + num)
        for b in range(s0 + 1, s0 + n):
            assert e <= SINK + split_lengths(inp.wl.lengths[b])[1], "segment beyond the history"
            inp.K[b][a:e] = inp.K[s0][a:e]
            inp.V[b][a:e] = inp.V[s0][a:e]
    return inp


def plant_tokens(inp: SmallInputs, b: int, positions, kind: str, value: float = 0.0,
                 which: str = "kv") -> SmallInputs:
    """Overwrite tokens of sequence b (in place, token order positions) with
    degenerate content: kind "zero" (every channel +0) or "const" (every
    channel `value`, rounded to bf16); which = "k", "v" or "kv"."""
    bits = _f32_to_bf16_bits(np.array([0.0 if kind == "zero" else value], np.float32))[0]
    for t in positions:
        if "k" in which:
            inp.K[b][t] = bits
        if "v" in which:
            inp.V[b][t] = bits
    return inp


def page_permutation(seed: int, n_pages: int, extra: int = 0) -> np.ndarray:
    """Random physical page ids for n_pages logical pages out of a pool of
    n_pages + extra (page tables in random physical order)."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    return rng.permutation(n_pages + extra)[:n_pages].astype(np.int32)


# ----------------------------------------------------------------------------
# large workloads: device-side generation, block-seeded
# ----------------------------------------------------------------------------

def _seed64(*parts) -> int:
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def make_codebook(seed: int, Hkv: int, symmetric: bool = False) -> np.ndarray:
    """Lloyd-Max code levels float32 [Hkv][2][4] (K, V) for the codebook
    variant, standing in for offline calibration: levels pulled towards the
    middle of the group range, (0.35, 1.15, 1.85, 2.65) in units of the group
    scale, each moved by a seeded offset in [-0.05, 0.05] so that heads and
    K/V differ.  Ascending by construction.

    symmetric=True gives what a fit to a distribution symmetric about the
    middle of the range gives: levels 1.5 -+ a, 1.5 -+ b (a near 1.15, b near
    0.35, seeded offsets on a 1/1024 grid, so that every level and every
    difference of levels is exact in float32 and L3 - L2 = L1 - L0 holds
    exactly)."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    if symmetric:
        off = np.round(rng.uniform(-0.05, 0.05, (Hkv, 2, 2)) * 1024) / 1024
        a = np.round(1.15 * 1024) / 1024 + off[..., 0]
        b = np.round(0.35 * 1024) / 1024 + off[..., 1]
        return np.stack([1.5 - a, 1.5 - b, 1.5 + b, 1.5 + a], axis=-1).astype(np.float32)
    base = np.array([0.35, 1.15, 1.85, 2.65])
    return (base + rng.uniform(-0.05, 0.05, (Hkv, 2, 4))).astype(np.float32)


class LargeGen:
    """Device-side generator for 100K-class workloads.

    History content is addressed by *unique page* id u (0..n_unique-1): its
    16 tokens of K and V for all KV heads come from block u // PAGES_PER_BLOCK,
    so any page can be regenerated exactly on demand (for sampled oracle checks).
    Sequences that share a prefix (or a whole prompt) alias the same unique
    pages in their page tables.
    """

    PAGES_PER_BLOCK = 256

    def __init__(self, wl: Workload, device="cuda"):
        import torch
        self.torch = torch
        self.wl = wl
        self.device = device
        rng = np.random.Generator(np.random.PCG64(wl.seed))
        self.R_k = np.stack([make_rotation(rng, wl.D) for _ in range(wl.Hkv)])
        self.R_v = self.R_k.copy()
        self.out_k = _outliers(rng, wl.Hkv, wl.D, wl.n_outliers)
        self.out_v = _outliers(rng, wl.Hkv, wl.D, wl.n_outliers)
        self.clip_k, self.clip_v = clip_ratios(wl)
        self._build_page_map()
        self._scale_k = self._channel_scale(self.out_k)
        self._scale_v = self._channel_scale(self.out_v)

    def _channel_scale(self, out_idx):
        s = np.ones((self.wl.Hkv, self.wl.D), dtype=np.float32)
        for j in range(self.wl.Hkv):
            s[j, out_idx[j]] = self.wl.outlier_scale
        return self.torch.from_numpy(s).to(self.device)

    def _build_page_map(self):
        """unique-page ids per (sequence, logical history page), prefix/prompt aliasing."""
        wl = self.wl
        hist_pages = []
        n_hist = []
        for b in range(wl.B):
            _, h, _ = split_lengths(wl.lengths[b])
            h_final = h + wl.steps
            n_hist.append(h)
            hist_pages.append(-(-h_final // PAGE))
        self.hist_len0 = np.array(n_hist, dtype=np.int64)
        self.hist_pages_max = max(hist_pages) if hist_pages else 0
        # content source per sequence: prefix pages shared by all; suffix pages
        # shared by the non-distinct group, own pages for distinct sequences
        pre_pages = max(0, wl.shared_prefix - SINK) // PAGE if wl.shared_prefix else 0
        n_distinct = int(round(wl.distinct_frac * wl.B)) if wl.shared_prefix else wl.B
        key_to_u: Dict[tuple, int] = {}
        table = np.full((wl.B, self.hist_pages_max), -1, dtype=np.int64)
        for b in range(wl.B):
            # pages that later decode steps fill are always private to the sequence
            prompt_pages = self.hist_len0[b] // PAGE
            for p in range(hist_pages[b]):
                if p < pre_pages:
                    key = ("prefix", p)
                elif p < prompt_pages and wl.shared_prefix and b >= n_distinct:
                    key = ("shared", p)
                else:
                    key = ("own", b, p)
                if key not in key_to_u:
                    key_to_u[key] = len(key_to_u)
                table[b, p] = key_to_u[key]
        self.unique_of = table              # [B][pages] unique page id
        self.n_unique = len(key_to_u)
        perm = page_permutation(wl.seed, self.n_unique)
        self.phys_of_unique = perm          # unique id -> physical INT2 page
        self.hist_table = np.where(table >= 0, perm[np.maximum(table, 0)], 0).astype(np.int32)
        # a page's tokens that come from the shared prompt are identical across the
        # sequences aliasing it; partially-filled tail pages are private

    def shared_segments(self):
        """The aliasing of the page tables as shared-page segments
        (first_page, num_pages, seq_begin, num_seqs): the prefix pages shared
        by every sequence, then the rest of the prompt's full pages shared by
        the sequences without a distinct suffix (those come last)."""
        wl = self.wl
        if not wl.shared_prefix:
            return []
        pre = max(0, wl.shared_prefix - SINK) // PAGE
        n_distinct = int(round(wl.distinct_frac * wl.B))
        segs = [(0, pre, 0, wl.B)] if pre > 0 and wl.B >= 2 else []
        rest = int(min(self.hist_len0[n_distinct:] // PAGE)) - pre if n_distinct < wl.B else 0
        if rest > 0 and wl.B - n_distinct >= 2:
            segs.append((pre, rest, n_distinct, wl.B - n_distinct))
        return segs

    def history_block(self, blk: int):
        """K, V bf16 tensors [PAGES_PER_BLOCK*16][Hkv][D] for unique pages of block blk."""
        torch = self.torch
        wl = self.wl
        gen = torch.Generator(device=self.device)
        gen.manual_seed(_seed64(wl.seed, "hist", blk))
        n = self.PAGES_PER_BLOCK * PAGE
        k = torch.randn((n, wl.Hkv, wl.D), generator=gen, device=self.device, dtype=torch.float32)
        v = torch.randn((n, wl.Hkv, wl.D), generator=gen, device=self.device, dtype=torch.float32)
        k = (k * self._scale_k).to(torch.bfloat16)
        v = (v * self._scale_v).to(torch.bfloat16)
        return k, v

    def unique_page(self, u: int):
        k, v = self.history_block(u // self.PAGES_PER_BLOCK)
        o = (u % self.PAGES_PER_BLOCK) * PAGE
        return k[o:o + PAGE], v[o:o + PAGE]

    def bf16_tokens(self, b: int):
        """Sink + recent tokens of sequence b before the first step: [n][Hkv][D] bf16."""
        torch = self.torch
        wl = self.wl
        s, _, r = split_lengths(wl.lengths[b])
        gen = torch.Generator(device=self.device)
        # sequences sharing a prompt share its sink tokens
        src = 0 if (wl.shared_prefix and wl.shared_prefix >= SINK) else b
        gen.manual_seed(_seed64(wl.seed, "sink", src))
        ks = torch.randn((s, wl.Hkv, wl.D), generator=gen, device=self.device)
        vs = torch.randn((s, wl.Hkv, wl.D), generator=gen, device=self.device)
        gen.manual_seed(_seed64(wl.seed, "recent", b))
        kr = torch.randn((r, wl.Hkv, wl.D), generator=gen, device=self.device)
        vr = torch.randn((r, wl.Hkv, wl.D), generator=gen, device=self.device)
        k = (torch.cat([ks, kr]) * self._scale_k).to(torch.bfloat16)
        v = (torch.cat([vs, vr]) * self._scale_v).to(torch.bfloat16)
        return k, v

    def step_tokens(self, step: int):
        """New-token K, V [B][Hkv][D] and q [B][Hq][D] (bf16) for decode step `step`."""
        torch = self.torch
        wl = self.wl
        gen = torch.Generator(device=self.device)
        gen.manual_seed(_seed64(wl.seed, "step", step))
        k = torch.randn((wl.B, wl.Hkv, wl.D), generator=gen, device=self.device)
        v = torch.randn((wl.B, wl.Hkv, wl.D), generator=gen, device=self.device)
        q = torch.randn((wl.B, wl.Hq, wl.D), generator=gen, device=self.device)
        return ((k * self._scale_k).to(torch.bfloat16), (v * self._scale_v).to(torch.bfloat16),
                q.to(torch.bfloat16))
