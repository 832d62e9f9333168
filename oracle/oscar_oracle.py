"""CPU oracle for OSCAR's split-cache INT2 decode path (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never calls it, and this module imports nothing from the
product.

What it computes, and where the pages state it (page titles abbreviated:
  [snilld]  "OSCAR fra Together AI goer 2-bit KV-cache mere praktisk" (snilld.dk)
  [arddev]  "OSCAR 2bit KV cache" (arddev.tech)
  [thmotor] the Chinese repost of the authors' article (m.th-motor.com)):

* compose_rotation: R = U . Hadamard . bit-reversal permutation
  ([thmotor], the paragraph after Fig. 1 that writes the final rotation;
  [snilld] section "Hvad OSCAR gor anderledes", third paragraph; [arddev]
  section "Analytics", second paragraph).  Row-vector convention x = k . R.
* rotate / quantize_groups / pack_rows / pack_channel_major: the demotion step
  that rotates, clips, quantises and packs the oldest recent token, four 2-bit
  values per byte ([thmotor], the paragraph on the split cache that follows the
  rotation formula).  Quantisation is per group of G consecutive rotated
  channels with an asymmetric bf16 scale / zero point and a clipping ratio.
* dequant: the INT2 kernel's unpack and scale/zero-point restore ([thmotor],
  same paragraph, decode stage).
* lloyd_max_levels / quantize_groups_codebook / dequant_codebook: the Lloyd-Max
  codebook variant ([thmotor], closing paragraph; reading in the section
  comment above those functions).
* decode_attention: one softmax over the BF16 sink/recent tokens and the INT2
  history together; the history contribution is computed in the rotated basis
  and un-rotated by R_v^T.  decode_attention_split + lse_merge: the same result
  from per-chunk partials merged by online softmax ([thmotor], decode stage:
  the BF16 and INT2 segments are merged by an online-softmax merge).

Readings taken where the pages are silent:
  clip ratio c scales the group min and max: range [c*mn, c*mx]; scale =
  (c*mx - c*mn)/3, zero = c*mn, both rounded to bf16 directly from fp64 (round
  to nearest even); codes = clamp(rint((x - zero_b)/scale_b), 0, 3) with
  round-half-even and the *rounded* scale/zero; a group whose bf16 scale is 0
  gets all-zero codes; bit order inside a byte is LSB first; query rotation
  q . R_k for the history (keys matter only through QK^T); softmax scale
  1/sqrt(D); GQA map h -> h // (Hq/Hkv) unless a map is given.

Parity status of each function is given in its docstring.  Everything here is
pinned by tests under tests/ (hand-worked fixtures in tests/golden/, closed
forms, invariants, library routines and brute force) except the conventions
the pages leave open, which are pinned only by the written reading above.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# bf16 helpers
# ----------------------------------------------------------------------------

BF16_MIN_SUB_EXP = -133      # smallest bf16 subnormal is 2**-133
BF16_MAX = float.fromhex("0x1.fe00000000000p+127")


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round_scalar(x: float) -> float:
    """Round a float64 to the nearest bf16 value, ties to even, in one step.

    bf16 keeps 8 significant bits (7 stored) and fp32's exponent range.  The
    quantum at x is 2**(e-8) where x = m * 2**e, 0.5 <= |m| < 1, but never below
    the subnormal quantum 2**-133.  Dividing by a power of two is exact, so
    rint() performs the single rounding.  Overflow beyond the largest finite
    bf16 gives +-inf (never reached by the workloads).
    """
    if x == 0.0 or not math.isfinite(x):
        return x
    _, e = math.frexp(x)
    qexp = max(e - 8, BF16_MIN_SUB_EXP)
    r = math.ldexp(float(np.rint(math.ldexp(x, -qexp))), qexp)
    if abs(r) > BF16_MAX:
        return math.copysign(math.inf, x)
    return r


def bf16_round(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat = x.reshape(-1)
    o = out.reshape(-1)
    # vectorised form of bf16_round_scalar
    nz = (flat != 0) & np.isfinite(flat)
    o[~nz] = flat[~nz]
    if nz.any():
        v = flat[nz]
        _, e = np.frexp(v)
        qexp = np.maximum(e.astype(np.int64) - 8, BF16_MIN_SUB_EXP)
        r = np.ldexp(np.rint(np.ldexp(v, -qexp)), qexp)
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, v), r)
        o[nz] = r
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """Bit patterns of float64 values that are exactly bf16-representable."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), x, equal_nan=True), "not bf16-representable"
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "not bf16-representable"
    return (u >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# rotation R = U . H . P
# ----------------------------------------------------------------------------

def hadamard(D: int) -> np.ndarray:
    """Normalised Walsh-Hadamard matrix of order D (Sylvester's construction):
    H[i, j] = (-1)**popcount(i & j) / sqrt(D)."""
    assert D >= 1 and (D & (D - 1)) == 0
    i = np.arange(D)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0) / math.sqrt(D)


def bitrev_indices(nbits: int) -> np.ndarray:
    """bitrev[i] = i with its nbits binary digits reversed."""
    out = []
    for i in range(1 << nbits):
        s = format(i, f"0{nbits}b") if nbits else ""
        out.append(int(s[::-1], 2) if nbits else 0)
    return np.array(out, dtype=np.int64)


def bitrev_matrix(D: int) -> np.ndarray:
    """Permutation matrix P with P[i, bitrev(i)] = 1."""
    nb = int(round(math.log2(D)))
    P = np.zeros((D, D))
    P[np.arange(D), bitrev_indices(nb)] = 1.0
    return P


def compose_rotation(U: np.ndarray) -> np.ndarray:
    """R = U . H_D . P_bitrev in fp64.  Parity: pinned by a hand-worked D=4
    fixture and by orthogonality."""
    U = np.asarray(U, dtype=np.float64)
    D = U.shape[0]
    return U @ hadamard(D) @ bitrev_matrix(D)


# ----------------------------------------------------------------------------
# demotion: rotate, clip, quantise, pack
# ----------------------------------------------------------------------------

def rotate(x, R) -> np.ndarray:
    """x . R in fp64 for row vectors x [..., D] (bf16 or fp32 values) and R [D, D].
    Each product of a bf16 and an fp32 value is exact in fp64; the sum is fp64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(R, dtype=np.float64)


def quantize_groups(x, G: int, clip: float):
    """Group-wise asymmetric INT2 quantisation with clipping.

    x: float64 [n, D] rotated values; groups are G consecutive channels of a row.
    Returns codes uint8 [n, D] in {0,1,2,3}, scale and zero float64 [n, D/G]
    (bf16-representable).  Op sequence, each a single correctly-rounded fp64
    operation: mx, mn = max, min of the group; hi = c*mx; lo = c*mn;
    scale = (hi - lo)/3; zero = lo; s_b, z_b = bf16(scale), bf16(zero);
    code = clamp(rint((x - z_b)/s_b), 0, 3), or 0 when s_b == 0.
    """
    x = np.asarray(x, dtype=np.float64)
    n, D = x.shape
    assert D % G == 0
    xg = x.reshape(n, D // G, G)
    c = float(np.float32(clip))
    mx = xg.max(axis=2)
    mn = xg.min(axis=2)
    hi = c * mx
    lo = c * mn
    scale = (hi - lo) / 3.0
    zero = lo
    s_b = bf16_round(scale)
    z_b = bf16_round(zero)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xg - z_b[:, :, None]) / s_b[:, :, None]
        code = np.clip(np.rint(t), 0, 3)
    code = np.where(s_b[:, :, None] == 0, 0, code)
    return code.reshape(n, D).astype(np.uint8), s_b, z_b


def dequant(codes, s_b, z_b, G: int) -> np.ndarray:
    """x_hat = code * scale + zero (exact in fp64)."""
    codes = np.asarray(codes, dtype=np.float64)
    n, D = codes.shape
    cg = codes.reshape(n, D // G, G)
    return (cg * s_b[:, :, None] + z_b[:, :, None]).reshape(n, D)


# ----------------------------------------------------------------------------
# Lloyd-Max codebook variant
# ----------------------------------------------------------------------------
# [thmotor], closing paragraph: the authors' latest code adds a Lloyd-Max
# codebook to the attention-aware rotation.  The page says nothing more.
# Reading taken: the group scale/zero and clipping stay as above; the 4 levels
# of a code are not 0, 1, 2, 3 but a non-uniform codebook L (ascending, in
# units of the group scale above the zero point) per (KV head, K|V), fixed by
# offline calibration like R and the clip ratio:
#     x_hat = zero_b + scale_b * L[code]
# and a code is the nearest level, with the decision thresholds at the level
# midpoints.  L = (0, 1, 2, 3) is the uniform quantiser.  Parity unpinned
# against the pages (they give no level values); pinned by the uniform special
# case, brute force, and Lloyd-Max's textbook solution for a Gaussian.

def lloyd_max_levels(samples, n_levels: int = 4, init=None, iters: int = 200) -> np.ndarray:
    """Lloyd's algorithm on 1-D samples (Lloyd 1957 / Max 1960): alternate
    decision thresholds at the midpoints of adjacent levels and levels at the
    mean of the samples between their thresholds, until the levels stop
    moving.  Returns the ascending levels (float64).  A level whose cell is
    empty keeps its value."""
    x = np.sort(np.asarray(samples, dtype=np.float64).ravel())
    if init is None:
        lv = np.quantile(x, (np.arange(n_levels) + 0.5) / n_levels)
    else:
        lv = np.array(init, dtype=np.float64)
    for _ in range(iters):
        th = 0.5 * (lv[:-1] + lv[1:])
        cell = np.searchsorted(th, x, side="left")      # x <= th[0] -> cell 0
        new = lv.copy()
        for k in range(n_levels):
            sel = x[cell == k]
            if sel.size:
                new[k] = sel.mean()
        if np.array_equal(new, lv):
            break
        lv = new
    return lv


def codebook_thresholds(levels) -> np.ndarray:
    """Decision thresholds of a 4-level codebook given as float32 values:
    (L_k + L_{k+1}) / 2 in fp64 (both exact, the sum and the halving exact
    too for float32 inputs)."""
    L = np.asarray(levels, dtype=np.float32).astype(np.float64)
    return 0.5 * (L[:-1] + L[1:])


def quantize_groups_codebook(x, G: int, clip: float, levels):
    """The group quantiser with a codebook: scale, zero and their bf16 rounding
    exactly as quantize_groups; then u = (x - zero_b) / scale_b (one fp64
    division) and code = the number of thresholds strictly below u, i.e. the
    nearest level, a tie going to the lower one; 0 when scale_b == 0.
    Returns codes uint8 [n, D], scale and zero float64 [n, D/G]."""
    x = np.asarray(x, dtype=np.float64)
    n, D = x.shape
    xg = x.reshape(n, D // G, G)
    c = float(np.float32(clip))
    mx = xg.max(axis=2)
    mn = xg.min(axis=2)
    scale = (c * mx - c * mn) / 3.0
    zero = c * mn
    s_b = bf16_round(scale)
    z_b = bf16_round(zero)
    th = codebook_thresholds(levels)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (xg - z_b[:, :, None]) / s_b[:, :, None]
    code = (u[..., None] > th).sum(axis=-1)
    code = np.where(s_b[:, :, None] == 0, 0, code)
    return code.reshape(n, D).astype(np.uint8), s_b, z_b


def dequant_codebook(codes, s_b, z_b, G: int, levels) -> np.ndarray:
    """x_hat = zero_b + scale_b * L[code], L the float32 levels (fp64 arithmetic)."""
    L = np.asarray(levels, dtype=np.float32).astype(np.float64)
    codes = np.asarray(codes)
    n, D = codes.shape
    lv = L[codes].reshape(n, D // G, G)
    return (z_b[:, :, None] + s_b[:, :, None] * lv).reshape(n, D)


def quantize_tokens_codebook(kv_bf16_vals, R, G: int, clip: float, levels):
    """Rotate, then quantise with a codebook (see quantize_groups_codebook)."""
    return quantize_groups_codebook(rotate(kv_bf16_vals, R), G, clip, levels)


def pack_rows(codes) -> np.ndarray:
    """Four codes per byte along the channel axis, LSB first:
    byte[i] = c[4i] | c[4i+1] << 2 | c[4i+2] << 4 | c[4i+3] << 6."""
    c = np.asarray(codes, dtype=np.uint8)
    n, D = c.shape
    c4 = c.reshape(n, D // 4, 4)
    return (c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)).astype(np.uint8)


def unpack_rows(packed, D: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    n = p.shape[0]
    out = np.empty((n, D), dtype=np.uint8)
    for k in range(4):
        out[:, k::4] = (p >> (2 * k)) & 3
    return out


def pack_channel_major(codes16) -> np.ndarray:
    """V codes of one 16-token page, one 32-bit word per channel: token t's code
    in bits 2t..2t+1 (LSB first, i.e. 4 codes per byte).  Input codes [16, D];
    output uint32 [D] indexed by channel."""
    c = np.asarray(codes16, dtype=np.uint32)
    assert c.shape[0] == 16
    w = np.zeros(c.shape[1], dtype=np.uint32)
    for t in range(16):
        w |= c[t] << np.uint32(2 * t)
    return w


def k_row_words(codes_row) -> np.ndarray:
    """K codes of one token as D/16 32-bit words.  Word q = kb*(D/64) + blk holds
    channels 64*blk + 16*kb + i in bits 2i (i = 0..15): the row's 16-channel
    slices taken slice-of-block-major, so that the slices a reader needs for
    every 64-channel block are adjacent.  For D = 64 this is channel order."""
    c = np.asarray(codes_row, dtype=np.uint32)
    D = c.shape[0]
    nblk = max(1, D // 64)
    out = np.zeros(D // 16, dtype=np.uint32)
    for blk in range(nblk):
        for kb in range(min(4, D // 16)):
            w = 0
            for i in range(16):
                w |= int(c[64 * blk + 16 * kb + i]) << (2 * i)
            out[kb * nblk + blk] = w
    return out


# ----------------------------------------------------------------------------
# INT2 page record (layout of one (physical page, KV head) record in HBM)
# ----------------------------------------------------------------------------

def record_bytes(D: int, G: int) -> int:
    """Code region of 64 lane slots x D/32 words (2*16*D/4 bytes) | scale/zero
    region of 16 token slots x 2*D/G words (2*16*(D/G)*4 bytes)."""
    return 2 * 16 * (D // 4) + 2 * 16 * (D // G) * 4


def encode_record(kc, ks, kz, vc, vs, vz, D: int, G: int) -> np.ndarray:
    """Bytes of one page record (16 tokens of one KV head) from codes [16, D]
    and bf16 scale/zero [16, D/G] for K and V.  Words are little-endian; D is a
    multiple of 64.  Token rows not yet written are all-zero (pass zeros).

    Code region: lane slot l = 16*kb + t (kb = 0..3, t = 0..15) holds, in this
    order, the D/64 K words of token t for part kb (word blk = k_row_words word
    kb*(D/64) + blk: channels 64*blk + 16*kb + i in bits 2i), then the D/64 V
    words of channels l, l + 64, ... (pack_channel_major: token t in bits 2t).
    Scale/zero region: token slot t holds the K words of groups 0..D/G-1, then
    the V words; each word is scale (bf16) | zero (bf16) << 16."""
    nblk, ng = D // 64, D // G
    sw = D // 32
    vw = pack_channel_major(vc)
    codes = np.zeros(64 * sw, dtype=np.uint32)
    for t in range(16):
        krow = k_row_words(kc[t])
        for kb in range(4):
            l = 16 * kb + t
            for blk in range(nblk):
                codes[l * sw + blk] = krow[kb * nblk + blk]
    for l in range(64):
        for h2 in range(nblk):
            codes[l * sw + nblk + h2] = vw[l + 64 * h2]

    def szw(s, z):
        sb = f64_to_bf16_bits(s).astype(np.uint32)
        zb = f64_to_bf16_bits(z).astype(np.uint32)
        return sb | (zb << np.uint32(16))            # [16][D/G]
    sz = np.concatenate([szw(ks, kz), szw(vs, vz)], axis=1).reshape(-1)   # [16][2*D/G]
    out = np.concatenate([codes.astype("<u4").view(np.uint8), sz.astype("<u4").view(np.uint8)])
    assert out.size == record_bytes(D, G)
    return out


def decode_record(rec, D: int, G: int):
    """Inverse of encode_record: (kc, ks, kz, vc, vs, vz)."""
    rec = np.asarray(rec, dtype=np.uint8)
    nblk, ng = D // 64, D // G
    sw = D // 32
    codes = rec[:64 * sw * 4].view("<u4").reshape(64, sw)
    kc = np.zeros((16, D), np.uint8)
    vc = np.zeros((16, D), np.uint8)
    for l in range(64):
        kb, t = l >> 4, l & 15
        for blk in range(nblk):
            w = int(codes[l, blk])
            for i in range(16):
                kc[t, 64 * blk + 16 * kb + i] = (w >> (2 * i)) & 3
        for h2 in range(nblk):
            w = int(codes[l, nblk + h2])
            for tt in range(16):
                vc[tt, l + 64 * h2] = (w >> (2 * tt)) & 3
    sz = rec[64 * sw * 4:].view("<u4").reshape(16, 2 * ng)
    lo = (sz & np.uint32(0xFFFF)).astype(np.uint16)
    hi = (sz >> np.uint32(16)).astype(np.uint16)
    return (kc, bf16_bits_to_f64(lo[:, :ng]), bf16_bits_to_f64(hi[:, :ng]),
            vc, bf16_bits_to_f64(lo[:, ng:]), bf16_bits_to_f64(hi[:, ng:]))


def quantize_tokens(kv_bf16_vals, R, G: int, clip: float):
    """Rotate then quantise token vectors [n, D] (float64 values of bf16).
    Returns codes [n, D], scale [n, D/G], zero [n, D/G]."""
    x = rotate(kv_bf16_vals, R)
    return quantize_groups(x, G, clip)


# ----------------------------------------------------------------------------
# attention over the split cache
# ----------------------------------------------------------------------------

def default_head_map(Hq: int, Hkv: int) -> np.ndarray:
    g = Hq // Hkv
    return np.arange(Hq) // g


def _segment_logits(qv, keys, sm_scale):
    return sm_scale * (keys @ qv)


def decode_attention(q, kv_head_of_q, bf16_k, bf16_v, hist_khat, hist_vhat,
                     R_k, R_v, sm_scale: Optional[float] = None):
    """Decode attention of one sequence over its split cache, one fp64 softmax.

    q           [Hq, D]       query values (bf16 values as float64)
    bf16_k/v    [Tb, Hkv, D]  sink + recent tokens (unrotated)
    hist_khat/v [Th, Hkv, D]  dequantised history, in the rotated basis
    R_k, R_v    [Hkv, D, D]   rotations (R_v None: identity)
    Returns out [Hq, D] float64 and lse [Hq] (natural log of the softmax
    denominator, logits in natural units); a head with no tokens gets out = 0,
    lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.zeros((Hq, D))
    lse = np.full(Hq, -np.inf)
    for h in range(Hq):
        j = int(kv_head_of_q[h])
        sb = _segment_logits(q[h], np.asarray(bf16_k, dtype=np.float64)[:, j, :], sm_scale) \
            if len(bf16_k) else np.zeros(0)
        qr = q[h] @ np.asarray(R_k[j], dtype=np.float64)
        sh = _segment_logits(qr, np.asarray(hist_khat, dtype=np.float64)[:, j, :], sm_scale) \
            if len(hist_khat) else np.zeros(0)
        s = np.concatenate([sb, sh])
        if s.size == 0:
            continue
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        pb, ph = e[:sb.size] / l, e[sb.size:] / l
        o = pb @ np.asarray(bf16_v, dtype=np.float64)[:, j, :] if sb.size else np.zeros(D)
        if sh.size:
            orot = ph @ np.asarray(hist_vhat, dtype=np.float64)[:, j, :]
            Rv = np.eye(D) if R_v is None else np.asarray(R_v[j], dtype=np.float64)
            o = o + orot @ Rv.T
        out[h] = o
        lse[h] = m + math.log(l)
    return out, lse


def partial_softmax(s, vals):
    """(m, l, o) of one chunk: m = max s, l = sum exp(s-m), o = sum exp(s-m) v
    (unnormalised).  Empty chunk: (-inf, 0, 0)."""
    s = np.asarray(s, dtype=np.float64)
    if s.size == 0:
        return -np.inf, 0.0, np.zeros(vals.shape[-1])
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ vals


def lse_merge(parts):
    """Online-softmax merge of partials (m_i, l_i, o_i): M = max m_i,
    L = sum l_i e^{m_i-M}, O = sum o_i e^{m_i-M}.  Returns (M, L, O)."""
    ms = [p[0] for p in parts]
    M = max(ms) if ms else -np.inf
    if M == -np.inf:
        D = parts[0][2].shape[-1] if parts else 0
        return -np.inf, 0.0, np.zeros(D)
    L = 0.0
    O = np.zeros_like(parts[0][2], dtype=np.float64)
    for m, l, o in parts:
        if m == -np.inf:
            continue
        w = math.exp(m - M)
        L += l * w
        O = O + o * w
    return M, L, O


def decode_attention_split(q, kv_head_of_q, bf16_k, bf16_v, hist_khat, hist_vhat,
                           R_k, R_v, chunks: Sequence[Tuple[int, int]],
                           sm_scale: Optional[float] = None):
    """Same result as decode_attention, computed the way the split path does:
    one partial for the BF16 segment, one per history chunk [a, b) in the
    rotated basis, the history partials merged, un-rotated by R_v^T, then merged
    with the BF16 partial."""
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.zeros((Hq, D))
    lse = np.full(Hq, -np.inf)
    bk = np.asarray(bf16_k, dtype=np.float64)
    bv = np.asarray(bf16_v, dtype=np.float64)
    hk = np.asarray(hist_khat, dtype=np.float64)
    hv = np.asarray(hist_vhat, dtype=np.float64)
    for h in range(Hq):
        j = int(kv_head_of_q[h])
        if len(bk):
            pb = partial_softmax(sm_scale * (bk[:, j, :] @ q[h]), bv[:, j, :])
        else:
            pb = (-np.inf, 0.0, np.zeros(D))
        qr = q[h] @ np.asarray(R_k[j], dtype=np.float64)
        hparts = []
        for a, b in chunks:
            if b > a:
                hparts.append(partial_softmax(sm_scale * (hk[a:b, j, :] @ qr), hv[a:b, j, :]))
            else:
                hparts.append((-np.inf, 0.0, np.zeros(D)))
        Mh, Lh, Oh = lse_merge(hparts) if hparts else (-np.inf, 0.0, np.zeros(D))
        Rv = np.eye(D) if R_v is None else np.asarray(R_v[j], dtype=np.float64)
        Oh = Oh @ Rv.T
        M, L, O = lse_merge([pb, (Mh, Lh, Oh)])
        if M == -np.inf:
            continue
        out[h] = O / L
        lse[h] = M + math.log(L)
    return out, lse


# ----------------------------------------------------------------------------
# layout arithmetic
# ----------------------------------------------------------------------------

def history_bits_per_element(G: int, meta_bits: int = 32) -> float:
    """Bits per history element: 2-bit code + (bf16 scale + bf16 zero)/G."""
    return 2.0 + meta_bits / G


def bits_per_element(L: int, G: int, sink: int = 64, recent: int = 256) -> float:
    """Average bits per KV element over a context of L tokens: the BF16 sink and
    recent windows at 16 bits, the rest of the history at history_bits_per_element."""
    nb = min(L, sink + recent)
    nh = L - nb
    return (nh * history_bits_per_element(G) + nb * 16.0) / L
