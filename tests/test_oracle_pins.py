"""Pins of the CPU oracle against facts fixed outside the oracle itself:
hand-worked fixtures (tests/golden), closed forms, invariants, a library routine
and brute force on tiny inputs.  CPU only."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oscar_oracle as orc
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def test_bf16_rounding_golden():
    for c in _load("bf16_rounding_cases.json")["cases"]:
        x = float.fromhex(c["x"])
        want = float.fromhex(c["bf16"])
        assert orc.bf16_round_scalar(x) == want, c["why"]
        assert orc.bf16_round(np.array([x]))[0] == want, c["why"]


def test_bf16_rounding_matches_exact_nearest_even():
    """Brute force: for random fp64 values, the result is the nearest of the two
    neighbouring bf16 values (found with exact rational arithmetic), ties even."""
    rng = np.random.default_rng(5)
    xs = rng.standard_normal(3000) * np.exp2(rng.integers(-40, 40, 3000))
    xs = np.concatenate([xs, rng.standard_normal(200) * 2.0 ** -128])
    got = orc.bf16_round(xs)
    for x, r in zip(xs, got):
        # enumerate bf16 candidates by truncation of the fp32 bit pattern around x
        f = np.float32(x)
        u = int(np.array([f]).view(np.uint32)[0]) & 0xFFFF0000
        cands = set()
        for du in (-0x10000, 0, 0x10000, 0x20000):
            v = (u + du) & 0xFFFFFFFF
            cv = float(np.array([v], dtype=np.uint32).view(np.float32)[0])
            if math.isfinite(cv):
                cands.add(cv)
        cands.add(0.0)
        X = Fraction(float(x))
        best = min(cands, key=lambda c: (abs(Fraction(c) - X),
                                         (np.array([np.float32(c)]).view(np.uint32)[0] >> 16) & 1))
        assert r == best, (x, r, best)


# --------------------------------------------------------------------------
# rotation
# --------------------------------------------------------------------------

def test_rotation_d4_hand_worked():
    g = _load("rotation_d4.json")
    U = np.array(g["U"], dtype=np.float64)
    R = orc.compose_rotation(U)
    assert np.array_equal(R * 2, np.array(g["R_times_2"], dtype=np.float64))
    H = orc.hadamard(4)
    P = orc.bitrev_matrix(4)
    assert np.array_equal(H @ P * 2, np.array(g["HP_times_2"], dtype=np.float64))
    x = orc.rotate(np.array(g["k"], dtype=np.float64), R)
    assert np.array_equal(x, np.array(g["x"], dtype=np.float64))
    assert list(orc.bitrev_indices(3)) == g["bitrev3"]


def test_hadamard_closed_form():
    h2 = np.array([[1, 1], [1, -1]]) / math.sqrt(2)
    assert np.allclose(orc.hadamard(2), h2, atol=0, rtol=0)
    for D in (8, 64, 128):
        H = orc.hadamard(D)
        assert np.allclose(H @ H.T, np.eye(D), atol=1e-13)
        assert np.all(np.abs(np.abs(H) - 1 / math.sqrt(D)) < 1e-15)
        # Sylvester recursion H_2D = [[H, H], [H, -H]] / sqrt(2)
        Hh = orc.hadamard(D // 2)
        assert np.allclose(H, np.block([[Hh, Hh], [Hh, -Hh]]) / math.sqrt(2), atol=1e-15)


def test_bitrev_permutation_properties():
    for nb in range(1, 8):
        r = orc.bitrev_indices(nb)
        assert sorted(r) == list(range(1 << nb))
        assert np.array_equal(r[r], np.arange(1 << nb))     # involution
        P = orc.bitrev_matrix(1 << nb)
        assert np.array_equal(P, P.T) and np.array_equal(P @ P, np.eye(1 << nb))


@pytest.mark.parametrize("D", [64, 128])
def test_generated_rotation_orthogonal_and_composed(D):
    """The generator's R is U.H.P for its U: the oracle's independent
    composition of the same U reproduces it (to fp32 storage), and R R^T = I."""
    rng = np.random.Generator(np.random.PCG64(11))
    Rf = synth.make_rotation(rng, D)
    rng = np.random.Generator(np.random.PCG64(11))
    A = rng.standard_normal((2 * D, D))
    w, V = np.linalg.eigh(A.T @ A / (2 * D))
    V = V[:, np.argsort(-w, kind="stable")]
    V = V * np.sign(V[np.argmax(np.abs(V), axis=0), np.arange(D)])
    R64 = orc.compose_rotation(V)
    assert np.abs(R64 @ R64.T - np.eye(D)).max() < 1e-12
    assert np.abs(R64.astype(np.float32) - Rf).max() == 0.0
    Rs = Rf.astype(np.float64)
    assert np.abs(Rs @ Rs.T - np.eye(D)).max() < 1e-6


# --------------------------------------------------------------------------
# quantiser
# --------------------------------------------------------------------------

def test_quantizer_golden():
    for c in _load("quantizer_cases.json")["cases"]:
        x = np.array([c["x"]], dtype=np.float64)
        codes, s, z = orc.quantize_groups(x, 4, c["clip"])
        assert list(codes[0]) == c["codes"], c["name"]
        assert s[0, 0] == c["scale"] and z[0, 0] == c["zero"], c["name"]
        xh = orc.dequant(codes, s, z, 4)
        assert list(xh[0]) == c["x_hat"], c["name"]


def _brute_group(xg, clip):
    """Scalar brute force of one group with exact rationals for the
    half-integer comparison: the nearest of the 4 levels (ties: even code),
    restricted to the clamp range."""
    c = float(np.float32(clip))
    mx, mn = max(xg), min(xg)
    hi, lo = c * mx, c * mn
    s = orc.bf16_round_scalar((hi - lo) / 3.0)
    z = orc.bf16_round_scalar(lo)
    if s == 0.0:
        return [0] * len(xg), s, z
    out = []
    for x in xg:
        t = (x - z) / s            # the one rounded fp64 quotient of the reading
        T = Fraction(t)
        best = min(range(4), key=lambda k: (abs(T - k), k % 2))
        out.append(best)
    return out, s, z


def test_quantizer_brute_force_random():
    rng = np.random.default_rng(7)
    for trial in range(300):
        G = int(rng.choice([4, 8, 32]))
        clip = float(rng.choice([1.0, 0.95, 0.8]))
        x = rng.standard_normal(G) * float(rng.choice([1e-3, 1.0, 30.0]))
        if trial % 17 == 0:
            x[:] = x[0]
        codes, s, z = orc.quantize_groups(x[None, :], G, clip)
        bc, bs, bz = _brute_group(list(x), clip)
        assert list(codes[0]) == bc and s[0, 0] == bs and z[0, 0] == bz


def test_quantizer_bounds_and_extremes():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((500, 64)) * 5
    codes, s, z = orc.quantize_groups(x, 32, 1.0)
    assert codes.max() <= 3 and codes.min() >= 0
    xg = x.reshape(500, 2, 32)
    cg = codes.reshape(500, 2, 32)
    # with c = 1 the group min maps to code 0 and the group max to code 3
    assert np.all(np.take_along_axis(cg, xg.argmin(2)[..., None], 2) == 0)
    assert np.all(np.take_along_axis(cg, xg.argmax(2)[..., None], 2) == 3)
    # inside the representable range the error is at most half a step
    xh = orc.dequant(codes, s, z, 32).reshape(500, 2, 32)
    inside = (xg >= z[..., None]) & (xg <= z[..., None] + 3 * s[..., None])
    err = np.abs(xg - xh)
    half = np.broadcast_to(s[..., None] / 2 * (1 + 1e-12), err.shape)
    assert np.all(err[inside] <= half[inside])


def test_quantizer_dropped_zero_or_unrounded_scale_fails():
    """Planted mistakes in a copy of the quantiser are caught by the fixtures."""
    cases = _load("quantizer_cases.json")["cases"]

    def bad_unrounded(x, G, clip):
        c = float(np.float32(clip))
        mx, mn = x.max(), x.min()
        s = (c * mx - c * mn) / 3.0
        z = c * mn
        return np.clip(np.rint((x - z) / s), 0, 3) if s else np.zeros_like(x)

    caught = 0
    for c in cases:
        x = np.array(c["x"], dtype=np.float64)
        try:
            got = list(bad_unrounded(x, 4, c["clip"]).astype(int))
        except ZeroDivisionError:
            got = None
        if got != c["codes"]:
            caught += 1
    assert caught >= 1


# --------------------------------------------------------------------------
# packing and page records
# --------------------------------------------------------------------------

def test_pack_golden():
    for r in _load("pack_cases.json")["rows"]:
        c = np.array([r["codes"]], dtype=np.uint8)
        assert list(orc.pack_rows(c)[0]) == r["bytes"]
        assert list(orc.unpack_rows(orc.pack_rows(c), c.shape[1])[0]) == r["codes"]


def test_pack_exhaustive_roundtrip():
    tuples = np.array(list(itertools.product(range(4), repeat=4)), dtype=np.uint8)
    packed = orc.pack_rows(tuples)
    assert sorted(packed[:, 0].tolist()) == list(range(256))
    assert np.array_equal(orc.unpack_rows(packed, 4), tuples)
    allb = np.arange(256, dtype=np.uint8)[:, None]
    assert np.array_equal(orc.pack_rows(orc.unpack_rows(allb, 4)), allb)


def test_channel_major_layout():
    c = np.zeros((16, 8), dtype=np.uint8)
    c[5, 2] = 3          # token 5, channel 2 -> channel 2's word, bits 10..11
    w = orc.pack_channel_major(c)
    assert w.shape == (8,) and w[2] == 3 << 10 and w.sum() == 3 << 10


def test_k_row_word_order():
    """D = 128: word q = kb*2 + blk holds channels 64*blk + 16*kb .. +15."""
    row = np.zeros(128, np.uint8)
    row[70] = 1          # blk 1, kb 0, i 6 -> word 1, bits 12..13
    row[16] = 3          # blk 0, kb 1, i 0 -> word 2, bits 0..1
    w = orc.k_row_words(row)
    assert w[1] == 1 << 12 and w[2] == 3 and w.sum() == (1 << 12) + 3


@pytest.mark.parametrize("D,G", [(64, 32), (128, 64), (128, 128)])
def test_record_roundtrip(D, G):
    rng = np.random.default_rng(D + G)
    x = rng.standard_normal((16, D)) * 3
    y = rng.standard_normal((16, D)) * 3
    kc, ks, kz = orc.quantize_groups(x, G, 0.95)
    vc, vs, vz = orc.quantize_groups(y, G, 0.95)
    rec = orc.encode_record(kc, ks, kz, vc, vs, vz, D, G)
    assert rec.size == orc.record_bytes(D, G)
    back = orc.decode_record(rec, D, G)
    for a, b in zip(back, (kc, ks, kz, vc, vs, vz)):
        assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _rand_orth(rng, D):
    q, r = np.linalg.qr(rng.standard_normal((D, D)))
    return q * np.sign(np.diag(r))


def test_rotation_invariance_unquantised():
    """softmax((qR_k)(KR_k)^T)(VR_v)R_v^T = softmax(qK^T)V when the history is not
    quantised (exactly orthogonal fp64 rotations, R_k != R_v, non-symmetric)."""
    rng = np.random.default_rng(1)
    D, Hkv, Hq = 16, 2, 4
    q = rng.standard_normal((Hq, D))
    K = rng.standard_normal((40, Hkv, D)) * 2
    V = rng.standard_normal((40, Hkv, D))
    Rk = np.stack([_rand_orth(rng, D) for _ in range(Hkv)])
    Rv = np.stack([_rand_orth(rng, D) for _ in range(Hkv)])
    hm = orc.default_head_map(Hq, Hkv)
    ref, lref = orc.decode_attention(q, hm, K, V, np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D)), Rk, Rv)
    Kr = np.einsum("thd,hde->the", K[10:], Rk)
    Vr = np.einsum("thd,hde->the", V[10:], Rv)
    got, lgot = orc.decode_attention(q, hm, K[:10], V[:10], Kr, Vr, Rk, Rv)
    assert np.abs(got - ref).max() < 1e-12 and np.abs(lgot - lref).max() < 1e-12
    # a transposed un-rotation breaks it
    bad, _ = orc.decode_attention(q, hm, K[:10], V[:10], Kr, Vr, Rk,
                                  np.transpose(Rv, (0, 2, 1)))
    assert np.abs(bad - ref).max() > 1e-3


def test_split_merge_equals_single_softmax():
    rng = np.random.default_rng(2)
    D, Hkv, Hq, Tb, Th = 8, 2, 4, 12, 37
    q = rng.standard_normal((Hq, D)) * 2
    bk = rng.standard_normal((Tb, Hkv, D))
    bv = rng.standard_normal((Tb, Hkv, D))
    hk = rng.standard_normal((Th, Hkv, D)) * 3
    hv = rng.standard_normal((Th, Hkv, D))
    Rk = np.stack([_rand_orth(rng, D) for _ in range(Hkv)])
    Rv = np.stack([_rand_orth(rng, D) for _ in range(Hkv)])
    hm = orc.default_head_map(Hq, Hkv)
    ref, lref = orc.decode_attention(q, hm, bk, bv, hk, hv, Rk, Rv)
    chunkings = [[(0, Th)], [(t, t + 1) for t in range(Th)], [(0, 5), (5, 5), (5, 30), (30, Th)]]
    cuts = sorted(rng.choice(np.arange(1, Th), 6, replace=False))
    chunkings.append(list(zip([0] + cuts, cuts + [Th])))
    for ch in chunkings:
        got, lgot = orc.decode_attention_split(q, hm, bk, bv, hk, hv, Rk, Rv, ch)
        assert np.abs(got - ref).max() < 1e-13 and np.abs(lgot - lref).max() < 1e-13


def test_empty_history_matches_torch_sdpa():
    import torch
    rng = np.random.default_rng(4)
    D, Hkv, Hq, T = 32, 2, 8, 50
    q = rng.standard_normal((Hq, D))
    K = rng.standard_normal((T, Hkv, D))
    V = rng.standard_normal((T, Hkv, D))
    hm = orc.default_head_map(Hq, Hkv)
    got, _ = orc.decode_attention(q, hm, K, V, np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D)),
                                  np.zeros((Hkv, D, D)), None)
    tq = torch.tensor(q)[:, None, :]                       # [Hq, 1, D]
    tk = torch.tensor(K).permute(1, 0, 2)[torch.tensor(hm)]  # [Hq, T, D]
    tv = torch.tensor(V).permute(1, 0, 2)[torch.tensor(hm)]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0, :].numpy()
    assert np.abs(got - ref).max() < 1e-13


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    D, Hkv = 8, 1
    v = rng.standard_normal((1, Hkv, D))
    k = rng.standard_normal((1, Hkv, D))
    R = np.stack([_rand_orth(rng, D)])
    hm = np.zeros(2, dtype=int)
    q = rng.standard_normal((2, D))
    # one BF16 token: output is that token's value
    o, lse = orc.decode_attention(q, hm, k, v, np.zeros((0, 1, D)), np.zeros((0, 1, D)), R, R)
    assert np.abs(o - v[0, 0]).max() < 1e-15
    assert np.abs(lse - (k[0, 0] @ q.T) / math.sqrt(D)).max() < 1e-14
    # one history token: output is its value un-rotated
    o, _ = orc.decode_attention(q, hm, np.zeros((0, 1, D)), np.zeros((0, 1, D)), k, v, R, R)
    assert np.abs(o - v[0, 0] @ R[0].T).max() < 1e-14
    # zero query: equal logits -> mean of all values
    V = rng.standard_normal((9, 1, D))
    K = rng.standard_normal((9, 1, D))
    o, lse = orc.decode_attention(np.zeros((2, D)), hm, K[:4], V[:4], K[4:], V[4:], R, None)
    assert np.abs(o - V[:, 0].mean(0)).max() < 1e-14
    assert np.abs(lse - math.log(9)).max() < 1e-14
    # empty sequence
    o, lse = orc.decode_attention(q, hm, np.zeros((0, 1, D)), np.zeros((0, 1, D)),
                                  np.zeros((0, 1, D)), np.zeros((0, 1, D)), R, R)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def _brute_decode(qv, bk, bv, hk_hat, hv_hat, Rk, Rv, sm):
    """Scalar loops + math.fsum: one softmax over every token, no vectorisation."""
    D = len(qv)
    qr = [math.fsum(qv[i] * Rk[i][c] for i in range(D)) for c in range(D)]
    logits = [sm * math.fsum(qv[c] * k[c] for c in range(D)) for k in bk]
    logits += [sm * math.fsum(qr[c] * k[c] for c in range(D)) for k in hk_hat]
    m = max(logits)
    e = [math.exp(s - m) for s in logits]
    L = math.fsum(e)
    nb = len(bk)
    o_b = [math.fsum(e[t] * bv[t][c] for t in range(nb)) for c in range(D)]
    o_r = [math.fsum(e[nb + t] * hv_hat[t][c] for t in range(len(hk_hat))) for c in range(D)]
    o_h = [math.fsum(o_r[i] * Rv[c][i] for i in range(D)) for c in range(D)]
    return [(o_b[c] + o_h[c]) / L for c in range(D)]


def test_brute_force_tiny_pipeline():
    """D=8, G=4, 40 tokens, Hkv=1, g=2: quantise the history and attend, then
    compare with scalar brute force (quantiser by nearest level, attention by
    explicit loops)."""
    rng = np.random.Generator(np.random.PCG64(9))
    D, G, n = 8, 4, 40
    R = synth.make_rotation(rng, D).astype(np.float64)
    K = synth.bf16_bits_to_f64(synth.inputs._f32_to_bf16_bits(rng.standard_normal((n, D)).astype(np.float32) * 3))
    V = synth.bf16_bits_to_f64(synth.inputs._f32_to_bf16_bits(rng.standard_normal((n, D)).astype(np.float32)))
    q = synth.bf16_bits_to_f64(synth.inputs._f32_to_bf16_bits(rng.standard_normal((2, D)).astype(np.float32)))
    hist = slice(6, 34)
    xk = np.array([[math.fsum(K[t, i] * R[i, c] for i in range(D)) for c in range(D)] for t in range(n)])
    xv = np.array([[math.fsum(V[t, i] * R[i, c] for i in range(D)) for c in range(D)] for t in range(n)])
    assert np.abs(xk - orc.rotate(K, R)).max() < 1e-13
    kc, ks, kz = orc.quantize_groups(orc.rotate(K[hist], R), G, 0.95)
    vc, vs, vz = orc.quantize_groups(orc.rotate(V[hist], R), G, 0.95)
    # brute-force quantiser on the exactly rounded rotation
    for t in range(kc.shape[0]):
        for gi in range(D // G):
            bc, bs, bz = _brute_group(list(xk[hist][t, gi * G:(gi + 1) * G]), 0.95)
            assert list(kc[t, gi * G:(gi + 1) * G]) == bc and ks[t, gi] == bs and kz[t, gi] == bz
    khat = orc.dequant(kc, ks, kz, G)
    vhat = orc.dequant(vc, vs, vz, G)
    bidx = list(range(0, 6)) + list(range(34, n))
    o, _ = orc.decode_attention(q, np.array([0, 0]), K[bidx][:, None, :], V[bidx][:, None, :],
                                khat[:, None, :], vhat[:, None, :], R[None], R[None])
    for h in range(2):
        ref = _brute_decode(list(q[h]), [list(r) for r in K[bidx]], [list(r) for r in V[bidx]],
                            [list(r) for r in khat], [list(r) for r in vhat],
                            [list(r) for r in R], [list(r) for r in R], 1 / math.sqrt(D))
        assert np.abs(np.array(ref) - o[h]).max() < 1e-14


# --------------------------------------------------------------------------
# layout arithmetic printed on the pages
# --------------------------------------------------------------------------

def test_bits_per_element_printed_values():
    g = _load("bits_per_element.json")
    for c in g["cases"]:
        v = orc.bits_per_element(c["L"], c["G"])
        assert round(v, c["decimals"]) == c["printed"], (c, v)
    s = g["bf16_share"]
    assert round(100 * 320 / s["L"], s["decimals"]) == s["printed_percent"]
    assert 16 / 2 == g["history_ratio"]["printed"]
    assert orc.history_bits_per_element(128) == 2.25 and orc.history_bits_per_element(64) == 2.5


def test_record_layout_hand_placed():
    """Byte positions of the page-record layout for D=64, G=32, worked by hand:
    64 lane slots of 2 words (K word of token t = l % 16, part kb = l // 16;
    V word of channel l) = 512 bytes, then 16 token slots of 4 words (K groups
    0, 1; V groups 0, 1; scale | zero << 16) = 256 bytes."""
    D, G = 64, 32
    kc = np.zeros((16, D), np.uint8); vc = np.zeros((16, D), np.uint8)
    ks = np.zeros((16, 2)); kz = np.zeros((16, 2)); vs = np.zeros((16, 2)); vz = np.zeros((16, 2))
    kc[3, 37] = 2         # channel 37 = 16*2 + 5: slot 35 word 0 (byte 280), bits 10..11 -> byte 281 = 0x08
    vc[9, 6] = 3          # channel 6: slot 6 word 1 (byte 52), token 9 bits 18..19 -> byte 54 = 0x0C
    vc[0, 17] = 1         # channel 17: slot 17 word 1 (byte 140), token 0 -> 0x01
    ks[2, 1] = 1.0        # token 2 slot at 512 + 32, K group 1 word at +4 -> 0x3F80
    kz[2, 1] = -2.0       # zero in the high half -> 0xC000
    vz[15, 0] = 0.5       # token 15 slot at 512 + 240, V group 0 word at +8, high half -> 0x3F00
    rec = orc.encode_record(kc, ks, kz, vc, vs, vz, D, G)
    assert rec.size == 768
    want = np.zeros(768, np.uint8)
    want[281] = 0x08
    want[54] = 0x0C
    want[140] = 0x01
    want[548:552] = [0x80, 0x3F, 0x00, 0xC0]
    want[762:764] = [0x00, 0x3F]
    assert np.array_equal(rec, want)


def test_record_layout_hand_placed_d128():
    """D=128, G=64: lane slots of 4 words (K blocks 0, 1 of token t part kb;
    V channels l, l + 64) = 1024 bytes, then token slots of 4 words (K groups 0, 1;
    V groups 0, 1) = 256 bytes; worked by hand."""
    D, G = 128, 64
    kc = np.zeros((16, D), np.uint8); vc = np.zeros((16, D), np.uint8)
    z2 = np.zeros((16, 2))
    kc[5, 70] = 1         # channel 70 = 64 + 16*0 + 6: slot 5 word 1 (byte 84), bits 12..13 -> byte 85 = 0x10
    kc[12, 127] = 3       # channel 127 = 64 + 16*3 + 15: slot 60 word 1 (byte 964), bits 30..31 -> byte 967 = 0xC0
    vc[1, 65] = 2         # channel 65: slot 1 word 3 (byte 28), token 1 bits 2..3 -> 0x08
    vc[15, 0] = 1         # channel 0: slot 0 word 2 (byte 8), token 15 bits 30..31 -> byte 11 = 0x40
    vs = z2.copy(); vs[7, 1] = 2.0   # token 7 slot at 1024 + 112, V group 1 word at +12 -> 0x4000
    rec = orc.encode_record(kc, z2, z2, vc, vs, z2, D, G)
    assert rec.size == 1280
    want = np.zeros(1280, np.uint8)
    want[85] = 0x10
    want[967] = 0xC0
    want[28] = 0x08
    want[11] = 0x40
    want[1024 + 112 + 12:1024 + 112 + 14] = [0x00, 0x40]
    assert np.array_equal(rec, want)


# --------------------------------------------------------------------------
# Lloyd-Max codebook variant
# --------------------------------------------------------------------------

def test_codebook_identity_levels_are_the_uniform_quantiser():
    """Levels (0, 1, 2, 3) reproduce quantize_groups (same codes, scales,
    zeros) on random groups; codebook dequantisation then equals dequant."""
    rng = np.random.default_rng(71)
    for G in (32, 64, 128):
        X = rng.standard_normal((500, 128)) * np.exp2(rng.integers(-6, 6, (500, 1)))
        a = orc.quantize_groups(X, G, 0.95)
        b = orc.quantize_groups_codebook(X, G, 0.95, (0.0, 1.0, 2.0, 3.0))
        for p, q in zip(a, b):
            assert np.array_equal(p, q)
        assert np.array_equal(orc.dequant(*a, G), orc.dequant_codebook(*b, G, (0.0, 1.0, 2.0, 3.0)))


def test_codebook_hand_worked():
    """One group worked by hand: x = 0..7 at G = 8, clip 1 -> scale 7/3
    (bf16 2.328125), zero 0; with levels (0.5, 1.25, 2, 2.75) the thresholds
    are 0.875, 1.625, 2.375, and u = x / 2.328125 = 0, 0.430, 0.859, 1.289,
    1.718, 2.148, 2.577, 3.007 gives codes 0,0,0,1,2,2,3,3 (0.859 is just
    below the first threshold); x_hat = 2.328125 * L[code]."""
    x = np.arange(8, dtype=np.float64)[None, :]
    L = (0.5, 1.25, 2.0, 2.75)
    c, s, z = orc.quantize_groups_codebook(x, 8, 1.0, L)
    assert s[0, 0] == 2.328125 and z[0, 0] == 0.0
    assert c[0].tolist() == [0, 0, 0, 1, 2, 2, 3, 3]
    assert np.array_equal(orc.dequant_codebook(c, s, z, 8, L)[0], 2.328125 * np.array(L)[c[0]])


def test_codebook_nearest_level_brute_force():
    """Every code is the level nearest to u = (x - zero_b)/scale_b (brute force
    over the 4 levels), for random ascending codebooks."""
    rng = np.random.default_rng(72)
    for _ in range(20):
        L = np.sort(rng.uniform(-0.2, 3.2, 4)).astype(np.float32)
        X = rng.standard_normal((40, 64)) * 2.0
        c, s, z = orc.quantize_groups_codebook(X, 32, 0.9, L)
        u = (X.reshape(40, 2, 32) - z[:, :, None]) / s[:, :, None]
        want = np.argmin(np.abs(u[..., None] - L.astype(np.float64)), axis=-1)
        assert np.array_equal(c.reshape(40, 2, 32), want)


def test_lloyd_max_gaussian_textbook_levels():
    """4-level Lloyd-Max quantiser of a unit Gaussian: levels +-0.4528 and
    +-1.510, thresholds 0 and +-0.9816, mean squared error 0.1175 (Max 1960,
    the N = 4 row of the Gaussian table)."""
    rng = np.random.default_rng(73)
    x = rng.standard_normal(2_000_000)
    x = np.concatenate([x, -x])                  # exactly symmetric sample
    lv = orc.lloyd_max_levels(x)
    assert np.allclose(lv, [-1.510, -0.4528, 0.4528, 1.510], atol=4e-3)
    assert np.allclose(0.5 * (lv[:-1] + lv[1:]), [-0.9816, 0.0, 0.9816], atol=4e-3)
    th = 0.5 * (lv[:-1] + lv[1:])
    mse = np.mean((x - lv[np.searchsorted(th, x)]) ** 2)
    assert abs(mse - 0.1175) < 1e-3


def test_lloyd_max_uniform_and_distortion():
    """On a uniform sample over [0, 3] the levels are the cell midpoints
    3(2k+1)/8; started from the uniform levels on Gaussian-shaped group values,
    the fitted codebook never has a larger quantisation error than the uniform
    one (each Lloyd step lowers the distortion)."""
    rng = np.random.default_rng(74)
    lv = orc.lloyd_max_levels(rng.uniform(0.0, 3.0, 1_000_000))
    assert np.allclose(lv, 3.0 * (2 * np.arange(4) + 1) / 8, atol=5e-3)
    X = rng.standard_normal((4000, 64))
    c, s, z = orc.quantize_groups(X, 64, 0.95)
    u = ((X.reshape(4000, 1, 64) - z[:, :, None]) / s[:, :, None]).ravel()
    L = orc.lloyd_max_levels(u, init=(0.0, 1.0, 2.0, 3.0)).astype(np.float32)
    err_u = np.mean((orc.dequant(c, s, z, 64) - X) ** 2)
    cb = orc.quantize_groups_codebook(X, 64, 0.95, L)
    err_l = np.mean((orc.dequant_codebook(*cb, 64, L) - X) ** 2)
    assert err_l < err_u
