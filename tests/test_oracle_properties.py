"""Property tests (hypothesis) of the CPU oracle: the group quantiser, the
codebook variant, packing and the log-sum-exp merge, over generated inputs
including the edge cases hypothesis searches for (constant groups, tiny and
huge magnitudes, empty chunks).  CPU only."""
import math

import numpy as np
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

from oracle import oscar_oracle as orc

FINITE = st.floats(min_value=-1e4, max_value=1e4, allow_nan=False, allow_infinity=False, width=32)
SETTINGS = settings(max_examples=150, deadline=None)


@st.composite
def groups(draw, G=8):
    rows = draw(st.integers(1, 4))
    x = draw(hnp.arrays(np.float64, (rows, 2 * G), elements=FINITE))
    scale = draw(st.sampled_from([1e-3, 1.0, 1e3]))
    return x * scale


@SETTINGS
@given(groups(), st.sampled_from([1.0, 0.95, 0.5]))
def test_quantiser_properties(x, clip):
    """Codes in {0..3}; scale and zero are bf16 values; scale >= 0; inside the
    clipped range every value is within half a step (plus the bf16 slack of
    scale and zero) of its dequantised value; a group whose scale rounds to 0
    has all codes 0."""
    G = 8
    c, s, z = orc.quantize_groups(x, G, clip)
    assert c.dtype == np.uint8 and c.max() <= 3
    assert np.all(orc.bf16_round(s) == s) and np.all(orc.bf16_round(z) == z)
    assert np.all(s >= 0)
    xh = orc.dequant(c, s, z, G).reshape(x.shape[0], -1, G)
    xg = x.reshape(x.shape[0], -1, G)
    cg = c.reshape(x.shape[0], -1, G)
    assert np.all(cg[s == 0] == 0)
    inside = (xg >= z[..., None]) & (xg <= z[..., None] + 3 * s[..., None])
    err = np.abs(xh - xg)
    bound = s[..., None] * (0.5 + 1e-12) + 1e-300
    assert np.all(err[inside & (s[..., None] > 0)] <= np.broadcast_to(bound, err.shape)[inside & (s[..., None] > 0)])


@SETTINGS
@given(groups(), st.lists(st.floats(-0.5, 3.5, allow_nan=False, width=32), min_size=4, max_size=4))
def test_codebook_nearest_level(x, lv):
    """With any ascending codebook, the code is the level nearest to
    u = (x - zero)/scale (ties to the lower level), and dequantisation gives
    zero + scale * level."""
    G = 8
    L = np.sort(np.array(lv, np.float32))
    c, s, z = orc.quantize_groups_codebook(x, G, 0.95, L)
    u = (x.reshape(x.shape[0], -1, G) - z[..., None]) / np.where(s == 0, 1.0, s)[..., None]
    d = np.abs(u[..., None] - L.astype(np.float64))
    cg = c.reshape(x.shape[0], -1, G)
    best = d.min(axis=-1)
    chosen = np.take_along_axis(d, cg[..., None].astype(np.int64), -1)[..., 0]
    live = np.broadcast_to((s != 0)[..., None], cg.shape)
    assert np.all(chosen[live] <= best[live] * (1 + 1e-12) + 1e-300)
    assert np.all(cg[~live] == 0)
    xh = orc.dequant_codebook(c, s, z, G, L).reshape(cg.shape)
    assert np.array_equal(xh, z[..., None] + s[..., None] * L.astype(np.float64)[cg])


@SETTINGS
@given(hnp.arrays(np.uint8, st.tuples(st.integers(1, 5), st.sampled_from([4, 16, 64, 128])),
                  elements=st.integers(0, 3)))
def test_pack_round_trip(codes):
    """Packing four codes per byte and unpacking is the identity, and byte i
    holds codes 4i..4i+3 LSB first."""
    packed = orc.pack_rows(codes)
    assert packed.shape == (codes.shape[0], codes.shape[1] // 4)
    assert np.array_equal(orc.unpack_rows(packed, codes.shape[1]), codes)
    i = codes.shape[1] // 4 - 1
    want = sum(int(codes[0, 4 * i + k]) << (2 * k) for k in range(4))
    assert int(packed[0, i]) == want


@SETTINGS
@given(st.integers(1, 60), st.integers(1, 6), st.data())
def test_merge_of_any_chunking_is_one_softmax(n, D, data):
    """Partials of any cut of the tokens into chunks (empty chunks included)
    merged by the log-sum-exp merge give the single-pass softmax."""
    s = np.array(data.draw(st.lists(st.floats(-50, 50, allow_nan=False), min_size=n, max_size=n)))
    v = np.array(data.draw(st.lists(st.floats(-10, 10, allow_nan=False), min_size=n * D,
                                    max_size=n * D))).reshape(n, D)
    cuts = sorted(data.draw(st.lists(st.integers(0, n), max_size=6)))
    edges = [0] + cuts + [n]
    parts = [orc.partial_softmax(s[a:b], v[a:b]) for a, b in zip(edges[:-1], edges[1:])]
    M, L, O = orc.lse_merge(parts)
    m = s.max()
    e = np.exp(s - m)
    assert M == m
    assert math.isclose(L, e.sum(), rel_tol=1e-12)
    assert np.allclose(O / L, (e @ v) / e.sum(), rtol=1e-12, atol=1e-12)


def test_symmetric_codebook_generator():
    """The symmetric Lloyd-Max stand-in: ascending levels inside the group
    range [0, 3], mirrored about 1.5, with L3 - L2 - L1 + L0 exactly 0 when
    evaluated in float32 in the kernels' order (the condition under which the
    matrix-core kernel skips its b0&b1 plane)."""
    from synth import inputs as syn
    for seed in range(5):
        cb = syn.make_codebook(seed, 8, symmetric=True)
        assert cb.dtype == np.float32 and cb.shape == (8, 2, 4)
        assert np.all(np.diff(cb, axis=-1) > 0) and np.all(cb >= 0) and np.all(cb <= 3)
        assert np.all(cb[..., 0] + cb[..., 3] == np.float32(3)) and np.all(cb[..., 1] + cb[..., 2] == np.float32(3))
        cc = ((cb[..., 3] - cb[..., 2]) - cb[..., 1]) + cb[..., 0]
        assert np.all(cc == 0)
        # the fitted (asymmetric) stand-in keeps a non-zero term
        fit = syn.make_codebook(seed, 8)
        assert np.any(((fit[..., 3] - fit[..., 2]) - fit[..., 1]) + fit[..., 0] != 0)
