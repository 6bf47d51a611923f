"""Seeded synthetic inputs: determinism and the stated distributions."""
import numpy as np

import synth


def test_seeded_and_distinct_streams():
    a = synth.make_layer(64, 48, 16, 2, cfg=3, block=1, layer=2)
    b = synth.make_layer(64, 48, 16, 2, cfg=3, block=1, layer=2)
    c = synth.make_layer(64, 48, 16, 2, cfg=3, block=1, layer=3)
    for name in ("U", "V", "s1", "g", "s2", "x"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert not np.array_equal(a.U, c.U)


def test_distributions():
    L = synth.make_layer(512, 256, 64, 4, scale_dtype="f16")
    assert set(np.unique(L.U)) == {-1, 1} and set(np.unique(L.V)) == {-1, 1}
    assert abs(L.U.mean()) < 0.02
    for s in (L.s1, L.g, L.s2):
        assert s.dtype == np.float16 and float(s.min()) >= 0.0999
    # x is bf16-representable: the low 16 bits of each fp32 word are zero
    assert np.all((L.x.view(np.uint32) & 0xFFFF) == 0)


def test_bf16_rounding_ties_to_even():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8], np.float32)
    r = synth.round_to_bf16(v)
    assert r[0] == 1.0 and r[1] == 1.0 + 2 * 2.0 ** -7 and r[2] == -1.0
