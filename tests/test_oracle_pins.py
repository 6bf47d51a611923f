"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

from oracle import nq_oracle as O
from tests.oracle_pins import PINS, load_golden

MODES = {"dense": O.linear_dense, "factored": O.linear_factored}


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, mode):
    pin(MODES[mode])


def test_dense_weight_hand_example():
    ex = load_golden("hand_examples.json")["examples"][1]
    W = O.reconstruct_weight(np.array(ex["U"], np.int8), np.array(ex["V"], np.int8),
                             ex["s1"], ex["g"], ex["s2"])
    assert np.array_equal(W, np.array(ex["W"]))


def test_rejects_non_signs():
    U = np.array([[1, 0]], np.int8)
    V = np.array([[1, 1]], np.int8)
    with pytest.raises(ValueError):
        O.linear_dense(np.ones((1, 1)), U, V, [1.0], [1.0, 1.0], [1.0])


# ------------------------------------------------------------------ storage accounting
def test_storage_examples():
    d = load_golden("storage_examples.json")
    for ex in d["examples"]:
        assert O.bits_per_weight(ex["m"], ex["n"], ex["r"], ex["scale_bits"]) == ex["bpw"]
        assert ex["r"] * (ex["m"] + ex["n"]) == ex["sign_bits"]


@pytest.mark.parametrize("m,n", [(256, 256), (4096, 4096), (11008, 4096), (4096, 11008),
                                 (8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672),
                                 (63, 17), (1, 1)])
@pytest.mark.parametrize("bpw", [0.55, 0.8, 1.0, 2.5])
def test_rank_for_bits_is_maximal(m, n, bpw):
    r = O.rank_for_bits(m, n, bpw, 16)
    if r == 0:
        assert O.bits_per_weight(m, n, 1, 16) > bpw
        return
    assert O.bits_per_weight(m, n, r, 16) <= bpw < O.bits_per_weight(m, n, r + 1, 16)


def test_rank_brute_force_small():
    """Against exhaustive search over every rank."""
    for m in range(1, 40, 7):
        for n in range(1, 40, 5):
            for bpw in (0.3, 0.8, 1.0, 3.0):
                best = max([r for r in range(1, 200) if O.bits_per_weight(m, n, r, 16) <= bpw],
                           default=0)
                assert O.rank_for_bits(m, n, bpw, 16) == best


def test_sub_one_bit_at_small_rank():
    """Small enough r puts the average below one bit (sub-1-bit accounting)."""
    r = O.rank_for_bits(8192, 8192, 0.8, 16)
    assert 0 < r and O.bits_per_weight(8192, 8192, r, 16) < 1.0
    # the 0.8 bpw operating point for a 70B-shaped q projection
    assert r == 3257


def test_compression_ratio_matches_pages_figure():
    """The pages print 138.04 GB -> 5.35 GB and call it 25.8x: the average stored
    bits per weight implied by the two sizes must give back the printed ratio."""
    d = load_golden("pages_figures.json")
    bpw = 16.0 * d["compressed_gb"] / d["fp16_gb"]          # about 0.62 bits per weight
    assert round(O.compression_ratio(bpw), d["ratio_decimals"]) == d["ratio_printed"]
    # the 0.8 bits/weight operating point alone would give 20x, not 25.8x: the
    # printed run used fewer bits per weight than the headline operating point
    assert O.compression_ratio(0.8) == 20.0 and bpw < 0.8


def test_stored_bytes_llama70b_linears_at_0p8():
    """80 blocks of q, k, v, o, gate, up, down at the 0.8 bpw ranks: the stored
    bytes equal 0.8 bits per weight over 68.45 G weights to within the rank
    rounding (every layer's realised bpw is at most 0.8 and above 0.798)."""
    shapes = [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192), (28672, 8192),
              (8192, 28672)]
    weights = 80 * sum(m * n for m, n in shapes)
    assert weights == 68_451_041_280
    total = 80 * sum(O.stored_bytes(m, n, O.rank_for_bits(m, n, 0.8, 16), 16) for m, n in shapes)
    assert 0.798 * weights / 8 < total <= 0.8 * weights / 8
    with pytest.raises(ValueError):
        O.compression_ratio(0.0)


# ------------------------------------------------------------------ pins catch mistakes
def _mutants():
    f64 = lambda a: np.asarray(a, np.float64)

    def swapped_scales(x, U, V, s1, g, s2):       # s1 and s2 trade places (square only)
        return O.linear_factored(x, U, V, s2[:len(s1)] if len(s2) >= len(s1) else np.resize(s2, len(s1)),
                                 g, np.resize(s1, len(s2)))

    def dropped_g(x, U, V, s1, g, s2):
        return O.linear_factored(x, U, V, s1, np.ones_like(f64(g)), s2)

    def dropped_s1(x, U, V, s1, g, s2):
        return O.linear_factored(x, U, V, np.ones_like(f64(s1)), g, s2)

    def dropped_s2(x, U, V, s1, g, s2):
        return O.linear_factored(x, U, V, s1, g, np.ones_like(f64(s2)))

    def sign_inverted_V(x, U, V, s1, g, s2):      # bit meaning flipped on one factor
        return O.linear_factored(x, U, -np.asarray(V), s1, g, s2)

    def transposed_W(x, U, V, s1, g, s2):         # y = x W_hat instead of x W_hat^T
        W = O.reconstruct_weight(U, V, s1, g, s2)
        if W.shape[0] != W.shape[1]:
            return (f64(x) @ np.resize(W, (W.shape[1], W.shape[0]))).astype(np.float64)
        return f64(x) @ W

    def rank_index_shift(x, U, V, s1, g, s2):     # g applied to the wrong rank index
        return O.linear_factored(x, U, V, s1, np.roll(f64(g), 1), s2)

    def one_term_dropped(x, U, V, s1, g, s2):     # last rank-1 term missing
        gg = f64(g).copy()
        gg[-1] = 0.0
        return O.linear_factored(x, U, V, s1, gg, s2)

    def abs_instead_of_sign(x, U, V, s1, g, s2):  # signs lost on U
        return O.linear_factored(x, np.abs(np.asarray(U)), V, s1, g, s2)

    def float32_accumulation(x, U, V, s1, g, s2):  # precision loss in the oracle
        xs = (np.asarray(x, np.float32) * np.asarray(s2, np.float32))
        t = (xs @ np.asarray(V, np.float32)) * np.asarray(g, np.float32)
        return (t @ np.asarray(U, np.float32).T) * np.asarray(s1, np.float32)

    return [swapped_scales, dropped_g, dropped_s1, dropped_s2, sign_inverted_V, transposed_W,
            rank_index_shift, one_term_dropped, abs_instead_of_sign, float32_accumulation]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutant):
    failures = 0
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            failures += 1
    assert failures >= 1, f"no pin caught {mutant.__name__}"
