"""The parity metrics themselves, on the CPU: the per-vector bound catches a single
wrong row or tile that the whole-tensor Frobenius ratio of the diffusers issue "Ring
attention backward uses stale iteration-0 KV" (section Reproduction) lets through, and
neither fails on rounding-sized noise or on vectors that are legitimately zero."""
import numpy as np
import pytest

from parity import BF16_TOL, check_bf16, rel, vec_rel_max


def _ref(shape=(1, 4096, 4, 128), seed=3):
    return np.random.default_rng(seed).standard_normal(shape)


def test_bf16_rounding_noise_passes_both():
    ref = _ref()
    got = ref * (1 + np.random.default_rng(4).uniform(-2 ** -8, 2 ** -8, ref.shape))
    r, v = check_bf16("noise", got, ref, log=False)
    assert r < 3e-3 and v < 1e-2


def test_one_wrong_row_fails_only_the_vector_bound():
    ref = _ref()
    got = ref.copy()
    got[0, 1234, 2] = 0.0  # one (row, head) vector of 16384 lost entirely
    assert rel(got, ref) < BF16_TOL            # invisible to the Frobenius ratio
    assert vec_rel_max(got, ref) > 0.9          # the vector bound sees it
    with pytest.raises(AssertionError):
        check_bf16("row", got, ref, log=False)


def test_wrong_tail_tile_fails():
    ref = _ref()
    got = ref.copy()
    got[0, -9:, :, :] *= 1.3  # a partial last tile of 9 rows off by 30 %
    assert rel(got, ref) < BF16_TOL
    with pytest.raises(AssertionError):
        check_bf16("tail", got, ref, log=False)


def test_zero_vectors_are_judged_against_the_floor():
    ref = _ref()
    ref[0, :100] = 0.0                       # e.g. masked rows: the true value is exactly 0
    got = ref.copy()
    assert vec_rel_max(got, ref) == 0.0
    got[0, :100] = 1e-4                      # tiny absolute error on a zero vector: fine
    assert vec_rel_max(got, ref) < 1e-3
    got[0, 7] = ref[0, 200]                  # a whole wrong vector where zero belongs: caught
    assert vec_rel_max(got, ref) > 0.5
