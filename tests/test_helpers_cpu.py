"""The parity metric of the GPU tests (tests/_helpers.rel_err), on the CPU.

rel_err takes the largest relative error over pieces of a tensor (a row cut
into runs of 256 columns; each element of a vector on its own), so that one
wrong column of a wide layer fails the bf16 bar of 2e-2 although it moves the
whole-tensor Frobenius error by only about 1/sqrt(columns)."""
import numpy as np

from _helpers import TOL, rel_err, rel_fro


def test_one_wrong_column_of_a_wide_matrix_fails():
    rng = np.random.default_rng(0)
    want = rng.standard_normal((64, 8192))
    got = want.copy()
    got[:, 5000] = rng.standard_normal(64)          # one column wrong
    assert rel_fro(got, want) < TOL["bf16"]           # averaged away ...
    assert rel_err(got, want) > TOL["bf16"]           # ... but not per piece


def test_one_wrong_sample_norm_fails():
    want = np.linspace(1.0, 2.0, 64)
    got = want.copy()
    got[17] *= 1.05
    assert rel_fro(got, want) < TOL["bf16"]
    assert abs(rel_err(got, want) - 0.05) < 1e-12


def test_uniform_noise_is_measured_like_the_tensor_metric():
    rng = np.random.default_rng(1)
    want = rng.standard_normal((128, 3072))
    got = want * (1.0 + 1e-3 * rng.standard_normal(want.shape))
    a, b = rel_fro(got, want), rel_err(got, want)
    assert a <= b <= 2.0 * a


def test_last_piece_and_zero_reference():
    want = np.zeros((3, 300))
    got = np.zeros((3, 300))
    got[2, 299] = 1e-7
    assert rel_err(got, want) == 1e-7      # absolute where the reference is 0
    want[:, :] = 1.0
    got = want.copy()
    got[1, 260] = 1.1                        # in the last piece: columns 44..299
    assert abs(rel_err(got, want) - 0.1 / np.sqrt(256)) < 1e-12
    narrow = np.ones((2, 40))
    bad = narrow.copy()
    bad[0, 3] = 2.0                          # a row narrower than a piece
    assert abs(rel_err(bad, narrow) - 1.0 / np.sqrt(40)) < 1e-12


def test_dw_metric_takes_out_only_the_storage_rounding():
    """W_new = fl32(W_old + dW): the update itself is exact, so the metric is
    0 although the plain difference is off by up to 1e-5 of dW; an update
    wrong by 1e-4 is still seen (less at most half an ulp per element)."""
    from _helpers import rel_err_dw
    rng = np.random.default_rng(2)
    W_old = (rng.standard_normal((64, 512)) / 8.0).astype(np.float32)
    dW = 1e-3 * rng.standard_normal((64, 512))
    W_new = (W_old.astype(np.float64) + dW).astype(np.float32)
    plain = rel_err(W_new.astype(np.float64) - W_old, dW)
    assert plain > 2e-6                          # the rounding of W alone
    assert rel_err_dw(W_new, W_old, dW) == 0.0
    W_bad = (W_old.astype(np.float64) + dW * (1 + 1e-4)).astype(np.float32)
    assert 0.8e-4 < rel_err_dw(W_bad, W_old, dW) < 1.2e-4
