"""The parity checks themselves (CPU): the block-local bound catches a
localized error that the per-matrix relative Frobenius bound lets through."""
import numpy as np
import pytest

from helpers import BLOCK_FACTOR, TOL_16, block_errors, check_close, dw_discounted, rel_fro


def _orthogonal(n, seed):
    q, r = np.linalg.qr(np.random.default_rng(seed).standard_normal((n, n)))
    return q * np.sign(np.diag(r))


def _noisy(o, rel, seed):
    """o plus spread-out noise of relative Frobenius size ``rel`` (the shape
    of 16-bit rounding error)."""
    rms = np.sqrt(np.mean(o * o))
    return o + rel * rms * np.random.default_rng(seed).standard_normal(o.shape)


def test_spread_error_passes_both_checks():
    o = _orthogonal(1024, 1)
    gpu = _noisy(o, 1e-2, 2)
    assert rel_fro(gpu, o) < TOL_16
    check_close(gpu, o, TOL_16, "spread error")


@pytest.mark.parametrize("how", ["zero", "half", "sign"])
def test_one_wrong_mfma_block_fails_block_check(how):
    """One wrong 16 x 16 accumulator block in a 1024 x 1024 output: the
    matrix-wide relative error stays under the 2e-2 tolerance, the block
    check fails."""
    o = _orthogonal(1024, 3)
    gpu = _noisy(o, 1e-2, 4)
    blk = gpu[512:528, 272:288]
    if how == "zero":
        blk[:] = 0.0
    elif how == "half":
        blk *= 0.5
    else:
        blk[:4, :4] *= -1.0
    assert rel_fro(gpu, o) <= TOL_16, "the old check alone would pass this"
    with pytest.raises(AssertionError, match=r"block \(512, 256\)"):
        check_close(gpu, o, TOL_16, "planted")


def test_one_wrong_tile_in_a_tall_matrix():
    """One 64 x 64 output tile of a 4096 x 1024 matrix 20% off (a wrong
    scale on one wave's sub-tile): the matrix-wide error stays under half
    the tolerance, the tile's block reads 0.2, over 3x the block bound."""
    rng = np.random.default_rng(5)
    q, _ = np.linalg.qr(rng.standard_normal((4096, 1024)))
    gpu = _noisy(q, 5e-3, 6)
    gpu[1024:1088, 640:704] *= 1.2
    assert rel_fro(gpu, q) <= TOL_16
    with pytest.raises(AssertionError):
        check_close(gpu, q, TOL_16, "planted tile")


def test_block_errors_ragged_edges_and_units():
    ref = np.ones((70, 130))
    out = ref.copy()
    out[64:, 128:] += 2.0                 # the 6 x 2 corner block only
    b = block_errors(out, ref)
    assert b.shape == (2, 3)
    assert b[1, 2] == pytest.approx(2.0)  # rms error 2 in units of rms(ref) = 1
    assert np.count_nonzero(b) == 1
    assert BLOCK_FACTOR * TOL_16 < 2.0


def test_dw_discount_covers_only_the_fp32_store():
    """The dW check forgives the fp32 rounding of W_new and nothing more: a
    correctly rounded W_new passes at any update size, an update off by
    1e-4 of itself still fails."""
    rng = np.random.default_rng(9)
    w_old = (0.02 * rng.standard_normal((512, 512))).astype(np.float32).astype(np.float64)
    o = 1e-3 * rng.standard_normal((512, 512))          # tiny update (low-rank O scale)
    w_ref = w_old - 0.02 * (o + 0.01 * w_old)           # exact (fp64)
    w_gpu = w_ref.astype(np.float32).astype(np.float64)   # stored in fp32
    dw_ref, dw_gpu = w_ref - w_old, w_gpu - w_old
    assert rel_fro(dw_gpu, dw_ref) > 1e-5                 # the storage floor alone
    check_close(dw_discounted(dw_gpu, dw_ref, w_ref), dw_ref, 1e-5, "stored W_new")
    off = w_old + (1.0 + 1e-4) * dw_ref
    with pytest.raises(AssertionError):
        check_close(dw_discounted(off - w_old, dw_ref, w_ref), dw_ref, 1e-5, "wrong update")
