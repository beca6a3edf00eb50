"""The activation fake-quant's difference D = X_q - X is exact in the input format whenever no
block's scale saturated far below its amax (max|x| / (6 gX) <= 672): the accumulation that makes
X_q in the kernel stages D as one bf16 (or fp32) piece on that condition and splits it like a
stored X_q otherwise.  Checked here on the oracle's own quantizer (float64, exact rounding
decisions), with blocks at every scale from deep subnormal to saturated, E2M1 midpoints and
ties, and the exactness also failing where the condition does not hold (so the guard is needed)."""
import numpy as np

import oracle
from synth.configs import bf16_bits_from_f32


def _bf16(a):
    """float64 values of the bf16 rounding (nearest-even) of a."""
    b = bf16_bits_from_f32(np.asarray(a, dtype=np.float32))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _is_bf16(a):
    f = np.asarray(a, dtype=np.float32)
    return np.all(f.astype(np.float64) == a) and np.all((f.view(np.uint32) & 0xFFFF) == 0)


def _rows(rng, n):
    """Rows of 16-element blocks: Gaussian, heavy-tailed, one dominant element, all tiny, and
    elements on E2M1 midpoints of a power-of-two scale."""
    X = rng.standard_normal((n, 64))
    X[::5] = rng.standard_t(2, (len(X[::5]), 64))
    X[1::5, ::16] *= 300.0
    X[2::5] *= 2.0 ** rng.integers(-140, -120, (len(X[2::5]), 1))
    X[3::5] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5], (len(X[3::5]), 64)) * \
        2.0 ** rng.integers(-3, 3, (len(X[3::5]), 1)) * rng.choice([-1.0, 1.0], (len(X[3::5]), 64))
    return X


def test_difference_is_exact_unless_the_scale_saturates_far_below():
    rng = np.random.default_rng(91)
    # amax 0.7 of max|X|: scales saturate with y up to 640 (kept exact); 0.25: up to 1792 (some
    # blocks go to the split); 1e-30: every block saturates
    for bf16, amax_scale in [(True, 1.0), (True, 4.0), (False, 1.0), (True, 0.7), (False, 0.7),
                             (True, 0.25), (True, 1e-30), (False, 1e30)]:
        X = _rows(rng, 400)
        X = _bf16(X) if bf16 else X.astype(np.float32).astype(np.float64)
        amax = float(np.abs(X).max()) * amax_scale
        Xq = oracle.activation_fake_quant(X, [amax], np.array([0, len(X)]), bf16=bf16)
        D = Xq - X                                    # exact in float64
        gx = float(np.float32(np.float32(amax) / np.float32(2688.0)))
        y = np.abs(X).reshape(len(X), -1, 16).max(-1) / (6.0 * gx) if gx > 0 else np.zeros((len(X), 4))
        ok = np.repeat(~(y > 672.0), 16, axis=1)      # the kernel's condition, per element
        if bf16:
            exact = (_bf16(D) == D) | (D == 0)
        else:
            exact = D.astype(np.float32).astype(np.float64) == D
        assert np.all(exact[ok]), (bf16, amax_scale, np.argwhere(~exact & ok)[:3])
        if amax_scale >= 0.7:
            assert ok.all()                           # an amax near max|X| never saturates far
        else:
            assert not ok.all()                       # the guard's case occurs


def test_far_saturation_can_make_the_difference_inexact():
    # amax 2^-12 of the data: blocks saturate at 448 g, so x_q = 6 s is far below x and
    # x_q - x needs more than 8 significant bits
    X = _bf16(np.array([[1.0078125 * 2.0 ** 10] + [0.0] * 15]))
    amax = float(np.abs(X).max()) * 2.0 ** -12
    Xq = oracle.activation_fake_quant(X, [amax], np.array([0, 1]), bf16=True)
    D = Xq - X
    assert not _is_bf16(D[0, :1])
