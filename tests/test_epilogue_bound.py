"""CPU pin of the end-to-end bound used for the fused prefill epilogue
(kda_testutil.epilogue_bound): perturbing the oracle's o~ by any error within
the core's bound moves the oracle's own eq. (6) epilogue output by no more
than the bound says.  Random and adversarial perturbations (every element at
+/- e, the sign pattern that shrinks or grows the row's RMS), rows whose RMS
is far above, near and below e."""
import numpy as np

import oracle.layer as L
from kda_testutil import epilogue_bound


def _check(o, gate, w, eps, tol, d):
    dev, _ = epilogue_bound(o, gate, w, eps, tol)
    y0 = L.epilogue(o, gate, w, eps)
    y1 = L.epilogue(o + d, gate, w, eps)
    assert np.all(np.abs(y1 - y0) <= dev * (1 + 1e-12) + 1e-300), float(np.max(np.abs(y1 - y0) / dev))


def test_bound_holds_random_and_adversarial():
    rng = np.random.default_rng(0)
    T, H, D = 64, 3, 128
    o = rng.standard_normal((T, H, D))
    o[::7] *= 1e-3          # rows far below the allowed error
    o[1::7] *= 3e-2         # rows near it
    gate = rng.standard_normal((T, H, D))
    w = 1.0 + 0.1 * rng.standard_normal((H, D))
    tol, eps = 2e-2, 1e-6
    e = tol * np.max(np.abs(o))
    for trial in range(20):
        d = rng.uniform(-e, e, o.shape)
        _check(o, gate, w, eps, tol, d)
    # every element at +-e: same sign as o (grows the RMS), opposite (shrinks it), random signs
    _check(o, gate, w, eps, tol, e * np.sign(o))
    _check(o, gate, w, eps, tol, -e * np.sign(o))
    _check(o, gate, w, eps, tol, e * np.where(rng.random(o.shape) < 0.5, -1.0, 1.0))
    # a single element moved by e in the row's largest entry
    d = np.zeros_like(o)
    idx = np.argmax(np.abs(o), axis=-1)
    np.put_along_axis(d, idx[..., None], e, axis=-1)
    _check(o, gate, w, eps, tol, d)


def test_bound_is_not_vacuous_for_typical_rows():
    """For rows whose RMS is well above the allowed error the bound is a few
    times the allowed relative error, not the trivial 2 sqrt(d_v)."""
    rng = np.random.default_rng(1)
    o = rng.standard_normal((16, 2, 128))
    gate = np.zeros_like(o)
    w = np.ones((2, 128))
    dev, s = epilogue_bound(o, gate, w, 1e-6, 2e-2)
    # |n|_inf ~ 3-4 for Gaussian rows, e / r ~ 2e-2 * 4 -> bound ~ 0.5 * 0.08 * 5
    assert np.max(dev) < 0.5 and np.max(dev) < 2 * np.sqrt(128) * 0.5 / 10
