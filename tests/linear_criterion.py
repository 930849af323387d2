"""The named criterion of the linear product with q8_1 activations.

The product's reduction order and intermediate precision belong to the kernel
(NInfer "tensor-formats": the consumer paragraph of the conformance section);
its result is judged against the oracle's binary64 value y_ref by the
classical bound of a binary32 summation of K terms in any order, each term
carrying at most 8 further roundings (a product, an FMA chain of 8 within a
unit, a scale multiply):

    |y - y_ref| <= gamma(K + 8) * env + (K + 8) * 2^-148,
    gamma(n) = n u / (1 - n u), u = 2^-24,

with env = sum_k |x| E from the oracle (E = |w|, or |w| + 2|o| for the
formats whose value adds a code-independent term o).  The absolute term
covers results in binary32's subnormal range (each rounding there errs by
at most 2^-150).
"""
import numpy as np


def criterion(K, env):
    n = K + 8
    u = 2.0 ** -24
    return n * u / (1 - n * u) * np.asarray(env, dtype=np.float64) + n * 2.0 ** -148


def check(y, ref, env, K, what=""):
    """Assert y (any float array) is within the criterion of ref; returns
    the largest error as a fraction of the bound."""
    err = np.abs(np.asarray(y, dtype=np.float64) - ref)
    tol = criterion(K, env)
    bad = ~(err <= tol)  # NaN fails
    assert not np.any(bad), (f"{what}: {int(bad.sum())} outputs outside the criterion, first at "
                             f"{np.argwhere(bad)[0].tolist()}: got {np.asarray(y)[bad][0]!r}, "
                             f"oracle {ref[bad][0]!r}, bound {tol[bad][0]!r}")
    return float(np.max(err / tol)) if err.size else 0.0
