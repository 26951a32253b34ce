"""Rotations and the QJL projection (oracle side, float64).

Structured variant ([Design Study] "Dense and structured transform comparison";
[Reconstruction] section 9 "Transform Implementation Tradeoffs"): a seeded
Rademacher sign flip followed by a fast Walsh-Hadamard transform,
y = H_n D u with H_n = H / sqrt(d).  READING: H is the Sylvester (natural
order) Hadamard matrix, H[i, j] = (-1)^popcount(i & j).

Dense variant ([Reconstruction] section 5 "Step 2: Random Rotation"): Pi from
the QR decomposition of a standard Gaussian matrix, fixed globally.  READING:
the sign of each column of Q is fixed so that diag(R) > 0, which makes Pi a
function of the Gaussian matrix alone.

QJL projection ([Reconstruction] section 6 "The 1-Bit QJL Transform"): S with
i.i.d. N(0,1) entries in the dense variant.  READING for the structured
variant: S = H D2 H_n D1, a two-round Rademacher-Hadamard sketch whose rows have
squared norm d (S S^T = d I) like Gaussian rows in expectation; the page's
multiplier-free line replaces dense projections by Rademacher + FWHT.  One
round is measurably biased at d = 128; two rounds meet the < 0.1 % bias of
[README] "Paper Validation (Theorems 1-3)"; the unbiasedness test pins this.
"""
import numpy as np

from . import rng


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis, natural order.

    Butterfly stage with half-width h pairs index i with i + h inside blocks of
    2h and maps (a, b) -> (a + b, a - b); after all log2(d) stages the result is
    H x with H[i, j] = (-1)^popcount(i & j).
    """
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    if d & (d - 1):
        raise ValueError("FWHT needs a power-of-two length")
    lead = x.shape[:-1]
    h = 1
    while h < d:
        v = x.reshape(lead + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :]
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return x


def haar_orthogonal(seed: int, role: int, d: int) -> np.ndarray:
    """Pi = Q diag(sign(diag R)) for Q R = the seeded d x d Gaussian matrix."""
    a = rng.gaussian(seed, role, d, d)
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


class Transforms:
    """The four transforms of one configuration: key rotation, value rotation,
    the QJL projection S, and their transposes."""

    def __init__(self, d: int, rotation: str, seed: int):
        self.d = d
        self.rotation = rotation
        self.seed = seed
        if rotation == "fwht":
            self.dk = rng.sign_vector(seed, rng.ROLE_KEY_SIGNS, d)
            self.ds1 = rng.sign_vector(seed, rng.ROLE_SKETCH_SIGNS_1, d)
            self.ds2 = rng.sign_vector(seed, rng.ROLE_SKETCH_SIGNS_2, d)
            self.dv = rng.sign_vector(seed, rng.ROLE_VALUE_SIGNS, d)
        elif rotation == "dense":
            self.pk = haar_orthogonal(seed, rng.ROLE_KEY_GAUSS, d)
            self.g = rng.gaussian(seed, rng.ROLE_SKETCH_GAUSS, d, d)
            self.pv = haar_orthogonal(seed, rng.ROLE_VALUE_GAUSS, d)
        else:
            raise ValueError(rotation)

    # rows of x are vectors ------------------------------------------------
    def rot_key(self, x):
        if self.rotation == "fwht":
            return fwht(x * self.dk) / np.sqrt(self.d)
        return x @ self.pk.T

    def unrot_key(self, y):
        if self.rotation == "fwht":
            return fwht(y) / np.sqrt(self.d) * self.dk
        return y @ self.pk

    def rot_value(self, x):
        if self.rotation == "fwht":
            return fwht(x * self.dv) / np.sqrt(self.d)
        return x @ self.pv.T

    def unrot_value(self, y):
        if self.rotation == "fwht":
            return fwht(y) / np.sqrt(self.d) * self.dv
        return y @ self.pv

    def sketch(self, e):
        """w = S e."""
        if self.rotation == "fwht":
            return fwht(self.ds2 * (fwht(e * self.ds1) / np.sqrt(self.d)))
        return e @ self.g.T

    def sketch_t(self, s):
        """S^T s."""
        if self.rotation == "fwht":
            return self.ds1 * (fwht(self.ds2 * fwht(s)) / np.sqrt(self.d))
        return s @ self.g

    # explicit matrices (tests) --------------------------------------------
    def key_matrix(self):
        return self.rot_key(np.eye(self.d)).T

    def value_matrix(self):
        return self.rot_value(np.eye(self.d)).T

    def sketch_matrix(self):
        return self.sketch(np.eye(self.d)).T
