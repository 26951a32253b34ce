"""Lloyd-Max codebook for one coordinate of a uniformly random unit vector.

[Reconstruction] section 5, "Step 2: Random Rotation": after a random rotation
each coordinate of a unit vector follows a scaled Beta law on [-1, 1]; "Step 3"
notes it tends to N(0, 1/d); "Step 4: Lloyd-Max Boundaries and Centroids": the
boundaries and centroids are computed offline by continuous k-means on that
density, with centroids dense near zero.  [README] "How It Works": Lloyd-Max
scalar quantisation on the Beta-distributed rotated values.

READING: the exact finite-d marginal is used (not the Gaussian limit):

    f_d(x) = (1 - x^2)^((d-3)/2) / B(1/2, (d-1)/2),  x in [-1, 1],

i.e. (1+x)/2 ~ Beta((d-1)/2, (d-1)/2).  Cell masses come from the regularised
incomplete beta function and cell first moments from the closed-form
antiderivative of x f_d(x):

    int x f_d(x) dx = -(1 - x^2)^((d-1)/2) / ((d-1) B(1/2, (d-1)/2)).

Thresholds are midpoints of adjacent centroids (nearest-centroid rule,
[Reconstruction] "Step 5: Code Assignment").
"""
import numpy as np
from scipy import special


def marginal_pdf(x, d: int):
    x = np.asarray(x, dtype=np.float64)
    return (1.0 - x * x) ** ((d - 3) / 2.0) / special.beta(0.5, (d - 1) / 2.0)


def marginal_cdf(x, d: int):
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    a = (d - 1) / 2.0
    return special.betainc(a, a, (1.0 + x) / 2.0)


def marginal_moment_antiderivative(x, d: int):
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    return -((1.0 - x * x) ** ((d - 1) / 2.0)) / ((d - 1) * special.beta(0.5, (d - 1) / 2.0))


def _cells(edges, d):
    mass = np.diff(marginal_cdf(edges, d))
    mom = np.diff(marginal_moment_antiderivative(edges, d))
    return mass, mom


def lloyd_max(d: int, bits: int, rtol: float = 1e-13, max_iter: int = 20000):
    """Ascending Lloyd-Max centroids (float64) for 2**bits levels at dimension d.

    Lloyd iteration (centroid <- conditional mean of its cell, boundary <-
    midpoint) until the largest centroid move is below rtol * max|c|.
    """
    L = 1 << bits
    if L == 1:
        return np.zeros(1)      # no code bits: the single centroid is the mean, 0
    a = (d - 1) / 2.0
    # start from equal-mass cells
    q = special.betaincinv(a, a, np.arange(1, L) / L) * 2.0 - 1.0
    edges = np.concatenate(([-1.0], q, [1.0]))
    mass, mom = _cells(edges, d)
    c = mom / mass
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        mass, mom = _cells(edges, d)
        cn = mom / mass
        cn = 0.5 * (cn - cn[::-1])          # the density is even: keep the codebook odd
        delta = np.max(np.abs(cn - c))
        c = cn
        if delta < rtol * np.max(np.abs(c)):
            break
    return c


def thresholds(c):
    """Decision boundaries between adjacent centroids (midpoints)."""
    c = np.asarray(c, dtype=np.float64)
    return 0.5 * (c[:-1] + c[1:])


def distortion(c, d: int) -> float:
    """D_b(d) = d * E[(Y - Q(Y))^2] for Y ~ f_d under nearest-centroid coding.

    Computed cell by cell as d * sum_j int_cell (x - c_j)^2 f_d(x) dx with the
    cell moments of ``cell_second_moments`` and ``_cells``.
    """
    c = np.asarray(c, dtype=np.float64)
    edges = np.concatenate(([-1.0], thresholds(c), [1.0]))
    mass, mom = _cells(edges, d)
    m2 = cell_second_moments(edges, d)
    per_cell = m2 - 2.0 * c * mom + c * c * mass
    return float(d * per_cell.sum())


def cell_second_moments(edges, d: int):
    """int_{e_j}^{e_{j+1}} x^2 f_d(x) dx for each cell.

    Integrating x * (x f_d) by parts with M_d the antiderivative of x f_d:
    int x^2 f_d = [x M_d(x)] - int M_d, and -int M_d(x) dx =
    B(1/2, (d+1)/2) / ((d-1) B(1/2, (d-1)/2)) * F_{d+2}(x) = F_{d+2}(x) / d,
    where F_{d+2} is the marginal CDF at dimension d + 2, whose density is
    proportional to (1 - x^2)^((d-1)/2).
    """
    e = np.clip(np.asarray(edges, dtype=np.float64), -1.0, 1.0)
    cum = e * marginal_moment_antiderivative(e, d) + marginal_cdf(e, d + 2) / d
    return np.diff(cum)
