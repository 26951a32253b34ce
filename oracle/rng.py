"""Counter-based random draws used by the method (oracle side).

The method draws random signs for the Rademacher stage of the structured
transform and Gaussian matrices for the dense rotation and the QJL projection
([Reconstruction] section 5 "Step 2: Random Rotation", section 6 "The 1-Bit QJL
Transform"; [Design Study] "Dense and structured transform comparison": seeded
Rademacher pattern plus FWHT).  The pages fix no generator, only that the seed
identifies the transform ([Design Study] "Paging, lifecycle, and cache
identity").  READING: both sides implement SplitMix64 (Steele, Lea and Flood,
OOPSLA 2014; the 64-bit finaliser of Vigna's public-domain splitmix64.c) in its
counter form, output(k) = mix(seed + (k+1) * golden_gamma), and the Box-Muller
transform (Box and Muller, 1958) for normals.

Stream layout: counter = (role << 48) | index, with the roles below.
"""
import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

ROLE_KEY_SIGNS = 0        # D for the key rotation H_n D
ROLE_SKETCH_SIGNS_1 = 1   # first Rademacher stage of the structured QJL sketch
ROLE_SKETCH_SIGNS_2 = 2   # second Rademacher stage of the structured QJL sketch
ROLE_VALUE_SIGNS = 3      # D for the value rotation
ROLE_KEY_GAUSS = 4        # Gaussian matrix whose QR gives the dense key rotation
ROLE_SKETCH_GAUSS = 5     # i.i.d. N(0,1) QJL projection (dense variant)
ROLE_VALUE_GAUSS = 6      # Gaussian matrix whose QR gives the dense value rotation


def splitmix64(seed, counters) -> np.ndarray:
    """SplitMix64 outputs for an array of counters (uint64, wrapping arithmetic).

    ``seed`` may be an integer or an array that broadcasts against ``counters``.
    """
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.asarray(seed, dtype=np.uint64) + (c + np.uint64(1)) * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def _counters(role: int, n: int) -> np.ndarray:
    return (np.uint64(role) << np.uint64(48)) | np.arange(n, dtype=np.uint64)


def sign_vector(seed: int, role: int, d: int) -> np.ndarray:
    """Rademacher vector of length d (float64, entries +-1).

    Coordinate i takes bit (i % 64) of output word i // 64; a set bit means -1.
    """
    words = splitmix64(seed, _counters(role, (d + 63) // 64))
    i = np.arange(d)
    bits = (words[i // 64] >> (i % 64).astype(np.uint64)) & np.uint64(1)
    return np.where(bits == 1, -1.0, 1.0)


def sign_matrix(seeds, role: int, d: int) -> np.ndarray:
    """Rademacher vectors for many seeds at once: [len(seeds), d] (same rule as sign_vector)."""
    seeds = np.asarray(seeds, dtype=np.uint64)[:, None]
    words = splitmix64(seeds, _counters(role, (d + 63) // 64)[None, :])
    i = np.arange(d)
    bits = (words[:, i // 64] >> (i % 64).astype(np.uint64)) & np.uint64(1)
    return np.where(bits == 1, -1.0, 1.0)


def uniform01(seed: int, role: int, n: int) -> np.ndarray:
    """n doubles in [0, 1): the top 53 bits of each output times 2**-53."""
    return (splitmix64(seed, _counters(role, n)) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def gaussian(seed: int, role: int, rows: int, cols: int) -> np.ndarray:
    """rows x cols i.i.d. N(0,1) in row-major order by Box-Muller.

    Element 2k is r*cos(2 pi u2) and element 2k+1 is r*sin(2 pi u2), with
    u1 = (top53(out(2k)) + 1) * 2**-53 in (0, 1], u2 = top53(out(2k+1)) * 2**-53
    and r = sqrt(-2 ln u1).
    """
    n = rows * cols
    npairs = (n + 1) // 2
    raw = splitmix64(seed, _counters(role, 2 * npairs)) >> np.uint64(11)
    u1 = (raw[0::2].astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = raw[1::2].astype(np.float64) * 2.0 ** -53
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * npairs)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:n].reshape(rows, cols)
