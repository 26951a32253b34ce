"""Pins for the oracle's generator, codebook, transforms and byte layout.

Every check here compares the oracle with something other than itself: a
published generator output, a closed form, a textbook table, a library routine
(scipy's Hadamard, numerical quadrature), an invariant, or Monte Carlo.
"""
import json
import os

import numpy as np
import pytest
from scipy import integrate, special, stats
from scipy.linalg import hadamard

from oracle import codebook, layout, rng
from oracle.rotation import Transforms, fwht, haar_orthogonal

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- generator

def test_splitmix64_published_outputs():
    g = _gold("splitmix64.json")
    out = rng.splitmix64(g["seed"], np.arange(len(g["first_outputs_hex"])))
    assert [format(int(v), "016x") for v in out] == g["first_outputs_hex"]


def test_sign_vector_reproducible_and_balanced():
    a = rng.sign_vector(42, rng.ROLE_KEY_SIGNS, 4096)
    b = rng.sign_vector(42, rng.ROLE_KEY_SIGNS, 4096)
    c = rng.sign_vector(42, rng.ROLE_VALUE_SIGNS, 4096)
    assert np.array_equal(a, b)
    assert set(np.unique(a)) == {-1.0, 1.0}
    assert abs(a.mean()) < 4 / np.sqrt(4096)
    assert abs((a * c).mean()) < 4 / np.sqrt(4096)        # different roles are unrelated


def test_box_muller_is_standard_normal():
    z = rng.gaussian(7, rng.ROLE_SKETCH_GAUSS, 400, 500).ravel()
    assert abs(z.mean()) < 5 / np.sqrt(z.size)
    assert abs(z.var() - 1) < 5 * np.sqrt(2 / z.size)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    pairs = z[: z.size // 2 * 2].reshape(-1, 2)
    assert abs(np.corrcoef(pairs.T)[0, 1]) < 5 / np.sqrt(len(pairs))


# ---------------------------------------------------------------- codebook

@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_d3_is_uniform_quantizer(bits):
    # For d = 3 a coordinate of a uniform point on the sphere is uniform on
    # [-1, 1] (Archimedes), whose Lloyd-Max quantizer is the uniform grid.
    L = 1 << bits
    c = codebook.lloyd_max(3, bits)
    assert np.allclose(c, -1 + (2 * np.arange(L) + 1) / L, atol=1e-13)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_codebook_one_bit_closed_form(d):
    # One bit: the centroid is E[X | X > 0] = 2 int_0^1 x f_d = 2 / ((d-1) B(1/2, (d-1)/2)).
    c = codebook.lloyd_max(d, 1)
    exact = 2.0 / ((d - 1) * special.beta(0.5, (d - 1) / 2.0))
    assert np.allclose(c, [-exact, exact], rtol=1e-13)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_gaussian_limit_matches_max_table(bits):
    g = _gold("gaussian_lloyd_max.json")
    d = 1 << 16
    c = codebook.lloyd_max(d, bits) * np.sqrt(d)
    pos = c[len(c) // 2:]
    assert np.allclose(pos, g["positive_centroids"][str(bits)], atol=2.5e-4)
    D = codebook.distortion(codebook.lloyd_max(d, bits), d)
    assert abs(D - g["mse"][str(bits)]) < 1e-3 * g["mse"][str(bits)] + 6e-5


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (256, 4), (64, 2)])
def test_codebook_centroid_and_nearest_neighbour_conditions(d, bits):
    # Independent of the incomplete-beta path: adaptive quadrature of the pdf.
    c = codebook.lloyd_max(d, bits)
    t = codebook.thresholds(c)
    edges = np.concatenate(([-1.0], t, [1.0]))
    f = lambda x: codebook.marginal_pdf(x, d)
    for j in range(len(c)):
        m, _ = integrate.quad(f, edges[j], edges[j + 1], epsabs=1e-14, epsrel=1e-12, limit=200)
        mx, _ = integrate.quad(lambda x: x * f(x), edges[j], edges[j + 1], epsabs=1e-15, epsrel=1e-12, limit=200)
        assert abs(mx / m - c[j]) < 1e-9
    assert np.allclose(c, -c[::-1], atol=1e-15)
    y = np.random.default_rng(0).normal(0, 1 / np.sqrt(d), 20000)
    idx = np.searchsorted(t, y, side="left")
    assert np.array_equal(idx, np.argmin(np.abs(y[:, None] - c[None, :]), axis=1))


def test_codebook_total_mass_and_second_moment():
    for d in (3, 64, 128, 256):
        assert abs(codebook.marginal_cdf(1.0, d) - 1) < 1e-14
        m2 = codebook.cell_second_moments(np.array([-1.0, 1.0]), d)[0]
        assert abs(m2 - 1.0 / d) < 1e-14                   # E[X^2] = 1/d on the sphere


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (256, 2)])
def test_codebook_distortion_monte_carlo(d, bits):
    c = codebook.lloyd_max(d, bits)
    t = codebook.thresholds(c)
    g = np.random.default_rng(1).standard_normal((20000, d))
    u = g / np.linalg.norm(g, axis=1, keepdims=True)        # uniform on the sphere
    err = ((u - c[np.searchsorted(t, u, side="left")]) ** 2).sum(1)
    mc, se = err.mean(), err.std() / np.sqrt(len(err))
    assert abs(mc - codebook.distortion(c, d)) < 5 * se


def test_theorem1_bound_and_printed_ratios():
    # [README] "Paper Validation": Thm 1 holds for unit vectors and the
    # distortion tracks 1/4^b.  The bound's constant is an image on the page;
    # READING: sqrt(3) pi / 2.  2- and 3-bit ratios agree with the printed
    # 0.70x / 0.82x within 0.03; the printed 0.97x at 4 bits does not follow
    # from this constant (documented contradiction) and is only bounded.
    g = _gold("readme_validation.json")["thm1_bound_ratio_printed"]
    const = np.sqrt(3) * np.pi / 2
    for bits in (1, 2, 3, 4):
        D = codebook.distortion(codebook.lloyd_max(128, bits), 128)
        ratio = D / (const / 4 ** bits)
        assert ratio < 1.0
        if str(bits) in ("2", "3"):
            Dg = codebook.distortion(codebook.lloyd_max(1 << 16, bits), 1 << 16)
            assert abs(Dg / (const / 4 ** bits) - g[str(bits)]) < 0.03


def test_value_cosine_matches_readme_2bit():
    # E cos(v, v~) -> sqrt(1 - D_b(d)) (centroid condition: <y, yhat> = ||yhat||^2 on
    # average); the README measures 0.940 for 2-bit values at head_dim 256.
    d = 256
    g = _gold("readme_validation.json")
    c = codebook.lloyd_max(d, 2)
    closed = np.sqrt(1 - codebook.distortion(c, d))
    assert abs(closed - g["value_cos_2bit_head_dim256"]) < 1.5e-3
    T = Transforms(d, "fwht", 3)
    x = np.random.default_rng(2).standard_normal((4000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = T.rot_value(u)
    vt = T.unrot_value(c[np.searchsorted(codebook.thresholds(c), y, side="left")])
    cos = (u * vt).sum(1) / np.linalg.norm(vt, axis=1)
    assert abs(cos.mean() - closed) < 2e-3


# ---------------------------------------------------------------- transforms

@pytest.mark.parametrize("d", [2, 16, 128, 256])
def test_fwht_is_sylvester_hadamard(d):
    x = np.random.default_rng(d).standard_normal((7, d))
    assert np.allclose(fwht(x), x @ hadamard(d).T, atol=1e-12)


@pytest.mark.parametrize("rot,d", [("fwht", 128), ("fwht", 256), ("dense", 128), ("dense", 64)])
def test_rotations_orthogonal_and_invertible(rot, d):
    T = Transforms(d, rot, 11)
    for M in (T.key_matrix(), T.value_matrix()):
        assert np.abs(M @ M.T - np.eye(d)).max() < 1e-12
    x = np.random.default_rng(3).standard_normal((5, d))
    assert np.allclose(T.unrot_key(T.rot_key(x)), x, atol=1e-12)
    assert np.allclose(T.unrot_value(T.rot_value(x)), x, atol=1e-12)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    assert np.allclose(np.linalg.norm(T.rot_key(u), axis=1), 1.0, atol=1e-13)


@pytest.mark.parametrize("d", [128, 256])
def test_fwht_spreads_basis_vector(d):
    # [Reconstruction] section 13 golden vector: the canonical basis vector is
    # spread to magnitude 1/sqrt(d) in every coordinate.
    T = Transforms(d, "fwht", 5)
    y = T.rot_key(np.eye(d)[:1])[0]
    assert np.allclose(np.abs(y), 1 / np.sqrt(d), atol=1e-15)


def test_dense_rotation_is_the_positive_diagonal_qr_factor():
    # Q R = A with R upper triangular and diag(R) > 0 determines Q uniquely.
    d = 64
    A = rng.gaussian(9, rng.ROLE_KEY_GAUSS, d, d)
    Q = haar_orthogonal(9, rng.ROLE_KEY_GAUSS, d)
    R = Q.T @ A
    assert np.abs(np.tril(R, -1)).max() < 1e-12
    assert (np.diag(R) > 0).all()


def test_dense_rotation_coordinates_have_variance_one_over_d():
    d = 32
    u = np.ones(d) / np.sqrt(d)
    ys = np.stack([Transforms(d, "dense", s).rot_key(u[None])[0] for s in range(600)])
    assert abs((ys ** 2).mean() - 1 / d) < 4 * np.sqrt(2 / (600 * d)) / d * 3


@pytest.mark.parametrize("rot,d", [("fwht", 128), ("dense", 128)])
def test_sketch_transpose_and_row_norms(rot, d):
    T = Transforms(d, rot, 13)
    S = T.sketch_matrix()
    a, b = np.random.default_rng(4).standard_normal((2, 3, d))
    assert np.allclose((T.sketch(a) * b).sum(1), (a * T.sketch_t(b)).sum(1), atol=1e-9)
    if rot == "fwht":
        assert np.abs(S @ S.T - d * np.eye(d)).max() < 1e-10
    else:
        assert abs(np.diag(S @ S.T).mean() / d - 1) < 0.05


# ---------------------------------------------------------------- layout

def _fmt(d, key_bits, value_bits, **kw):
    from oracle import tq
    return tq.Config(d, 8, 2, key_bits, value_bits, **kw)


def test_record_sizes_match_storage_formula():
    for case in _gold("storage_formula.json")["cases"]:
        P = 16
        f = _fmt(case["d"], case["key_bits"], case["value_bits"])
        kb = layout.key_block_bytes(f, P)
        vb = layout.value_block_bytes(f, P)
        assert kb == P * case["key_record_bytes"]
        assert vb == P * case["value_record_bytes"]
        assert kb % 16 == 0 and vb % 16 == 0


def test_extended_record_sizes_match_the_bit_accounting():
    for case in _gold("extended_formats.json")["cases"]:
        f = _fmt(case["d"], case["key_bits"], case["value_bits"], key_mode=case["key_mode"],
                 key_bits_hi=case["key_bits_hi"], value_bits_hi=case["value_bits_hi"],
                 value_mode=case["value_mode"], key_outliers=case["key_outliers"])
        assert layout.key_block_bytes(f) == 16 * case["key_record_bytes"], case["_what"]
        assert layout.value_block_bytes(f) == 16 * case["value_record_bytes"], case["_what"]


@pytest.mark.parametrize("d,kb,vb,kw", [(128, 3, 2, {}), (128, 4, 4, {}), (256, 3, 2, {}), (256, 4, 3, {}),
                                        (128, 3, 2, dict(key_bits_hi=4, value_bits_hi=3)),
                                        (64, 2, 1, dict(key_bits_hi=4, value_bits_hi=4, key_outliers=3)),
                                        (128, 3, 2, dict(key_mode="scaled_unbiased", key_outliers=4,
                                                         value_mode="group")),
                                        (256, 2, 4, dict(key_mode="scaled_mse", key_bits_hi=3, value_mode="group",
                                                         value_bits_hi=2, key_outliers=8))])
def test_pack_unpack_roundtrip(d, kb, vb, kw):
    from oracle import tq
    f = _fmt(d, kb, vb, **kw)
    g = np.random.default_rng(d + kb)
    shape = (3, 2, 16, d)
    kbits = f.key_bits_of(d)
    codes = g.integers(0, 1 << kbits, shape)
    z = g.integers(0, 2, shape).astype(bool) & f.qjl
    nu = g.random((3, 2, 16)).astype(np.float32)
    gam = g.random((3, 2, 16)).astype(np.float32)
    k = f.key_outliers
    sidx = g.integers(0, d, (3, 2, 16, k)).astype(np.uint8)
    sval = g.standard_normal((3, 2, 16, k)).astype(np.float16)
    scnt = g.integers(0, k + 1, (3, 2, 16)).astype(np.uint8)
    buf = layout.pack_key_block(f, codes, z, nu, gam, sidx, sval, scnt)
    assert buf.shape[-1] == layout.key_block_bytes(f)
    c2, z2, n2, g2, si2, sv2, sc2 = layout.unpack_key_block(f, buf)
    assert np.array_equal(c2, codes) and np.array_equal(z2, z)
    assert np.array_equal(n2, nu) and np.array_equal(g2, gam)
    assert np.array_equal(si2, sidx) and np.array_equal(sv2.view(np.uint16), sval.view(np.uint16))
    assert np.array_equal(sc2, scnt)
    vcodes = g.integers(0, 1 << f.value_bits_of(d), shape)
    vs = g.random((3, 2, 16, d // 32)).astype(np.float16)
    vz = g.standard_normal((3, 2, 16, d // 32)).astype(np.float16)
    vbuf = layout.pack_value_block(f, vcodes, nu, vs, vz)
    assert vbuf.shape[-1] == layout.value_block_bytes(f)
    vc2, vn2, vs2, vz2 = layout.unpack_value_block(f, vbuf)
    assert np.array_equal(vc2, vcodes)
    if f.value_mode == "group":
        assert np.array_equal(vs2, vs) and np.array_equal(vz2, vz)
    else:
        assert np.array_equal(vn2, nu)


def test_layout_bit_positions_by_hand():
    d, m = 128, 2
    f = _fmt(d, m + 1, 2)
    codes = np.zeros((16, d), int)
    z = np.zeros((16, d), bool)
    codes[3, 37] = 2          # plane 1, token 3, coordinate 37 = group 1 bit 5
    z[5, 100] = True          # QJL plane (2), token 5, coordinate 100 = group 3 bit 4
    buf = layout.pack_key_block(f, codes, z, np.zeros(16), np.zeros(16))
    words_per_token = (d // 32) * (m + 1)
    w1 = 3 * words_per_token + 1 * (m + 1) + 1
    w2 = 5 * words_per_token + 3 * (m + 1) + 2
    assert list(np.flatnonzero(buf)) == [4 * w1, 4 * w2]
    assert buf[4 * w1] == 1 << 5 and buf[4 * w2] == 1 << 4
    nu = np.arange(16, dtype=np.float32)
    gam = -np.arange(16, dtype=np.float32)
    buf = layout.pack_key_block(f, codes, z, nu, gam)
    pairs = buf[16 * words_per_token * 4:].view("<f4").reshape(16, 2)
    assert np.array_equal(pairs[:, 0], nu) and np.array_equal(pairs[:, 1], gam)
    vcodes = np.zeros((16, d), int)
    vcodes[9, 70] = 3         # both planes, slot 9, coordinate 70 = low half of pair 35
    vcodes[2, 71] = 1         # plane 0, slot 2, coordinate 71 = high half of pair 35
    vbuf = layout.pack_value_block(f, vcodes, np.zeros(16))
    words = vbuf[:d * 2 * 2].view("<u4").reshape(d // 2, 2)
    assert words[35, 0] == (1 << 9) | (1 << (16 + 2)) and words[35, 1] == 1 << 9
    assert np.count_nonzero(words) == 2


def test_extended_layout_positions_by_hand():
    """Mixed rates, scaled keys, sidecar and group scales at hand-computed offsets."""
    d = 128
    f = _fmt(d, 3, 2, key_mode="scaled_unbiased", key_bits_hi=4, value_bits_hi=3, key_outliers=2)
    # key planes per group: 3, 3 (lower half), 4, 4 (upper half), no QJL plane -> 14 words per token
    codes = np.zeros((16, d), int)
    codes[1, 70] = 8          # plane 3 of group 2 (coordinate 70 = group 2 bit 6)
    sidx = np.zeros((16, 2), np.uint8)
    sval = np.zeros((16, 2), np.float16)
    scnt = np.zeros(16, np.uint8)
    scnt[4], sidx[4, 1], sval[4, 1] = 2, 99, np.float16(-2.5)
    buf = layout.pack_key_block(f, codes, np.zeros((16, d), bool), np.zeros(16), np.zeros(16), sidx, sval, scnt)
    w = 1 * 14 + (3 + 3) + 3
    assert list(np.flatnonzero(buf[:16 * 14 * 4])) == [4 * w] and buf[4 * w] == 1 << 6
    side = buf[16 * 14 * 4 + 16 * 8:]
    assert len(side) == 16 * 8                 # count + 2 indices (+ pad) + 2 fp16 = 7 -> 8 bytes per token
    rec = side[4 * 8:5 * 8]
    assert rec[0] == 2 and rec[1] == 0 and rec[2] == 99
    assert rec[4:8].view("<f2")[1] == np.float16(-2.5)
    # values: pairs 0..31 carry 2 planes, pairs 32..63 carry 3
    vcodes = np.zeros((16, d), int)
    vcodes[7, 65] = 4         # plane 2 of pair 32 (its first pair), odd coordinate, slot 7
    vbuf = layout.pack_value_block(f, vcodes, np.zeros(16))
    words = vbuf[:4 * (32 * 2 + 32 * 3)].view("<u4")
    assert list(np.flatnonzero(words)) == [32 * 2 + 2] and words[32 * 2 + 2] == 1 << (16 + 7)
    g = _fmt(d, 3, 2, value_mode="group")
    vbuf = layout.pack_value_block(g, np.zeros((16, d), int), None,
                                   np.full((16, 4), 0.5, np.float16), np.full((16, 4), -1.0, np.float16))
    tail = vbuf[4 * 64 * 2:].view("<f2").reshape(16, 4, 2)
    assert np.all(tail[..., 0] == 0.5) and np.all(tail[..., 1] == -1.0)
