"""Pins of the encode oracle (per-block truncated factorisation) against
facts fixed by the mathematics, not by the oracle itself: brute-force
optimal projections on tiny inputs, matrices of known singular value
decomposition, exact recovery at full and planted rank, and invariances."""
import numpy as np
import pytest

import synth
from oracle import encode as enc


def _rng(seed):
    return np.random.default_rng(seed)


def test_rank1_matches_brute_force_direction_search():
    """d = 2: the best rank-1 approximation projects onto the unit direction
    v(phi) maximising ||X v||; a grid over phi finds it by search."""
    x = _rng(1).standard_normal((9, 2)) * np.array([3.0, 1.0]) + np.array([0.5, -0.2])
    phi = np.linspace(0.0, np.pi, 200001)
    v = np.stack([np.cos(phi), np.sin(phi)], axis=1)            # [n][2]
    err = np.array([np.sum((x - np.outer(x @ vv, vv)) ** 2) for vv in v[::50]])
    k = int(np.argmin(err)) * 50
    lo, hi = max(0, k - 50), min(len(phi), k + 51)
    err_f = [np.sum((x - np.outer(x @ vv, vv)) ** 2) for vv in v[lo:hi]]
    best = lo + int(np.argmin(err_f))
    u, w, s = enc.encode_block(x, 1)
    got = np.sum((x - u @ w) ** 2)
    assert abs(got - err_f[best - lo]) <= 1e-9 * np.sum(x ** 2)
    assert abs(abs(w[0] @ v[best]) - 1.0) < 1e-8


def test_rank2_of_three_columns_matches_brute_force_normal_search():
    """d = 3, r = 2: the best rank-2 approximation removes the component along
    the unit normal n minimising ||X n||; search n over a sphere grid."""
    x = _rng(2).standard_normal((11, 3)) @ np.diag([2.0, 1.3, 0.4])
    th = np.linspace(0, np.pi, 721)
    ph = np.linspace(0, 2 * np.pi, 1441)
    T, P = np.meshgrid(th, ph, indexing="ij")
    n = np.stack([np.sin(T) * np.cos(P), np.sin(T) * np.sin(P), np.cos(T)], axis=-1).reshape(-1, 3)
    resid = np.sum((x @ n.T) ** 2, axis=0)          # ||X n||^2 = error of removing n
    got = np.sum((x - enc.approx(x, 2)) ** 2)
    assert got <= resid.min() + 1e-12                 # never worse than any grid normal
    assert resid.min() - got <= 2e-4 * np.sum(x ** 2)  # and the grid gets within its resolution


@pytest.mark.parametrize("T,d", [(40, 8), (8, 8), (5, 8)])
def test_known_singular_value_decomposition(T, d):
    """X = Q1 diag(sigma) Q2^T with chosen sigma: the oracle returns sigma and,
    at every rank, the known truncation Q1_r diag(sigma_r) Q2_r^T."""
    rng = _rng(3 + T)
    m = min(T, d)
    q1, _ = np.linalg.qr(rng.standard_normal((T, m)))
    q2, _ = np.linalg.qr(rng.standard_normal((d, d)))
    sig = np.array([9.0, 6.5, 4.0, 3.0, 2.2, 1.1, 0.6, 0.25])[:m]
    x = q1 @ np.diag(sig) @ q2[:, :m].T
    s, _ = enc.block_spectrum(x)
    np.testing.assert_allclose(s[:m], sig, rtol=1e-12, atol=1e-12)
    assert np.all(s[m:] == 0)
    for r in range(0, d + 1):
        rr = min(r, m)
        want = q1[:, :rr] @ np.diag(sig[:rr]) @ q2[:, :rr].T
        np.testing.assert_allclose(enc.approx(x, r), want, atol=1e-12)
        # Eckart-Young: the squared error is the sum of the dropped sigma^2
        assert abs(np.sum((x - enc.approx(x, r)) ** 2) - np.sum(sig[rr:] ** 2)) < 1e-10


def test_factor_shapes_orthonormal_rows_and_u_equals_xwt():
    x = _rng(4).standard_normal((30, 16))
    for r in (0, 1, 7, 16):
        u, w, s = enc.encode_block(x, r)
        assert u.shape == (30, r) and w.shape == (r, 16)
        np.testing.assert_allclose(w @ w.T, np.eye(r), atol=1e-12)
        np.testing.assert_allclose(u, x @ w.T, atol=1e-12)
        if r:
            # columns of U are orthogonal with norms sigma (U = U_x diag(s))
            np.testing.assert_allclose(u.T @ u, np.diag(s[:r] ** 2), atol=1e-9)


def test_full_rank_reproduces_block_and_rank_zero_is_empty():
    x = _rng(5).standard_normal((12, 6))
    np.testing.assert_allclose(enc.approx(x, 6), x, atol=1e-12)
    u, w, _ = enc.encode_block(x, 0)
    assert u.shape == (12, 0) and w.shape == (0, 6)
    assert np.all(enc.approx(x, 0) == 0)


def test_empty_block():
    s, vt = enc.block_spectrum(np.zeros((0, 4)))
    assert np.all(s == 0) and np.allclose(vt, np.eye(4))
    u, w, _ = enc.encode_block(np.zeros((0, 4)), 2)
    assert u.shape == (0, 2) and w.shape == (2, 4)


def test_column_permutation_equivariance():
    """Permuting the head dimension permutes the approximation's columns."""
    rng = _rng(6)
    x = rng.standard_normal((25, 10)) @ np.diag(0.7 ** np.arange(10))
    p = rng.permutation(10)
    np.testing.assert_allclose(enc.approx(x[:, p], 4), enc.approx(x, 4)[:, p], atol=1e-12)


def test_planted_context_is_recovered_to_rounding():
    """A block of rank r0 (flat spectrum) stored in bf16: the rank-r0
    approximation leaves only the rounding noise (relative ~2^-9), and the
    spectrum drops by three orders of magnitude after sigma_r0."""
    cfg = synth.get_encode_config("enc_small")
    ctx = synth.make_dense_context(cfg, "planted")
    r0 = cfg.planted_rank
    for b in range(cfg.n_blocks):
        x = ctx.dense_f64(0, b, 1)
        s, _ = enc.block_spectrum(x)
        assert s[r0] < 2e-3 * s[r0 - 1]
        assert np.linalg.norm(x - enc.approx(x, r0)) < 2e-3 * np.linalg.norm(x)


def test_context_helpers_agree_with_block_calls():
    cfg = synth.get_encode_config("enc_small").with_(n_blocks=2, block_tokens=40)
    ctx = synth.make_dense_context(cfg, tokens=[40, 3])
    sp = enc.context_spectra(ctx)
    assert sp.shape == (2, 2, 2, 128)
    ap = enc.context_approx(ctx, np.array([[5, 9], [2, 0]]))
    np.testing.assert_allclose(ap[1][1, 0], enc.approx(ctx.dense_f64(0, 1, 1), 2), atol=1e-12)
    assert np.all(ap[1][0, 1] == 0)                   # r' = 0
    np.testing.assert_allclose(ap[0][1, 1], enc.approx(ctx.dense_f64(1, 0, 1), 9), atol=1e-12)
    np.testing.assert_allclose(sp[0, 1, 1], enc.block_spectrum(ctx.dense_f64(1, 0, 1))[0])
