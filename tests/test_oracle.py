"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to a closed form, a textbook or library routine,
a published known answer (tests/golden/), an invariant of the mathematics, or brute
force on a tiny input, so that a dropped term, a wrong sign, index or block offset,
or a transposed operand in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from conftest import read_golden

U32 = 2.0 ** -24  # fp32 unit roundoff


def hadamard256():
    i = np.arange(256)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0) / 16.0


H = hadamard256()


def rotate_dense(X):
    """fp64 block-diagonal rotation of the last axis (blocks of 256), from the closed form."""
    X = np.asarray(X, dtype=np.float64)
    K = X.shape[-1]
    out = np.empty_like(X)
    for b in range(0, K, 256):
        out[..., b:b + 256] = X[..., b:b + 256] @ H  # H is symmetric
    return out


def e4m3_torch_decode(codes):
    return torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def e4m3_torch_encode(x):
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


# ----------------------------------------------------------------------------- rotation

def test_hadamard_closed_form_is_orthonormal_and_symmetric():
    assert np.array_equal(H @ H.T, np.eye(256))  # entries +-1/16: every product and sum exact
    assert np.array_equal(H, H.T)


def test_fwht_basis_vectors_match_closed_form_exactly():
    for i in range(256):
        e = np.zeros(256, np.float32)
        e[i] = 1.0
        assert np.array_equal(O.fwht256(e).astype(np.float64), H[:, i]), i


def test_fwht_special_vectors():
    ones = np.ones(256, np.float32)
    want = np.zeros(256)
    want[0] = 16.0
    assert np.array_equal(O.fwht256(ones), want)
    alt = np.array([(-1) ** bin(j).count("1") for j in range(256)], np.float32)  # row 255 of 16H
    want = np.zeros(256)
    want[255] = 16.0
    assert np.array_equal(O.fwht256(alt), want)


def test_fwht_round_trip_exact_on_small_integers():
    rng = np.random.default_rng(1)
    for _ in range(20):
        v = rng.integers(-127, 128, 256).astype(np.float32)
        assert np.array_equal(O.fwht256(O.fwht256(v)), v)


def test_fwht_agrees_with_dense_within_rounding_bound():
    x = S.normal(5, 1, 256 * 64).astype(np.float32).reshape(64, 256) * 3
    for row in x:
        got = O.fwht256(row).astype(np.float64)
        want = H @ row.astype(np.float64)
        bound = 8 * U32 * np.abs(row.astype(np.float64)).sum() / 16
        assert np.all(np.abs(got - want) <= bound)
        assert abs(np.linalg.norm(got) - np.linalg.norm(row)) <= 16 * U32 * np.linalg.norm(row) + bound


def test_rotate_rows_is_blockwise_dense_rotation():
    W = S.weights(8, 768, seed=3)
    got = O.rotate_rows(W).astype(np.float64)
    want = rotate_dense(W)
    bound = 8 * U32 * np.abs(W).astype(np.float64).max() * 256 / 16
    assert np.abs(got - want).max() <= bound
    # block alignment: a spike in block 2 only changes block 2
    Z = np.zeros((1, 768), np.float32)
    Z[0, 600] = 1.0
    r = O.rotate_rows(Z)
    assert np.all(r[0, :512] == 0) and np.all(np.abs(r[0, 512:]) == 1 / 16)


def test_rotation_consistency_of_product():
    W = S.weights(16, 512, seed=4).astype(np.float64)
    x = S.activations(3, 512, seed=4, n_outliers=2).astype(np.float64)
    lhs = x @ W.T
    rhs = rotate_dense(x) @ rotate_dense(W).T
    assert np.all(np.abs(lhs - rhs) <= 1e-12 * (np.abs(x) @ np.abs(W).T))


# ----------------------------------------------------------------------------- e4m3

def test_e4m3_decode_all_codes_match_torch_and_spec_points():
    ours = np.array([O.e4m3_decode(c) for c in range(256)])
    ref = e4m3_torch_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    for code, val in read_golden("e4m3fn_points.txt"):
        c = int(code, 16)
        if val == "nan":
            assert math.isnan(O.e4m3_decode(c))
        else:
            assert O.e4m3_decode(c) == float(val)
            assert math.copysign(1, O.e4m3_decode(c)) == math.copysign(1, float(val))


def test_e4m3_encode_matches_torch_rne_on_dense_sweep():
    codes = np.arange(0x7F)
    vals = e4m3_torch_decode(codes)
    mids = (vals[:-1] + vals[1:]) / 2  # exact ties
    pts = [vals, mids]
    for m in mids:
        f = np.float32(m)
        pts.append(np.array([np.nextafter(f, np.float32(-1)), np.nextafter(f, np.float32(2))], np.float64))
    pts.append(S.uniform01(11, 1, 40000))  # [0, 1]: the range of group/row ratios
    pts.append(S.uniform01(11, 2, 20000) * 448.0)
    pts.append(2.0 ** (-12 * S.uniform01(11, 3, 20000)))
    x = np.concatenate(pts).astype(np.float32)
    x = x[(x >= 0) & (x <= 448)]
    ours = np.array([O.e4m3_encode(v) for v in x], np.uint8)
    assert np.array_equal(ours, e4m3_torch_encode(x))
    for c in range(0x7F):  # encode(decode(c)) == c
        assert O.e4m3_encode(O.e4m3_decode(c)) == c


# ----------------------------------------------------------------------------- sampling

def test_splitmix64_known_answers():
    want = [int(r[0], 16) for r in read_golden("splitmix64_seed0.txt")]
    assert [O.splitmix64_at(0, i) for i in range(len(want))] == want


def test_fit_sample_small_takes_all_and_large_draws_uniform_positions():
    v = np.arange(1000, dtype=np.float32)
    assert np.array_equal(np.sort(O.fit_sample(v, 7)), v)
    NK = 3 * (1 << 20) + 17
    v = np.arange(NK, dtype=np.float32)  # value == position (exact below 2^24)
    s = O.fit_sample(v, 42)
    assert s.size == 1 << 20
    for i in (0, 1, 2, 1000, (1 << 20) - 1):
        u = O.splitmix64_at(42, i)
        assert s[i] == float((u * NK) >> 64)
    hist = np.bincount((s.astype(np.int64) * 16) // NK, minlength=16)
    assert np.all(np.abs(hist - (1 << 16)) < 6 * 256)  # ~6 sigma of a binomial count


# ----------------------------------------------------------------------------- Lloyd-Max

def _nearest(s, c):
    return np.argmin(np.abs(s[:, None] - c[None, :]), axis=1)


def test_lloyd_max_fixed_point_conditions():
    s = S.normal(2, 3, 20000).astype(np.float32) ** 3  # skewed, heavy-tailed
    c, n, b = O.lloyd_max16(s)
    assert n < 100, "converged sample expected"
    assert np.all(np.diff(c) > 0)
    ss = np.sort(s.astype(np.float64))
    cell = _nearest(ss, c)
    # midpoint condition: every sample sits in the cell of its nearest level
    assert np.array_equal(np.bincount(cell, minlength=16), np.diff(b))
    # centroid condition: every level is its cell's mean
    for j in range(16):
        mean = math.fsum(ss[cell == j]) / np.sum(cell == j)
        assert abs(c[j] - mean) <= 1e-12 * max(1.0, abs(mean))


def test_lloyd_max_distortion_never_increases():
    s = S.student_t4(9, 1, 50000).astype(np.float32)
    prev = np.inf
    for it in range(0, 25):
        c, n, _ = O.lloyd_max16(s, it)
        d = np.mean((s - c[_nearest(s.astype(np.float64), c)]) ** 2)
        assert d <= prev * (1 + 1e-12)
        prev = d


def test_lloyd_max_recovers_sixteen_distinct_values_exactly():
    levels = np.array([-7, -5, -4, -3, -2, -1.5, -1, -0.5, 0.25, 1, 2, 2.5, 3, 4, 6, 8], np.float32)
    s = np.repeat(levels, 300)
    s = s[np.argsort(S.u64(1, 1, s.size))]  # shuffled
    c, n, b = O.lloyd_max16(s)
    assert np.array_equal(c, levels.astype(np.float64))
    assert n == 1 and np.array_equal(np.diff(b), np.full(16, 300))


def test_lloyd_max_uniform_source_gives_uniform_levels():
    u = (S.uniform01(3, 4, 1 << 20) * 2 - 1).astype(np.float32)
    c, n, _ = O.lloyd_max16(u)
    assert np.abs(c - (-1 + (2 * np.arange(16) + 1) / 16)).max() < 0.01


def _continuous_gauss_lloyd(iters):
    from scipy.stats import norm
    c = norm.ppf((2 * np.arange(16) + 1) / 32)  # the same mid-quantile start
    for _ in range(iters):
        t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
        a, bb = t[:-1], t[1:]
        c = (norm.pdf(a) - norm.pdf(bb)) / (norm.cdf(bb) - norm.cdf(a))  # truncated-normal means
    return c


def test_continuous_gauss_lloyd_reaches_max_1960_table():
    c = _continuous_gauss_lloyd(3000)
    want = np.array([float(r[0]) for r in read_golden("gauss_lloyd_max16.txt")])
    assert np.abs(c[8:] - want).max() < 1.5e-4
    assert np.abs(c[:8] + want[::-1]).max() < 1.5e-4


def test_lloyd_max_gaussian_sample_tracks_continuous_iteration():
    z = S.normal(7, 9, 1 << 20).astype(np.float32)
    c, n, _ = O.lloyd_max16(z)
    ref = _continuous_gauss_lloyd(n)
    assert np.abs(c - ref)[2:-2].max() < 0.006
    assert np.abs(c - ref).max() < 0.02  # the two outer cells hold ~1 % of the sample


# ----------------------------------------------------------------------------- quantize

LEVELS = np.array([-8, -7, -6, -5, -4, -3, -2, -1, 1, 2, 3, 4, 5, 6, 7, 8], np.float64) / 8


def constructed_layer(N=8, K=512, seed=5):
    """A layer exactly representable in the format, and its rotated-back weights."""
    G = K // 16
    r = S.u64(seed, 1, N * G * 17)
    idx = np.empty((N, K), np.int64)
    for gi in range(N * G):
        perm = np.argsort(r[gi * 16:(gi + 1) * 16])
        idx.reshape(-1, 16)[gi] = perm
    codes = np.array([0x38, 0x30, 0x28, 0x20], np.uint8)[(r[N * G * 16:N * G * 17] % 4).astype(int)]
    s_rel = codes.reshape(N, G).copy()
    s_rel[:, 0] = 0x38
    s_ch = np.array([0.5, 0.25] * (N // 2), np.float32)
    w_rot = s_ch[:, None].astype(np.float64) * e4m3_torch_decode(s_rel).repeat(16, axis=1) * LEVELS[idx]
    W = rotate_dense(w_rot)
    assert np.array_equal(rotate_dense(W), w_rot)  # exact dyadic arithmetic
    W32 = W.astype(np.float32)
    assert np.array_equal(W32.astype(np.float64), W)
    packed = (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8).view(np.int8)
    return W32, dict(packed=packed, s_rel=s_rel, s_ch=s_ch, cb=LEVELS.astype(np.float32), idx=idx)


def test_quantize_recovers_a_constructed_layer_exactly():
    W, truth = constructed_layer()
    q = O.quantize_weight(W, seed=0)
    assert np.array_equal(q["cb"], truth["cb"])
    assert np.array_equal(q["s_ch"], truth["s_ch"])
    assert np.array_equal(q["s_rel"], truth["s_rel"])
    assert np.array_equal(q["packed"], truth["packed"])
    assert q["updates"] == 1


def test_quantize_steps_rederived_with_library_routines():
    W = S.weights(64, 512, seed=6)
    q = O.quantize_weight(W, seed=0, want_v=True)
    wr = O.rotate_rows(W)  # pinned above against the dense rotation
    N, K = W.shape
    a = np.abs(wr)
    assert np.array_equal(q["s_ch"], a.max(axis=1))
    gmax = a.reshape(N, K // 16, 16).max(axis=2)
    ratio = (gmax / q["s_ch"][:, None]).astype(np.float32)
    assert np.array_equal(q["s_rel"], e4m3_torch_encode(ratio))
    d = (q["s_ch"][:, None] * e4m3_torch_decode(q["s_rel"]).astype(np.float32)).astype(np.float32)
    v = (wr.reshape(N, K // 16, 16) / d[:, :, None]).astype(np.float32).reshape(N, K)
    assert np.array_equal(v, q["v"])
    idx = np.empty((N, K), np.int64)
    idx[:, 0::2] = q["packed"].view(np.uint8) & 15
    idx[:, 1::2] = q["packed"].view(np.uint8) >> 4
    dist = np.abs(v.astype(np.float64)[:, :, None] - q["cb"].astype(np.float64)[None, None, :])
    chosen = np.take_along_axis(dist, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all(chosen <= dist.min(axis=2))  # nearest level
    c, n, _ = O.lloyd_max16(q["v"].ravel())
    assert np.array_equal(c.astype(np.float32), q["cb"]) and n == q["updates"]


def test_quantize_determinism_seed_and_shape_rule():
    W = S.weights(2048, 768, seed=8)  # N*K > 2^20: the fit samples
    a = O.quantize_weight(W, seed=42)
    b = O.quantize_weight(W, seed=42)
    c = O.quantize_weight(W, seed=43)
    for key in ("packed", "s_rel", "s_ch", "cb"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(a["s_ch"], c["s_ch"]) and np.array_equal(a["s_rel"], c["s_rel"])
    assert not np.array_equal(a["cb"], c["cb"])
    with pytest.raises(ValueError):
        O.quantize_weight(np.zeros((4, 4304), np.float32))  # 4304 = 16 * 269: no 256-blocks


def test_quantize_zero_rows_and_underflowing_groups():
    W = S.weights(4, 256, seed=9)
    W[1] = 0.0
    wr = rotate_dense(W)
    wr[2, 16:32] *= 1e-4  # a group far below 2^-10 of its row maximum
    W = rotate_dense(wr).astype(np.float32)
    q = O.quantize_weight(W, seed=0)
    assert q["s_ch"][1] == 0 and np.all(q["s_rel"][1] == 0)
    assert q["s_rel"][2, 1] == 0
    w_hat = O.dequant(q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    assert np.all(w_hat[1] == 0) and np.all(w_hat[2, 16:32] == 0)


# ----------------------------------------------------------------------------- packing

def test_nibble_order_exhaustive_over_all_bytes():
    packed = np.arange(256, dtype=np.uint8).view(np.int8).reshape(1, 256)  # K = 512
    cb = np.arange(16, dtype=np.float32) * 0.5 - 3.0
    s_rel = np.full((1, 32), 0x38, np.uint8)
    w = O.dequant(packed, s_rel, np.ones(1, np.float32), cb)
    b = np.arange(256)
    assert np.array_equal(w[0, 0::2], cb[b & 15])  # element 2j: low nibble
    assert np.array_equal(w[0, 1::2], cb[b >> 4])


def test_dequant_uses_group_of_sixteen_and_row_scale():
    N, K = 3, 512
    packed = np.full((N, K // 2), 0x11, np.int8)  # every index 1
    s_rel = np.zeros((N, K // 16), np.uint8)
    s_rel[:, 5] = 0x38  # only group 5 (k = 80..95) is non-zero
    s_ch = np.array([1.0, 2.0, -4.0], np.float32)
    cb = np.zeros(16, np.float32)
    cb[1] = 0.75
    w = O.dequant(packed, s_rel, s_ch, cb)
    want = np.zeros((N, K))
    want[:, 80:96] = (s_ch * 0.75)[:, None]
    assert np.array_equal(w, want)


# ----------------------------------------------------------------------------- prepare

def test_prepare_quantisation_bounds():
    x = S.activations(6, 768, seed=12, n_outliers=2)
    x[3] *= 1e-3
    xq, sx = O.prepare(x)
    xr = rotate_dense(x)
    rot_err = 8 * U32 * np.abs(x).astype(np.float64).sum(axis=1) / 16
    amax = np.abs(xr).max(axis=1)
    assert np.all(np.abs(sx - amax / 127) <= (rot_err + U32 * amax) / 127 * 2)
    for m in range(6):
        err = np.abs(xr[m] - sx[m] * xq[m].astype(np.float64))
        assert np.all(err <= sx[m] / 2 * (1 + 4 * U32) + rot_err[m])
        assert np.abs(xq[m]).max() == 127
        assert xq[m][np.argmax(np.abs(xr[m]))] == 127 * np.sign(xr[m][np.argmax(np.abs(xr[m]))])


def test_prepare_ties_round_to_even_and_zero_row():
    xr = np.zeros((2, 256))
    xr[0, :8] = [127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -126.5]
    x = rotate_dense(xr).astype(np.float32)  # exact: dyadic values
    xq, sx = O.prepare(x)
    assert sx[0] == 1.0
    assert list(xq[0, :8]) == [127, 2, 4, -2, 0, 0, 2, -126]
    assert np.all(xq[0, 8:] == 0)
    assert sx[1] == 0 and np.all(xq[1] == 0)


# ----------------------------------------------------------------------------- product

def _layer(N, K, M, seed):
    W = S.weights(N, K, seed=seed)
    x = S.activations(M, K, seed=seed, n_outliers=2)
    q = O.quantize_weight(W, seed=seed)
    xq, sx = O.prepare(x)
    return W, x, q, xq, sx


def test_linear_two_routes_agree():
    W, x, q, xq, sx = _layer(48, 512, 5, 13)
    y, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    w_hat = O.dequant(q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    y2 = (sx.astype(np.float64)[:, None] * xq.astype(np.float64)) @ w_hat.T
    assert np.all(np.abs(y - y2) <= 1e-12 * A)
    A2 = np.abs(sx.astype(np.float64)[:, None] * xq.astype(np.float64)) @ np.abs(w_hat).T
    assert np.allclose(A, A2, rtol=1e-12, atol=0)
    rows, toks = np.array([47, 0, 13]), np.array([4, 1])
    ys, As = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows, toks)
    assert np.array_equal(ys, y[np.ix_(toks, rows)]) and np.array_equal(As, A[np.ix_(toks, rows)])


def test_linear_hand_values():
    K = 256
    packed = np.full((2, K // 2), 0x33, np.int8)  # every index 3
    packed[1, :8] = np.int8(0x5A)  # row 1, k < 16: even k -> 10, odd k -> 5
    s_rel = np.full((2, K // 16), 0x38, np.uint8)  # 1.0
    s_rel[1, 0] = 0x30  # 0.5 for row 1, group 0
    s_ch = np.array([2.0, 1.0], np.float32)
    cb = np.zeros(16, np.float32)
    cb[3], cb[5], cb[10] = 0.5, -1.0, 4.0
    xq = np.ones((1, K), np.int8)
    sx = np.array([0.25], np.float32)
    y, A = O.linear_ref(xq, sx, packed, s_rel, s_ch, cb)
    # row 0: 256 * 0.25 * 2 * 0.5 = 64.  row 1: k<16: 8*(4.0) + 8*(-1.0) at 0.5 -> 12,
    # times 0.25 -> 3; k>=16: 240 * 0.5 * 0.25 = 30; total 33; A: (8*4+8*1)*0.5*0.25 + 30 = 35
    assert y[0, 0] == 64.0 and y[0, 1] == 33.0
    assert A[0, 0] == 64.0 and A[0, 1] == 35.0


def test_linear_i8_partials_exact_and_codebook_properties():
    W, x, q, xq, sx = _layer(32, 512, 3, 14)
    s_cb, cbi8 = O.codebook_i8(q["cb"])
    assert s_cb == np.float32(np.abs(q["cb"]).max()) / np.float32(127)
    assert np.abs(cbi8).max() == 127
    assert np.all(np.abs(cbi8 * np.float64(s_cb) - q["cb"]) <= s_cb / 2 * (1 + 1e-6))
    y8, A8, P = O.linear_i8_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"], want_p=True)
    N, K = 32, 512
    idx = np.empty((N, K), np.int64)
    idx[:, 0::2] = q["packed"].view(np.uint8) & 15
    idx[:, 1::2] = q["packed"].view(np.uint8) >> 4
    wi = cbi8.astype(np.int64)[idx]  # [N, K]
    Pn = np.einsum("mgi,ngi->mng", xq.astype(np.int64).reshape(3, K // 16, 16), wi.reshape(N, K // 16, 16))
    assert np.array_equal(P.astype(np.int64), Pn)
    sg = e4m3_torch_decode(q["s_rel"])  # [N, G]
    y8n = (sx.astype(np.float64)[:, None] * q["s_ch"].astype(np.float64)[None, :] * s_cb
           * np.einsum("mng,ng->mn", Pn.astype(np.float64), sg))
    assert np.all(np.abs(y8 - y8n) <= 1e-12 * A8)


def test_int8_codebook_rounding_term_on_sparse_activations():
    """The int8 route's one approximation beyond fp32 rounding: each codebook level moves to
    the nearest multiple of s_cb, by at most s_cb / 2.  With one non-zero activation per
    token nothing averages that out, so each output's error is exactly the rounding of one
    level times its scales: bounded by s_x * s_ch * |dec(s_rel)| * (s_cb / 2) * |x_q| and
    equal to s_x * s_ch * dec(s_rel) * |cb_i8 * s_cb - cb| * |x_q| up to the fp64 sums.  On
    the seed-0 256 x 512 layer that rounding is far outside the 4e-3 * sum |x w| gate for
    tokens that fall on the smallest levels: the route meets the gate only statistically."""
    N, K = 256, 512
    W = S.weights(N, K, seed=0)
    q = O.quantize_weight(W, seed=0)
    s_cb, cbi8 = O.codebook_i8(q["cb"])
    cb = q["cb"].astype(np.float64)
    lvl_err = np.abs(cbi8.astype(np.float64) * np.float64(s_cb) - cb)
    assert np.all(lvl_err <= s_cb / 2 * (1 + 1e-6))
    # one token per column k, with x_q = 127 there and 0 elsewhere; s_x = 1 / 127
    ks = np.arange(0, K, 7)
    M = ks.size
    xq = np.zeros((M, K), np.int8)
    xq[np.arange(M), ks] = 127
    sx = np.full(M, np.float32(1.0 / 127.0), np.float32)
    y, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    y8, _ = O.linear_i8_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    idx = np.empty((N, K), np.int64)
    idx[:, 0::2] = q["packed"].view(np.uint8) & 15
    idx[:, 1::2] = q["packed"].view(np.uint8) >> 4
    dec = e4m3_torch_decode(q["s_rel"])[:, ks // 16].T                 # [M, N]
    scale = sx.astype(np.float64)[:, None] * q["s_ch"].astype(np.float64)[None, :] * np.abs(dec) * 127
    want = scale * lvl_err[idx[:, ks].T]                                 # the level's rounding
    err = np.abs(y8 - y)
    assert np.all(np.abs(err - want) <= 1e-9 * scale + 1e-300)
    assert np.all(err <= scale * s_cb / 2 * (1 + 1e-6))
    # the gate is A-relative; on the smallest levels the rounding exceeds it many times over
    ratio = err[A > 0] / (4e-3 * A[A > 0])
    smallest = np.argmin(np.abs(cb))
    print(f"one-hot x_q: max |y8 - y| / (4e-3 A) = {ratio.max():.2f}; smallest level {cb[smallest]:.4f} "
          f"moves by {lvl_err[smallest] / abs(cb[smallest]) * 100:.2f}%")
    assert lvl_err[smallest] / abs(cb[smallest]) > 4e-3
    assert ratio.max() > 1.0


def test_linear_i8_abs_sum_with_signed_scales():
    """A8, the bound's scale in the int8 route, is the sum over k of |s_x x_q cb_i8 s_cb
    dec(s_rel) s_ch| term by term, whatever the signs: random layer bytes with every finite
    group-scale code, the negative ones included, against that sum taken directly."""
    N, K, M = 12, 512, 3
    g = np.random.default_rng(4)
    packed = g.integers(-128, 128, size=(N, K // 2), dtype=np.int8)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    s_rel = g.choice(codes, size=(N, K // 16))
    s_ch = (0.01 + 0.02 * g.random(N)).astype(np.float32)
    cb = np.sort(g.standard_normal(16)).astype(np.float32)
    xq = g.integers(-127, 128, size=(M, K), dtype=np.int8)
    sx = (0.01 + g.random(M)).astype(np.float32)
    y8, A8 = O.linear_i8_ref(xq, sx, packed, s_rel, s_ch, cb)
    s_cb, cbi8 = O.codebook_i8(cb)
    idx = np.empty((N, K), np.int64)
    idx[:, 0::2] = packed.view(np.uint8) & 15
    idx[:, 1::2] = packed.view(np.uint8) >> 4
    wsc = (e4m3_torch_decode(s_rel).repeat(16, axis=1) * cbi8.astype(np.float64)[idx]
           * s_ch.astype(np.float64)[:, None] * np.float64(s_cb))       # [N, K]
    terms = sx.astype(np.float64)[:, None, None] * xq.astype(np.float64)[:, None, :] * wsc[None]
    assert np.all(np.abs(A8 - np.abs(terms).sum(-1)) <= 1e-12 * A8)
    assert np.all(np.abs(y8 - terms.sum(-1)) <= 1e-12 * A8)
    assert np.any(np.abs(terms.sum(-1)) < 0.5 * A8)   # signs do cancel in y8


# Integer codebook with max |level| = 127, so s_cb = 1 exactly and the table entries below
# are hand values: t[c][j] = level_j * dec(c) rounded half to even, clamped to +-127.
RQ_CB = np.array([-127, -64, -5, -3, -1, 0, 1, 3, 5, 7, 9, 11, 50, 64, 100, 127], np.float32)
RQ_HAND = {
    0x38: [-127, -64, -5, -3, -1, 0, 1, 3, 5, 7, 9, 11, 50, 64, 100, 127],       # 1.0
    0x30: [-64, -32, -2, -2, 0, 0, 0, 2, 2, 4, 4, 6, 25, 32, 50, 64],             # 0.5
    0x28: [-32, -16, -1, -1, 0, 0, 0, 1, 1, 2, 2, 3, 12, 16, 25, 32],             # 0.25
    0x34: [-95, -48, -4, -2, -1, 0, 1, 2, 4, 5, 7, 8, 38, 48, 75, 95],            # 0.75
    0x40: [-127, -127, -10, -6, -2, 0, 2, 6, 10, 14, 18, 22, 100, 127, 127, 127], # 2.0: clamps
    0xB8: [127, 64, 5, 3, 1, 0, -1, -3, -5, -7, -9, -11, -50, -64, -100, -127],   # -1.0
    0x00: [0] * 16,                                                               # +0
    0x7F: [0] * 16, 0xFF: [0] * 16,                                               # NaN codes
}


def test_rq_table_hand_values_and_rounding_bound():
    t = O.rq_table(RQ_CB)
    for c, want in RQ_HAND.items():
        assert t[c].tolist() == want, hex(c)
    # a fitted codebook: the row of scale 1 is the separately pinned int8 codebook, and every
    # code with |dec| <= 1 rounds each decoded level to the nearest multiple of s_cb
    W, x, q, xq, sx = _layer(32, 512, 3, 14)
    s_cb, cbi8 = O.codebook_i8(q["cb"])
    t = O.rq_table(q["cb"])
    assert np.array_equal(t[0x38], cbi8)
    dec = e4m3_torch_decode(np.arange(256))
    for c in range(256):
        if np.isnan(dec[c]) or abs(dec[c]) > 1:
            continue
        exact = dec[c] * q["cb"].astype(np.float64)
        assert np.abs(t[c]).max() <= 127
        assert np.all(np.abs(t[c] * np.float64(s_cb) - exact) <= s_cb / 2 * (1 + 1e-6) + 1e-12), hex(c)


def test_rq_product_assembly_exact_case_and_error_bound():
    W, x, q, xq, sx = _layer(40, 768, 5, 15)
    N, K, M = 40, 768, 5
    yq = O.linear_rq_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    # assembly: per-weight table lookup (nibble order, group k/16), exact integer matmul,
    # the three fp32 roundings of the epilogue
    t = O.rq_table(q["cb"])
    s_cb, _ = O.codebook_i8(q["cb"])
    idx = np.empty((N, K), np.int64)
    idx[:, 0::2] = q["packed"].view(np.uint8) & 15
    idx[:, 1::2] = q["packed"].view(np.uint8) >> 4
    code = np.repeat(q["s_rel"].astype(np.int64), 16, axis=1)
    wq = t[code, idx].astype(np.int64)
    acc = xq.astype(np.int64) @ wq.T
    sw = q["s_ch"] * np.float32(s_cb)
    ye = (acc.astype(np.float32) * sw[None, :]) * sx[:, None]
    assert ye.dtype == np.float32 and np.array_equal(yq.view(np.uint32), ye.view(np.uint32))
    # against the exact product: the rounding of each weight is at most s_cb / 2 in units of
    # the row scale (every group scale the quantiser writes is at most 1)
    y, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    assert np.all(e4m3_torch_decode(q["s_rel"]) <= 1)
    step = (np.abs(sx.astype(np.float64))[:, None] * q["s_ch"].astype(np.float64)[None, :] * s_cb / 2
            * np.abs(xq.astype(np.float64)).sum(1)[:, None])
    assert np.all(np.abs(yq - y) <= step * (1 + 1e-5) + 8 * U32 * A)
    print(f"rq vs exact: max |dy| / (4e-3 A) = {(np.abs(yq - y) / (4e-3 * A)).max():.4f}")
    # subsets address the same outputs
    rows, toks = np.array([39, 0, 17]), np.array([4, 1])
    ys = O.linear_rq_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows, toks)
    assert np.array_equal(ys, yq[np.ix_(toks, rows)])
    # a codebook on the integer grid with unit group scales: requantisation is exact and the
    # result is the exact product up to the epilogue's roundings
    cbi = np.sort(RQ_CB)
    s1 = np.full_like(q["s_rel"], 0x38)
    yi = O.linear_rq_ref(xq, sx, q["packed"], s1, q["s_ch"], cbi)
    yr, Ar = O.linear_ref(xq, sx, q["packed"], s1, q["s_ch"], cbi)
    assert np.all(np.abs(yi - yr) <= 3 * U32 * np.abs(yr))
    assert np.abs(yr).max() > 0


def test_plausibility_against_unquantised_product():
    W, x, q, xq, sx = _layer(256, 512, 4, 0)
    y, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    ytrue = x.astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(y - ytrue) / np.linalg.norm(ytrue)
    w_hat = O.dequant(q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    wrel = np.linalg.norm(w_hat - rotate_dense(W)) / np.linalg.norm(W)
    print(f"output rel err {rel:.4f}, weight rel RMS {wrel:.4f}")
    assert rel < 0.15 and wrel < 0.15


# ----------------------------------------------------------------------------- W8A8 comparator

def test_w8_quantisation_is_per_row_int8_of_the_rotated_row():
    """Pinned to the separately pinned activation preparation: a weight row quantises exactly
    like a token (same rotation, scale and rounding), and to the rounding bound."""
    W = S.weights(64, 512, seed=21)
    W[3] = 0.0                                             # zero row
    wq, sw = O.quantize_w8(W)
    xq, sx = O.prepare(W)                                  # rows as tokens
    assert np.array_equal(wq, xq) and np.array_equal(sw.view(np.uint32), sx.view(np.uint32))
    assert sw[3] == 0 and not wq[3].any()
    rot = rotate_dense(W)
    for r in range(64):
        if sw[r] == 0:
            continue
        err = np.abs(rot[r] - sw[r] * wq[r].astype(np.float64))
        assert err.max() <= sw[r] * (0.5 + 1e-5)
        assert np.abs(wq[r]).max() == 127


def test_w8_product_equals_integer_matmul():
    W = S.weights(48, 768, seed=22)
    x = S.activations(3, 768, seed=22, n_outliers=2)
    wq, sw = O.quantize_w8(W)
    xq, sx = O.prepare(x)
    y = O.linear_w8_ref(xq, sx, wq, sw)
    dot = xq.astype(np.int64) @ wq.astype(np.int64).T      # exact
    assert np.array_equal(y, sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] * dot)
    # hand value: one row of all-ones weights against a spike
    W1 = np.zeros((1, 256), dtype=np.float32)
    W1[0, 0] = 16.0                                        # rotated row: all entries 1
    x1 = np.zeros((1, 256), dtype=np.float32)
    x1[0, 0] = 16.0                                        # rotated token: all entries 1
    wq1, sw1 = O.quantize_w8(W1)
    xq1, sx1 = O.prepare(x1)
    assert (wq1 == 127).all() and (xq1 == 127).all()
    s32 = float(np.float32(1.0) / np.float32(127.0))        # both scales are the fp32 1/127
    assert sw1[0] == sx1[0] == np.float32(s32)
    assert O.linear_w8_ref(xq1, sx1, wq1, sw1)[0, 0] == s32 * s32 * (127 * 127 * 256)


def test_w8_plausibility_against_unquantised_product():
    W = S.weights(256, 512, seed=23)
    x = S.activations(4, 512, seed=23, n_outliers=2)
    wq, sw = O.quantize_w8(W)
    xq, sx = O.prepare(x)
    y = O.linear_w8_ref(xq, sx, wq, sw)
    ytrue = x.astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(y - ytrue) / np.linalg.norm(ytrue)
    print(f"W8A8 output rel err {rel:.4f}")
    assert rel < 0.05
