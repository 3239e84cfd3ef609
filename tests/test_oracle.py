"""Pins for the CPU oracle: each test checks it against something other than itself.

Sources: "Kronecker Product" (Definition, Why It Matters, Implementation Notes);
"FlatQuant: Fast Learnable Affine Quantization" (Symbol Map, Kronecker factorization,
Learning the affine transformation, Per-channel scaling and learnable clipping);
"Quantifying Incoherence in the QuIP Method" (orthogonal factors and their inverse);
"High-Rate Quantized Matrix Multiplication I" (absmax INT, high-rate noise model).
"""
import math
import os

import numpy as np
import pytest

from oracle import kq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------------------------------
# Kronecker product
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("sa,sb", [((2, 2), (2, 3)), ((3, 5), (4, 2)), ((1, 4), (3, 1)), ((4, 4), (4, 4))])
def test_kron_definition_matches_numpy_kron(sa, sb):
    A, B = _rand(sa, 1), _rand(sb, 2)
    K = O.kron_by_definition(A, B)
    assert K.shape == (sa[0] * sb[0], sa[1] * sb[1])
    assert np.array_equal(K, np.kron(A, B))


def test_kron_block_form_golden():
    """The page's 2x2 (x) 2x3 block-form example, expanded entry by entry."""
    rows = []
    with open(os.path.join(GOLDEN, "kron_block_2x2_2x3.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    assert len(rows) == 4 and all(len(r) == 6 for r in rows)
    A, B = _rand((2, 2), 3), _rand((2, 3), 4)
    G = np.empty((4, 6))
    for r, row in enumerate(rows):
        for col, tok in enumerate(row):
            a, b = tok.split("*")
            G[r, col] = A[int(a[1]) - 1, int(a[2]) - 1] * B[int(b[1]) - 1, int(b[2]) - 1]
    assert np.array_equal(O.kron_by_definition(A, B), G)
    assert np.array_equal(O.kron_library(A, B), G)


# ------------------------------------------------------------------------------------
# The transform
# ------------------------------------------------------------------------------------
FACTORS = [(2, 3), (3, 5), (8, 8), (4, 16), (16, 4), (2, 32), (12, 20)]


@pytest.mark.parametrize("n1,n2", FACTORS)
@pytest.mark.parametrize("with_c", [False, True])
def test_factored_equals_dense(n1, n2, with_c):
    """x (P1 (x) P2) (dense, library kron) == vec_r(P1^T V P2) (factored)."""
    rng = np.random.default_rng(n1 * 100 + n2)
    T = 5
    X = rng.standard_normal((T, n1 * n2))
    P1 = rng.standard_normal((n1, n1))          # deliberately non-symmetric
    P2 = rng.standard_normal((n2, n2))
    c = rng.uniform(0.5, 2.0, n1 * n2).astype(np.float32) if with_c else None
    Yd = O.transform_dense(X, P1, P2, c)
    Yf = O.transform(X, P1, P2, c)
    rel = np.linalg.norm(Yd - Yf) / np.linalg.norm(Yd)
    assert rel <= 1e-12


def test_one_hot_token_gives_outer_product_of_factor_rows():
    """x = e_(i*n2+k)  =>  Y[j, l] = P1[i, j] * P2[k, l]  (row i*n2+k of P1 (x) P2)."""
    n1, n2 = 3, 5
    rng = np.random.default_rng(7)
    P1, P2 = rng.standard_normal((n1, n1)), rng.standard_normal((n2, n2))
    for i in range(n1):
        for k in range(n2):
            x = np.zeros((1, n1 * n2))
            x[0, i * n2 + k] = 1.0
            Y = O.transform(x, P1, P2).reshape(n1, n2)
            for j in range(n1):
                for l in range(n2):
                    assert Y[j, l] == P1[i, j] * P2[k, l]


def test_identity_factors_are_exact():
    rng = np.random.default_rng(8)
    n1, n2 = 4, 6
    X = rng.standard_normal((3, n1 * n2))
    c = rng.uniform(0.5, 2, n1 * n2).astype(np.float32)
    assert np.array_equal(O.transform(X, np.eye(n1), np.eye(n2)), X)
    assert np.array_equal(O.transform(X, np.eye(n1), np.eye(n2), c), X * c.astype(np.float64))


def test_signed_permutation_factors_move_entries():
    """P1[i, s1(i)] = e1(i), P2[k, s2(k)] = e2(k)  =>  Y[s1(i), s2(k)] = e1(i) e2(k) V[i, k]."""
    rng = np.random.default_rng(9)
    n1, n2 = 5, 7
    s1, s2 = rng.permutation(n1), rng.permutation(n2)
    e1, e2 = rng.choice([-1.0, 1.0], n1), rng.choice([-1.0, 1.0], n2)
    P1 = np.zeros((n1, n1)); P1[np.arange(n1), s1] = e1
    P2 = np.zeros((n2, n2)); P2[np.arange(n2), s2] = e2
    X = rng.standard_normal((2, n1 * n2))
    Y = O.transform(X, P1, P2)
    for t in range(2):
        for i in range(n1):
            for k in range(n2):
                assert Y[t, s1[i] * n2 + s2[k]] == e1[i] * e2[k] * X[t, i * n2 + k]


def test_bf16_decoding_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x3F00, 0x0080, 0x7F7F, 0x0000, 0x8000, 0x4049], np.uint16)
    want = [1.0, -2.0, 0.5, 2.0 ** -126, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0, 3.140625]
    got = O.bf16_bits_to_f64(pats)
    for g, w in zip(got, want):
        assert g == w


def test_bf16_and_fp64_inputs_agree():
    rng = np.random.default_rng(10)
    n1, n2 = 4, 8
    f = rng.standard_normal((3, n1 * n2)).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)     # truncation: exact bf16 values
    exact = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    p1 = (rng.standard_normal((n1, n1)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    p2 = (rng.standard_normal((n2, n2)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Yb = O.transform(bits, p1, p2, dtype="bf16")
    Y64 = O.transform(exact, O.bf16_bits_to_f64(p1), O.bf16_bits_to_f64(p2))
    assert np.array_equal(Yb, Y64)


def _haar(n, rng):
    Q, R = np.linalg.qr(rng.standard_normal((n, n)))
    return Q * np.sign(np.diag(R))[None, :]


@pytest.mark.parametrize("n1,n2", [(8, 8), (4, 16), (16, 8)])
def test_orthogonal_factors_preserve_token_norms(n1, n2):
    rng = np.random.default_rng(11)
    P1, P2 = _haar(n1, rng), _haar(n2, rng)
    X = rng.standard_normal((6, n1 * n2)) * rng.uniform(0.1, 10, (6, 1))
    Y = O.transform(X, P1, P2)
    r = np.linalg.norm(Y, axis=1) / np.linalg.norm(X, axis=1)
    assert np.max(np.abs(r - 1)) <= 1e-12


@pytest.mark.parametrize("kind", ["orthogonal", "near_identity"])
def test_inverse_recovers_input(kind):
    rng = np.random.default_rng(12)
    n1, n2 = 6, 10
    if kind == "orthogonal":
        P1, P2 = _haar(n1, rng), _haar(n2, rng)
    else:
        P1 = np.eye(n1) + 0.1 * rng.standard_normal((n1, n1)) / math.sqrt(n1)
        P2 = np.eye(n2) + 0.1 * rng.standard_normal((n2, n2)) / math.sqrt(n2)
    c = rng.uniform(0.25, 4, n1 * n2).astype(np.float32)
    X = rng.standard_normal((4, n1 * n2))
    Xr = O.inverse_transform(O.transform(X, P1, P2, c), P1, P2, c)
    assert np.max(np.abs(Xr - X)) <= 1e-10 * np.max(np.abs(X))
    if kind == "orthogonal":  # the inverse is the transpose: transform with P1^T... no:
        # (P1 (x) P2)^{-1} = P1^T (x) P2^T for orthogonal factors
        Xt = O.transform(O.transform(X, P1, P2), P1.T, P2.T)
        assert np.max(np.abs(Xt - X)) <= 1e-12 * np.max(np.abs(X))


def test_weight_side_cancels_transform():
    """(X P)(P^{-1} W^T) = X W^T with P = P1 (x) P2 and P^{-1} = P1^{-1} (x) P2^{-1}."""
    rng = np.random.default_rng(13)
    n1, n2, m = 4, 8, 6
    P1 = np.eye(n1) + 0.3 * rng.standard_normal((n1, n1))
    P2 = np.eye(n2) + 0.3 * rng.standard_normal((n2, n2))
    X = rng.standard_normal((5, n1 * n2))
    W = rng.standard_normal((m, n1 * n2))
    XP = O.transform(X, P1, P2)
    # rows of W P^{-T} = W (P1^{-T} (x) P2^{-T})
    WPinvT = O.transform(W, np.linalg.inv(P1).T, np.linalg.inv(P2).T)
    got = XP @ WPinvT.T
    want = X @ W.T
    assert np.max(np.abs(got - want)) <= 1e-10 * np.max(np.abs(want))


# ------------------------------------------------------------------------------------
# Quantizer
# ------------------------------------------------------------------------------------
def test_clip_ratio_special_values():
    assert O.clip_ratio(math.inf) == np.float32(1.0)
    assert O.clip_ratio(-math.inf) == np.float32(0.0)
    assert O.clip_ratio(0.0) == np.float32(0.5)
    assert O.clip_ratio(math.log(3.0)) == np.float32(0.75)      # 1 / (1 + 1/3)
    assert O.clip_ratio(-math.log(3.0)) == np.float32(0.25)
    for a in (0.3, 2.0, 3.0, 7.5):
        assert abs(float(O.clip_ratio(a)) + float(O.clip_ratio(-a)) - 1.0) <= 2 ** -24
    assert abs(float(O.clip_ratio(2.0)) - 0.8807970779778823) <= 2 ** -24
    with pytest.raises(ValueError):
        O.clip_ratio(float("nan"))


def test_integer_token_with_absmax_7_is_reproduced_exactly():
    y = np.array([[7, -3, 0, 1, -7, 2, 5, -6]], np.float32)
    q, s = O.quantize_per_token(y, 1.0)
    assert s[0] == 1.0 and s.dtype == np.float16
    assert np.array_equal(q, y.astype(np.int8))


def test_ties_round_to_even():
    y = np.array([[7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 4.5, -3.5]], np.float32)
    q, s = O.quantize_per_token(y, 1.0)
    assert s[0] == 1.0
    assert q[0].tolist() == [7, 0, 2, 2, 0, -2, -2, 4, 4, -4]


def test_fp16_scale_rounding_ties_to_even():
    # s32 = 1 + 2^-11 sits halfway between fp16 1.0 and 1 + 2^-10: even mantissa wins (1.0)
    y = np.array([[7 * (1 + 2 ** -11), 1.0], [7 * (1 + 3 * 2 ** -11), 1.0]], np.float32)
    _, s = O.quantize_per_token(y, 1.0)
    assert s[0] == np.float16(1.0)
    assert s[1] == np.float16(1 + 2 ** -9)
    _, s32 = O.quantize_per_token(y, 1.0, scale_dtype="fp32")
    assert s32[0] == np.float32(1 + 2 ** -11) and s32.dtype == np.float32


def _torch_quint4x2_bytes(y, scale):
    torch = pytest.importorskip("torch")
    t = torch.quantize_per_tensor(torch.from_numpy(np.ascontiguousarray(y)), float(scale), 8, torch.quint4x2)
    return t.int_repr().numpy()


@pytest.mark.parametrize("k", [-3, 0, 2, 9])
@pytest.mark.parametrize("alpha", [math.inf, 0.0])
def test_power_of_two_scales_match_library_int4_quantizer(k, alpha):
    """With absmax = 7*2^k the scale is exactly clip*2^k, so the whole quantizer (RNE,
    clamp, nibble packing) must agree with PyTorch's per-tensor quint4x2 quantizer
    (offset-binary nibbles with zero point 8, element 2m in the low nibble)."""
    rng = np.random.default_rng(100 + k)
    T, n = 6, 64
    y = rng.uniform(-1, 1, (T, n)) * 7 * 2.0 ** k
    y[np.arange(T), rng.integers(0, n, T)] = 7 * 2.0 ** k * rng.choice([-1, 1], T)
    # a few exact ties at the quantization midpoints
    clip = float(O.clip_ratio(alpha))
    step = clip * 2.0 ** k
    y[:, 1] = (np.arange(T) - 2.5) * step
    y = y.astype(np.float32)
    q, s = O.quantize_per_token(y, O.clip_ratio(alpha))
    assert np.all(s.astype(np.float64) == step)
    codes = O.pack_int4(q)
    for t in range(T):
        ref = _torch_quint4x2_bytes(y[t], step) ^ np.uint8(0x88)
        assert np.array_equal(codes[t], ref), t


def test_quantization_error_bound_and_range():
    rng = np.random.default_rng(14)
    y = (rng.standard_t(3, (64, 512)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    for alpha in (math.inf, 3.0, 2.0, 1.0):
        clip = O.clip_ratio(alpha)
        q, s = O.quantize_per_token(y, clip)
        assert q.min() >= -8 and q.max() <= 7
        sf = s.astype(np.float64)[:, None]
        r = y.astype(np.float64) / sf
        inside = np.abs(r) <= 7.0
        err = np.abs(y - q * sf)
        assert np.all(err[inside] <= 0.5 * sf.repeat(y.shape[1], 1)[inside] * (1 + 2 ** -20))
        # saturated entries keep their sign at the extreme codes
        assert np.all(q[r > 7.5] == 7) and np.all(q[r < -8.5] == -8)
        if alpha == math.inf:
            am = np.argmax(np.abs(y), axis=1)
            assert np.all(np.abs(q[np.arange(64), am]) == 7)


def test_monotone_within_token():
    rng = np.random.default_rng(15)
    y = rng.standard_normal((8, 256)).astype(np.float32)
    q, _ = O.quantize_per_token(y, O.clip_ratio(1.5))
    for t in range(8):
        o = np.argsort(y[t], kind="stable")
        assert np.all(np.diff(q[t][o].astype(int)) >= 0)


def test_zero_and_degenerate_tokens():
    y = np.zeros((3, 16), np.float32)
    y[1, 3] = 5.0
    q, s = O.quantize_per_token(y, 1.0)
    assert s[0] == 0 and np.all(q[0] == 0) and s[2] == 0
    assert q[1, 3] == 7
    q, s = O.quantize_per_token(y, O.clip_ratio(-math.inf))       # clip 0: scale 0
    assert np.all(s == 0) and np.all(q == 0)


def test_fp32_step_whose_reciprocal_overflows_is_an_underflow():
    """Reading R9: with fp32 steps, a token whose step s = fp32(a / 7) is at most 2^-128
    (fp32(1 / s) = inf) is stored with step 0 and all-zero codes, like a zero token; a step
    just above that range still quantizes normally and keeps the half-step error bound."""
    y = np.zeros((4, 8), np.float32)
    y[0, :3] = [1e-38, 3e-39, 0.0]                                # s32 = 1.43e-39
    y[1, :2] = [7 * np.float32(2.0 ** -128), np.float32(2.0 ** -128)]  # s32 = 2^-128
    y[2, :2] = [7 * np.float32(2.0 ** -127), -np.float32(2.0 ** -126)]  # s32 = 2^-127
    y[3, :2] = [np.float32(2.0 ** -120), -np.float32(2.0 ** -121)]      # s32 ~ 1.1e-37
    q, s = O.quantize_per_token(y, 1.0, "fp32")
    for t in (0, 1):
        assert s[t] == 0 and np.all(q[t] == 0)
    assert s[2] == np.float32(2.0 ** -127) and q[2, 0] == 7 and q[2, 1] == -2
    assert s[3] > 0 and q[3, 0] == 7 and q[3, 1] in (-3, -4)
    for t in (2, 3):
        err = np.abs(y[t].astype(np.float64) - q[t] * np.float64(s[t]))
        assert np.all(err <= np.float64(s[t]) / 2)
    # fp16 steps never reach that range: the same tokens give step 0 by fp16 underflow
    q16, s16 = O.quantize_per_token(y, 1.0, "fp16")
    assert np.all(s16 == 0) and np.all(q16 == 0)


def test_pack_nibble_order_and_roundtrip():
    assert O.pack_int4(np.array([[1, -1]])).tolist() == [[0xF1]]
    assert O.pack_int4(np.array([[-8, 7]])).tolist() == [[0x78]]
    assert O.pack_int4(np.array([[7, -8]])).tolist() == [[0x87]]
    assert O.pack_int4(np.array([[-1, -1, 0, 0]])).tolist() == [[0xFF, 0x00]]
    rng = np.random.default_rng(16)
    q = rng.integers(-8, 8, (5, 64)).astype(np.int8)
    assert np.array_equal(O.unpack_int4(O.pack_int4(q)), q)
    with pytest.raises(ValueError):
        O.pack_int4(np.array([[8, 0]]))


def test_high_rate_noise_model():
    """Unclipped per-token RTN error on Gaussian tokens is close to uniform: E[e^2] ~ s^2/12."""
    rng = np.random.default_rng(17)
    y = rng.standard_normal((512, 4096)).astype(np.float32)
    q, s = O.quantize_per_token(y, 1.0)
    sf = s.astype(np.float64)[:, None]
    e2 = ((y - q * sf) / sf) ** 2
    assert abs(e2.mean() - 1 / 12) <= 0.05 / 12


def test_absmax_penalty_drops_after_random_orthogonal_kronecker_transform():
    """absmax-INT distortion factor a^2 n / |y|^2 is large for outlier-laden tokens and
    drops towards ~2 ln n after a random orthogonal Kronecker transform."""
    rng = np.random.default_rng(18)
    n1, n2 = 16, 32
    n = n1 * n2
    X = rng.standard_normal((64, n))
    X[:, [5, 77]] *= 40
    P1, P2 = _haar(n1, rng), _haar(n2, rng)
    Y = O.transform(X, P1, P2)
    d = lambda Z: np.median(np.max(np.abs(Z), 1) ** 2 * n / np.sum(Z ** 2, 1))
    assert d(X) > 100
    assert d(Y) < 4 * math.log(n)


def test_full_path_identity_factors_match_library_quantizer():
    """P1 = I, P2 = I: the whole pipeline is per-token absmax RTN of x, checked against
    the library quantizer on tokens whose absmax is 7 * 2^k."""
    rng = np.random.default_rng(19)
    n1, n2, T = 4, 8, 5
    X = rng.uniform(-1, 1, (T, n1 * n2)) * 7 * 2.0 ** np.arange(T)[:, None]
    X[:, 0] = 7 * 2.0 ** np.arange(T)
    X = X.astype(np.float32)
    Y, codes, s = O.transform_quant(X, np.eye(n1, dtype=np.float32), np.eye(n2, dtype=np.float32),
                                    None, math.inf, "fp32")
    assert np.array_equal(Y, X.astype(np.float64))
    for t in range(T):
        assert np.array_equal(codes[t], _torch_quint4x2_bytes(X[t], 2.0 ** t) ^ np.uint8(0x88))


# ---- weight side and the INT4 consumer ------------------------------------------------
def _rand_codes(rng, rows, k):
    return O.pack_int4(rng.integers(-8, 8, size=(rows, k)).astype(np.int8))


def test_int4_gemm_matches_dequantized_float_product():
    """The integer route equals dequantize-then-multiply (library float64 matmul) up to
    the two fp32 roundings of the epilogue."""
    rng = np.random.default_rng(11)
    cx, cw = _rand_codes(rng, 7, 96), _rand_codes(rng, 9, 96)
    sx = rng.uniform(0.01, 2, 7).astype(np.float16)
    sw = rng.uniform(0.01, 2, 9).astype(np.float16)
    out = O.int4_gemm(cx, sx, cw, sw)
    ref = O.dequantize(cx, sx) @ O.dequantize(cw, sw).T
    assert out.dtype == np.float32
    np.testing.assert_allclose(out, ref, rtol=2.5e-7, atol=0)


def test_int4_gemm_unit_scales_give_the_integer_product():
    rng = np.random.default_rng(12)
    qx = rng.integers(-8, 8, size=(5, 64))
    qw = rng.integers(-8, 8, size=(3, 64))
    out = O.int4_gemm(O.pack_int4(qx.astype(np.int8)), np.ones(5, np.float16),
                      O.pack_int4(qw.astype(np.int8)), np.ones(3, np.float16))
    # an independent sum: element by element in Python integers
    for t in range(5):
        for j in range(3):
            assert out[t, j] == float(sum(int(a) * int(b) for a, b in zip(qx[t], qw[j])))


def test_int4_gemm_bf16_output_rounds_like_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    cx, cw = _rand_codes(rng, 6, 64), _rand_codes(rng, 8, 64)
    sx = rng.uniform(0.001, 3, 6).astype(np.float32)
    sw = rng.uniform(0.001, 3, 8).astype(np.float32)
    f32 = O.int4_gemm(cx, sx, cw, sw, "fp32")
    bits = O.int4_gemm(cx, sx, cw, sw, "bf16")
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(O.int4_gemm(cx, sx, cw, sw, "fp16"), f32.astype(np.float16))


def test_weight_side_factors_reproduce_the_layer_product():
    """(X P)(P^-1 W^T) = X W^T with non-symmetric, non-orthogonal factors: a transposed or
    non-inverted factor fails this."""
    rng = np.random.default_rng(14)
    n1, n2 = 3, 5
    P1 = np.eye(n1) + 0.3 * rng.standard_normal((n1, n1))
    P2 = np.eye(n2) + 0.3 * rng.standard_normal((n2, n2))
    X = rng.standard_normal((4, n1 * n2))
    W = rng.standard_normal((6, n1 * n2))
    Q1, Q2 = O.weight_factors(P1, P2)
    XP = O.transform(X, P1, P2)
    WPinvT = O.transform(W, Q1, Q2)
    np.testing.assert_allclose(XP @ WPinvT.T, X @ W.T, rtol=1e-10, atol=1e-10)
    # with the dense Kronecker product written out: W P^-T
    Pd = O.kron_library(P1, P2)
    np.testing.assert_allclose(WPinvT, W @ np.linalg.inv(Pd).T, rtol=1e-10, atol=1e-10)


def test_orthogonal_kronecker_transform_lowers_int4_gemm_error_on_outliers():
    """End to end on the CPU: Q(X P) Q(P^-1 W^T) approximates X W^T better than Q(X) Q(W^T)
    when X has outlier channels ("FlatQuant" page, The flatness target)."""
    rng = np.random.default_rng(15)
    n1, n2, T, N = 16, 32, 64, 48
    n = n1 * n2
    X = rng.standard_normal((T, n))
    X[:, rng.choice(n, 6, replace=False)] *= 40.0
    W = rng.standard_normal((N, n)) / np.sqrt(n)

    def qmm(Xt, Wt):
        qx, sx = O.quantize_per_token(Xt.astype(np.float32), np.float32(1.0), "fp32")
        qw, sw = O.quantize_per_token(Wt.astype(np.float32), np.float32(1.0), "fp32")
        return O.int4_gemm(O.pack_int4(qx), sx, O.pack_int4(qw), sw).astype(np.float64)

    def orth(m):
        q, r = np.linalg.qr(rng.standard_normal((m, m)))
        return q * np.sign(np.diag(r))

    P1, P2 = orth(n1), orth(n2)
    ref = X @ W.T
    rel = lambda Y: np.linalg.norm(Y - ref) / np.linalg.norm(ref)
    Q1, Q2 = O.weight_factors(P1, P2)
    XP, WP = O.transform(X, P1, P2), O.transform(W, Q1, Q2)
    # both sides quantized (the INT4 GEMM): about 0.26 -> 0.21 here
    err_plain, err_rot = rel(qmm(X, W)), rel(qmm(XP, WP))
    assert err_rot < 0.85 * err_plain, (err_rot, err_plain)

    # activation side alone (float weights): about 0.23 -> 0.17
    def qdq(A):
        q, s = O.quantize_per_token(A.astype(np.float32), np.float32(1.0), "fp32")
        return O.dequantize(O.pack_int4(q), s)

    assert rel(qdq(XP) @ WP.T) < 0.8 * rel(qdq(X) @ W.T)


# ---- INT8 codes ----------------------------------------------------------------------
@pytest.mark.parametrize("k", [-3, 0, 2])
def test_int8_power_of_two_scales_match_library_qint8_quantizer(k):
    """With absmax = 127*2^k and clip 1 the step is exactly 2^k, so the INT8 quantizer
    (RNE, clamp) must agree with PyTorch's per-tensor qint8 quantizer, ties included."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(200 + k)
    T, n = 5, 96
    step = 2.0 ** k
    y = rng.uniform(-1, 1, (T, n)) * 127 * step
    y[np.arange(T), rng.integers(0, n, T)] = 127 * step * rng.choice([-1, 1], T)
    y[:, 1] = (np.arange(T) * 11 - 20.5) * step   # exact midpoints
    y = y.astype(np.float32)
    q, s = O.quantize_per_token(y, np.float32(1.0), "fp32", bits=8)
    assert np.all(s == np.float32(step))
    for t in range(T):
        ref = torch.quantize_per_tensor(torch.from_numpy(y[t]), step, 0, torch.qint8).int_repr().numpy()
        assert np.array_equal(q[t], ref), t
    assert np.array_equal(O.pack_int8(q).view(np.int8), q)


def test_int8_integer_tokens_and_error_bound():
    rng = np.random.default_rng(201)
    # integer tokens with absmax 127 and clip 1: step 1, codes = the integers
    yi = rng.integers(-127, 128, size=(4, 64)).astype(np.float32)
    yi[:, 0] = 127.0
    q, s = O.quantize_per_token(yi, np.float32(1.0), "fp16", bits=8)
    assert np.all(s == np.float16(1.0)) and np.array_equal(q, yi.astype(np.int8))
    # error bound inside the clip range, range of the codes
    y = rng.standard_normal((50, 256)).astype(np.float32) * rng.uniform(0.1, 10, (50, 1)).astype(np.float32)
    clip = np.float32(0.9)
    q, s = O.quantize_per_token(y, clip, "fp32", bits=8)
    assert q.min() >= -128 and q.max() <= 127
    sf = s.astype(np.float64)[:, None]
    inside = np.abs(y) <= 0.9 * np.abs(y).max(axis=1, keepdims=True)
    err = np.abs(y.astype(np.float64) - q * sf)
    assert np.all(err[inside] <= sf.repeat(256, 1)[inside] / 2 * (1 + 2 ** -20))
    with pytest.raises(ValueError):
        O.quantize_per_token(y, clip, "fp32", bits=3)
