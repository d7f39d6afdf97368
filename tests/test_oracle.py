"""Pins for the fp64 oracle (CPU only).

The pages print no worked numbers, so the oracle is pinned to things other
than itself: hand-derived fixtures (tests/golden), closed forms (linear
attention at zero decay, Toeplitz decay at constant a), special cases, brute
force of the dual quadratic form, invariants (linearity, chunk-size
invariance, split-sequence composition) and cross-formulation agreement.
Each test names the mistake it is there to catch.
"""
import numpy as np
import pytest

import oracle
import ssd_inputs as si
from parity import read_golden, state_err, y_err


def rand_case(rng, Bz=2, L=37, H=4, P=3, N=5, G=2, a_scale=1.0):
    X = rng.standard_normal((Bz, L, H, P))
    B = rng.standard_normal((Bz, L, G, N))
    C = rng.standard_normal((Bz, L, G, N))
    a = -a_scale * rng.uniform(0.0, 1.5, size=(Bz, L, H))
    return X, a, B, C


def golden_inputs(g):
    Bz, L, H, P, N, G = [int(v) for v in g["shape"]]
    X = g["X"].reshape(Bz, L, H, P)
    a = np.log(g["a_exp"]).reshape(Bz, L, H)
    B = g["B"].reshape(Bz, L, G, N)
    C = g["C"].reshape(Bz, L, G, N)
    return (Bz, L, H, P, N, G), X, a, B, C


@pytest.mark.parametrize("name", ["scalar_halving.txt", "orientation_p2_n3.txt"])
def test_golden_fixtures(name):
    # catches: transposed state, B/C swapped, a_t applied to the current
    # input, output read from the pre-update state
    g = read_golden(name)
    (Bz, L, H, P, N, G), X, a, B, C = golden_inputs(g)
    Y, S = oracle.fwd(X, a, B, C)
    np.testing.assert_allclose(Y.ravel(), g["Y"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S.ravel(), g["S_fin"], rtol=0, atol=1e-14)
    for Q in (1, 2, 3):
        out = oracle.chunked_fwd(X, a, B, C, Q)
        np.testing.assert_allclose(out["Y"].ravel(), g["Y"], atol=1e-14)
        np.testing.assert_allclose(out["S_fin"].ravel(), g["S_fin"], atol=1e-14)
    Yq = oracle.quadratic(X, a, B, C)
    np.testing.assert_allclose(Yq.ravel(), g["Y"], atol=1e-14)


def test_golden_decode_step():
    g = read_golden("decode_step.txt")
    Bz, L, H, P, N, G = [int(v) for v in g["shape"]]
    S, y = oracle.step(g["state"].reshape(Bz, H, P, N), g["X"].reshape(Bz, H, P),
                       np.log(g["a_exp"]).reshape(Bz, H), g["B"].reshape(Bz, G, N),
                       g["C"].reshape(Bz, G, N))
    np.testing.assert_allclose(y.ravel(), g["Y"], atol=1e-14)
    np.testing.assert_allclose(S.ravel(), g["S_fin"], atol=1e-14)


@pytest.mark.parametrize("seed,G", [(0, 1), (1, 2), (2, 4)])
def test_recurrence_matches_quadratic_bruteforce(seed, G):
    # the SSM <-> masked-attention duality: any dropped term, wrong index or
    # group mapping in either formulation breaks agreement
    rng = np.random.default_rng(seed)
    X, a, B, C = rand_case(rng, Bz=2, L=41, H=4, P=3, N=6, G=G)
    Y, _ = oracle.fwd(X, a, B, C)
    Yq = oracle.quadratic(X, a, B, C)
    assert y_err(Y, Yq) < 1e-12


def test_tiny_fp32_workload_matches_quadratic():
    d = si.make_fwd(si.FWD_CONFIGS["tiny_f32"])
    X, a, B, C = (si.widen(d[k], "f32") for k in ("X", "a", "B", "C"))
    Y, _ = oracle.fwd(X, a, B, C)
    Yq = oracle.quadratic(X, a, B, C)
    assert y_err(Y, Yq) < 1e-12


def test_zero_decay_is_causal_linear_attention():
    # a = 0: the mask is all-ones below the diagonal, so Y = tril(C B^T) X
    # (linear attention, the wiki review's "Transformers are RNNs" origin)
    rng = np.random.default_rng(3)
    X, a, B, C = rand_case(rng, Bz=1, L=29, H=2, P=4, N=3, G=1)
    a[:] = 0.0
    Y, S = oracle.fwd(X, a, B, C)
    for h in range(2):
        ref = np.tril(C[0, :, 0] @ B[0, :, 0].T) @ X[0, :, h]
        np.testing.assert_allclose(Y[0, :, h], ref, rtol=1e-12, atol=1e-12)
        # final state = sum_t x_t (x) B_t
        np.testing.assert_allclose(S[0, h], X[0, :, h].T @ B[0, :, 0], rtol=1e-12, atol=1e-12)


def test_constant_decay_toeplitz_closed_form():
    # a = ln(gamma): L[t, s] = gamma^(t-s).  Catches a sign error on a and an
    # off-by-one in which step's a decays what.
    rng = np.random.default_rng(4)
    X, a, B, C = rand_case(rng, Bz=1, L=23, H=1, P=2, N=4, G=1)
    gamma = 0.8
    a[:] = np.log(gamma)
    Y, S = oracle.fwd(X, a, B, C)
    t = np.arange(23)
    Lm = np.where(t[:, None] >= t[None, :], gamma ** (t[:, None] - t[None, :]).astype(float), 0.0)
    ref = (Lm * (C[0, :, 0] @ B[0, :, 0].T)) @ X[0, :, 0]
    np.testing.assert_allclose(Y[0, :, 0], ref, rtol=1e-12, atol=1e-12)
    w = gamma ** (22 - t).astype(float)
    np.testing.assert_allclose(S[0, 0], (w[:, None] * X[0, :, 0]).T @ B[0, :, 0], rtol=1e-12)


def test_zero_B_gives_zero():
    rng = np.random.default_rng(5)
    X, a, B, C = rand_case(rng)
    B[:] = 0.0
    Y, S = oracle.fwd(X, a, B, C)
    assert not Y.any() and not S.any()
    out = oracle.chunked_fwd(X, a, B, C, 8)
    assert not out["Y"].any() and not out["S_fin"].any()


def test_strong_decay_keeps_only_the_diagonal():
    # a = -1e4: exp underflows to 0, so y_t = (C_t . B_t) x_t
    rng = np.random.default_rng(6)
    X, a, B, C = rand_case(rng, G=1)
    a[:] = -1e4
    Y, _ = oracle.fwd(X, a, B, C)
    ref = np.einsum("bln,bln->bl", C[:, :, 0], B[:, :, 0])[:, :, None, None] * X
    np.testing.assert_allclose(Y, ref, rtol=1e-13, atol=1e-13)


def test_single_step_ignores_a0():
    rng = np.random.default_rng(7)
    X, a, B, C = rand_case(rng, L=1, G=1)
    Y1, _ = oracle.fwd(X, a, B, C)
    a2 = a - 3.0
    Y2, _ = oracle.fwd(X, a2, B, C)
    np.testing.assert_array_equal(Y1, Y2)
    ref = np.einsum("bn,bn->b", C[:, 0, 0], B[:, 0, 0])[:, None, None] * X[:, 0]
    np.testing.assert_allclose(Y1[:, 0], ref, rtol=1e-13)


def test_linearity_in_X_and_initial_state():
    rng = np.random.default_rng(8)
    X1, a, B, C = rand_case(rng)
    X2 = rng.standard_normal(X1.shape)
    S0 = rng.standard_normal((2, 4, 3, 5))
    Y1, F1 = oracle.fwd(X1, a, B, C)
    Y2, F2 = oracle.fwd(X2, a, B, C)
    Y12, F12 = oracle.fwd(2.0 * X1 - 0.5 * X2, a, B, C)
    np.testing.assert_allclose(Y12, 2.0 * Y1 - 0.5 * Y2, rtol=1e-11, atol=1e-11)
    # the initial state enters linearly: response to S0 alone plus response to X
    Ys, Fs = oracle.fwd(np.zeros_like(X1), a, B, C, S0=S0)
    Yb, Fb = oracle.fwd(X1, a, B, C, S0=S0)
    np.testing.assert_allclose(Yb, Y1 + Ys, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Fb, F1 + Fs, rtol=1e-11, atol=1e-11)


def test_initial_state_response_closed_form():
    # with X = 0, S_t = exp(a_0 + ... + a_t) S0, so y_t = exp(cumsum) S0 C_t
    rng = np.random.default_rng(9)
    X, a, B, C = rand_case(rng, Bz=1, L=11, H=1, P=2, N=3, G=1)
    X[:] = 0.0
    S0 = rng.standard_normal((1, 1, 2, 3))
    Y, S = oracle.fwd(X, a, B, C, S0=S0)
    dec = np.exp(np.cumsum(a[0, :, 0]))
    ref = dec[:, None] * (C[0, :, 0] @ S0[0, 0].T)
    np.testing.assert_allclose(Y[0, :, 0], ref, rtol=1e-12)
    np.testing.assert_allclose(S[0, 0], dec[-1] * S0[0, 0], rtol=1e-12)


@pytest.mark.parametrize("Q", [1, 7, 16, 64, 256])
def test_chunked_form_equals_recurrence(Q):
    # chunk-size invariance, ragged last chunk whenever Q does not divide L
    rng = np.random.default_rng(10 + Q)
    X, a, B, C = rand_case(rng, Bz=2, L=150, H=2, P=3, N=4, G=1, a_scale=3.0)
    S0 = rng.standard_normal((2, 2, 3, 4))
    Y, S = oracle.fwd(X, a, B, C, S0=S0)
    out = oracle.chunked_fwd(X, a, B, C, Q, S0=S0)
    assert y_err(out["Y"], Y) < 1e-12
    assert state_err(out["S_fin"], S) < 1e-12
    np.testing.assert_allclose(out["Ydiag"] + out["Yoff"], out["Y"], rtol=1e-14, atol=1e-14)


def test_chunked_intermediates_are_consistent():
    # cs is the in-chunk inclusive prefix sum; S_in chains through dS and lam;
    # S_in of chunk c equals the recurrence's state at the chunk boundary
    rng = np.random.default_rng(11)
    X, a, B, C = rand_case(rng, Bz=1, L=40, H=1, P=2, N=3, G=1)
    Q = 16
    out = oracle.chunked_fwd(X, a, B, C, Q)
    nc = 3
    for c in range(nc):
        seg = a[0, c * Q:(c + 1) * Q, 0]
        np.testing.assert_allclose(out["cs"][0, 0, c, :len(seg)], np.cumsum(seg), rtol=1e-13)
        assert out["lam"][0, 0, c] == pytest.approx(seg.sum(), rel=1e-13)
        _, Sc = oracle.fwd(X[:, :c * Q], a[:, :c * Q], B[:, :c * Q], C[:, :c * Q]) if c else (None, np.zeros((1, 1, 2, 3)))
        np.testing.assert_allclose(out["S_in"][0, c, 0], Sc[0, 0], rtol=1e-12, atol=1e-14)
        if c + 1 < nc:
            nxt = np.exp(out["lam"][0, 0, c]) * out["S_in"][0, c, 0] + out["dS"][0, c, 0]
            np.testing.assert_allclose(out["S_in"][0, c + 1, 0], nxt, rtol=1e-12, atol=1e-14)
    # with a zero state entering, Yoff is 0 on the first chunk
    assert not out["Yoff"][0, :Q].any()


def test_split_sequence_composes_through_the_state():
    # running the first half, then the second half from its final state,
    # equals one pass: the constant-memory hand-off
    rng = np.random.default_rng(12)
    X, a, B, C = rand_case(rng, Bz=2, L=60, H=2, P=3, N=4, G=1)
    Y, S = oracle.fwd(X, a, B, C)
    Y1, S1 = oracle.fwd(X[:, :25], a[:, :25], B[:, :25], C[:, :25])
    Y2, S2 = oracle.fwd(X[:, 25:], a[:, 25:], B[:, 25:], C[:, 25:], S0=S1)
    np.testing.assert_allclose(np.concatenate([Y1, Y2], axis=1), Y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


def test_step_chain_equals_forward():
    rng = np.random.default_rng(13)
    X, a, B, C = rand_case(rng, Bz=2, L=17, H=4, P=3, N=5, G=2)
    S0 = rng.standard_normal((2, 4, 3, 5))
    Y, S = oracle.fwd(X, a, B, C, S0=S0)
    st = S0
    for t in range(17):
        st, y = oracle.step(st, X[:, t], a[:, t], B[:, t], C[:, t])
        np.testing.assert_allclose(y, Y[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, S, rtol=1e-12, atol=1e-12)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(14)
    X, a, B, C = rand_case(rng, Bz=3, L=33, H=4, P=3, N=5, G=2)
    Y1, S1 = oracle.fwd(X, a, B, C, nthreads=1)
    Y4, S4 = oracle.fwd(X, a, B, C, nthreads=4)
    np.testing.assert_array_equal(Y1, Y4)
    np.testing.assert_array_equal(S1, S4)


def test_bf16_rounding_helpers():
    # round-to-nearest-even at the bf16 boundary, exact widening
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, 65504.0], np.float32)
    bits = si.f32_to_bf16_bits(vals)
    back = si.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0, 65536.0], np.float32))
    # widening then rounding is the identity
    rng = np.random.default_rng(0)
    u = si.f32_to_bf16_bits(rng.standard_normal(1000).astype(np.float32))
    np.testing.assert_array_equal(si.f32_to_bf16_bits(si.bf16_bits_to_f32(u)), u)


def test_input_recipes_ranges():
    d = si.make_fwd(si.FwdShape(2, 300, 8, 4, 4, 1, 64, "f32", dt_recipe="mamba2_dt"))
    a = d["a"]
    assert a.dtype == np.float32 and (a <= -1e-3 * 1.0 + 1e-9).all() and (a >= -1.6 - 1e-6).all()
    d2 = si.make_fwd(si.FwdShape(2, 300, 8, 4, 4, 1, 64, "bf16"))
    assert d2["X"].dtype == np.uint16 and (d2["a"] < 0).all()
    # same seed, same draws
    d3 = si.make_fwd(si.FwdShape(2, 300, 8, 4, 4, 1, 64, "bf16"))
    np.testing.assert_array_equal(d2["X"], d3["X"])


# ---- gradients: the adjoint of the recurrence ---------------------------------

def _loss(X, a, B, C, S0, dY, dS):
    Y, S = oracle.fwd(X, a, B, C, S0=S0)
    return float(np.sum(dY * Y) + np.sum(dS * S))


@pytest.mark.parametrize("G", [1, 2])
def test_gradients_match_central_differences(G):
    # every gradient against central differences of the forward oracle on a
    # tiny case with an initial state and a final-state gradient; catches a
    # dropped adjoint term, a decay applied at the wrong step, a missing
    # group sum for dB/dC or a transposed contraction
    rng = np.random.default_rng(40 + G)
    Bz, L, H, P, N = 1, 9, 2, 3, 4
    X, a, B, C = rand_case(rng, Bz, L, H, P, N, G)
    S0 = rng.standard_normal((Bz, H, P, N))
    dY = rng.standard_normal((Bz, L, H, P))
    dS = rng.standard_normal((Bz, H, P, N))
    gr = oracle.bwd(X, a, B, C, dY, S0=S0, dS_fin=dS)
    args = {"X": X, "a": a, "B": B, "C": C, "S0": S0}
    eps = 1e-6
    for name, arr in args.items():
        num = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = _loss(args["X"], args["a"], args["B"], args["C"], args["S0"], dY, dS)
            arr[idx] = keep - eps
            lm = _loss(args["X"], args["a"], args["B"], args["C"], args["S0"], dY, dS)
            arr[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        got = gr["d" + name]
        scale = np.max(np.abs(num))
        assert np.max(np.abs(got - num)) <= 1e-7 * scale, name


def test_dX_is_the_transposed_quadratic_form():
    # dX = M^T dY with M = Lmask o (C B^T) per slice (the brute-force dual
    # form, built independently of the recurrence); zero initial state and no
    # final-state gradient
    rng = np.random.default_rng(7)
    X, a, B, C = rand_case(rng, Bz=2, L=23, H=4, P=3, N=5, G=2)
    dY = rng.standard_normal(X.shape)
    gr = oracle.bwd(X, a, B, C, dY)
    Bz, L, H, P = X.shape
    G = B.shape[2]
    for b in range(Bz):
        for h in range(H):
            g = h * G // H
            M = oracle.decay_mask(a[b, :, h]) * (C[b, :, g, :] @ B[b, :, g, :].T)
            np.testing.assert_allclose(gr["dX"][b, :, h, :], M.T @ dY[b, :, h, :], rtol=0, atol=1e-11)


def test_da_equals_reverse_cumsum_identity():
    # da_t = sum_{k>=t} (dY_k . Y_k - X_k . dX_k) + <dS_fin, S_fin>: the loss
    # depends on a only through the prefix sums cs_k, with dl/dcs_k = row sum
    # minus column sum of the weighted mask; an independent formula for da
    rng = np.random.default_rng(8)
    X, a, B, C = rand_case(rng, Bz=2, L=31, H=3, P=4, N=3, G=1)
    S0 = rng.standard_normal((2, 3, 4, 3))
    dY = rng.standard_normal(X.shape)
    dS = rng.standard_normal(S0.shape)
    Y, S = oracle.fwd(X, a, B, C, S0=S0)
    gr = oracle.bwd(X, a, B, C, dY, S0=S0, dS_fin=dS)
    term = np.sum(dY * Y, axis=3) - np.sum(X * gr["dX"], axis=3)          # [Bz, L, H]
    rev = np.flip(np.cumsum(np.flip(term, axis=1), axis=1), axis=1)
    expect = rev + np.sum(dS * S, axis=(2, 3))[:, None, :]
    np.testing.assert_allclose(gr["da"], expect, rtol=0, atol=1e-10 * np.max(np.abs(expect)))


def test_zero_decay_gradients_are_linear_attention_gradients():
    # a = 0: Y = tril(C B^T) X per slice, so dC_t = sum_{s<=t} (dY_t . X_s) B_s
    # and dB_s = sum_{t>=s} (dY_t . X_s) C_t, summed over the group's heads
    rng = np.random.default_rng(9)
    X, _, B, C = rand_case(rng, Bz=1, L=17, H=4, P=3, N=5, G=2)
    a = np.zeros(X.shape[:3])
    dY = rng.standard_normal(X.shape)
    gr = oracle.bwd(X, a, B, C, dY)
    Bz, L, H, P = X.shape
    G = B.shape[2]
    dB = np.zeros(B.shape)
    dC = np.zeros(C.shape)
    for h in range(H):
        g = h * G // H
        W = np.tril(dY[0, :, h, :] @ X[0, :, h, :].T)      # W[t, s] = dY_t . X_s, s <= t
        dC[0, :, g, :] += W @ B[0, :, g, :]
        dB[0, :, g, :] += W.T @ C[0, :, g, :]
    np.testing.assert_allclose(gr["dC"], dC, rtol=0, atol=1e-11)
    np.testing.assert_allclose(gr["dB"], dB, rtol=0, atol=1e-11)


def test_gradients_across_recompute_segments():
    # a sequence longer than the oracle's 64-step recompute segment, checked
    # through the transposed quadratic form (dX) and the initial-state
    # response (dS0 = sum_t exp(cs_t) dY_t (x) C_t with zero dS_fin)
    rng = np.random.default_rng(10)
    X, a, B, C = rand_case(rng, Bz=1, L=150, H=2, P=2, N=3, G=1, a_scale=0.05)
    S0 = rng.standard_normal((1, 2, 2, 3))
    dY = rng.standard_normal(X.shape)
    gr = oracle.bwd(X, a, B, C, dY, S0=S0)
    for h in range(2):
        M = oracle.decay_mask(a[0, :, h]) * (C[0, :, 0, :] @ B[0, :, 0, :].T)
        np.testing.assert_allclose(gr["dX"][0, :, h, :], M.T @ dY[0, :, h, :], rtol=0, atol=1e-10)
        cs = np.cumsum(a[0, :, h])
        dS0 = np.einsum("t,tp,tn->pn", np.exp(cs), dY[0, :, h, :], C[0, :, 0, :])
        np.testing.assert_allclose(gr["dS0"][0, h], dS0, rtol=0, atol=1e-10)
