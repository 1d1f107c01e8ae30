"""Pins for the fp64 oracle: each check ties it to something other than itself.

The pages (PaddleFleet PR #1772, "Fuse HCA inverse RoPE into the VHA postmix,
and the sparse-attention KV index remap") print no worked numeric example, so
the oracle is pinned by:
  * a hand-worked rotation written as complex multiplication, with cos/sin from
    a high-precision Taylor series (no libm);
  * the rotation built as a matrix exponential of its generator (scipy expm);
  * reductions to the textbook batched GEMM (numpy einsum) when positions are
    zero or pe = 0;
  * invariants: inverse RoPE after RoPE is the identity, pair norms are kept,
    W = I returns the inverse-rotated input, the channel axis is a pure N
    dimension (each output column depends only on its own input column and,
    for pe channels, the rotation partner);
  * the adjoint identities <dY, Y> = <dO, O> = <dW, W> (Y is linear in O and W);
  * central finite differences for dO and dW (exact up to rounding: linear loss);
  * the one-by-one evaluators agree with the full ones;
  * the magnitude sums of the weight-gradient terms (each dW entry's
    conditioning, used by the GPU tests' dW bound) against brute force with
    the expm rotations, and against dW itself when every term is
    non-negative.
"""
from decimal import Decimal, localcontext

import numpy as np
import pytest
import scipy.linalg

import oracle
from rope_head_mixing_amd import synthetic

THETA = 10000.0


# --------------------------------------------------------------------------
# independent helpers (no oracle code, no libm trig)
# --------------------------------------------------------------------------

def _decimal_arctan_inv(n: int, digits: int) -> Decimal:
    """arctan(1/n) by its series, in the current decimal context."""
    x = Decimal(1) / n
    x2, term, total, k = x * x, x, x, 1
    tiny = Decimal(10) ** (-(digits + 5))
    while abs(term) > tiny:
        term = -term * x2
        total += term / (2 * k + 1)
        k += 1
    return total


def taylor_cos_sin(x: float, digits: int = 90) -> tuple[float, float]:
    """cos(x), sin(x) by their Maclaurin series in decimal arithmetic, after
    reducing x modulo 2*pi with pi from Machin's formula."""
    with localcontext() as ctx:
        ctx.prec = digits
        pi = 4 * (4 * _decimal_arctan_inv(5, digits) - _decimal_arctan_inv(239, digits))
        X = Decimal(float(x))  # the exact binary value of x
        X -= (X / (2 * pi)).to_integral_value() * 2 * pi
        c, s = Decimal(0), Decimal(0)
        tc, ts = Decimal(1), X
        n = 0
        tiny = Decimal(10) ** (-(digits - 10))
        while True:
            c += tc
            s += ts
            tc = -tc * X * X / ((2 * n + 1) * (2 * n + 2))
            ts = -ts * X * X / ((2 * n + 2) * (2 * n + 3))
            n += 1
            if n > 4 and abs(tc) < tiny and abs(ts) < tiny:
                break
        return float(c), float(s)


def rotation_matrix_expm(phis: np.ndarray, nope: int, pe: int, sign: int) -> np.ndarray:
    """d x d matrix exp(sign * sum_i phi_i * J_i), J_i the generator of the
    rotation in the (nope+i, nope+pe/2+i) plane that turns the first axis
    towards the second."""
    d, h2 = nope + pe, pe // 2
    # expm's scaling-and-squaring error grows with the norm, so turn each angle
    # into [0, 2*pi) first (costs ~k*|2pi_fp64 - 2pi| ~ 6e-13 rad at 16384 rad)
    phis = np.remainder(np.asarray(phis, np.float64), 2.0 * np.pi)
    G = np.zeros((d, d))
    for i in range(h2):
        a, b = nope + i, nope + h2 + i
        G[b, a] = phis[i]
        G[a, b] = -phis[i]
    return scipy.linalg.expm(sign * G)


def textbook_inv_freq(theta: float, pe: int) -> np.ndarray:
    """1 / theta^(2i/pe), i = 0..pe/2-1 (the usual RoPE frequency ladder)."""
    return 1.0 / (theta ** (np.arange(0, pe, 2, dtype=np.float64) / pe))


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def wmat(nh, seed):
    return np.eye(nh) + 0.3 * rand((nh, nh), seed)  # clearly non-symmetric


# --------------------------------------------------------------------------
# hand-worked rotation (complex multiplication, Taylor trig)
# --------------------------------------------------------------------------

def test_hand_worked_rotation_position_100():
    """pe=4, theta=1e4: the pairs turn by p*1 and p/100 rad; at p=100 that is
    100 rad and exactly 1 rad.  Inverse RoPE multiplies x_a + j*x_b by e^{-j phi}."""
    nope, pe = 2, 4
    row = np.array([1.0, 2.0, 3.0, 4.0, 5.0, 6.0])
    O = row.reshape(1, 1, 6)
    W = np.array([[1.0]])
    Y = oracle.fwd(O, W, [100], THETA, nope, pe)[0, 0]
    c0, s0 = taylor_cos_sin(100.0)
    c1, s1 = taylor_cos_sin(1.0)
    z0 = complex(3.0, 5.0) * complex(c0, -s0)
    z1 = complex(4.0, 6.0) * complex(c1, -s1)
    expect = np.array([1.0, 2.0, z0.real, z1.real, z0.imag, z1.imag])
    np.testing.assert_allclose(Y, expect, rtol=0, atol=1e-13)
    # and the bf16 entry point gives the same on bf16-exact integers
    Ob = synthetic.f32_to_bf16_bits(row.astype(np.float32)).reshape(1, 1, 6)
    Wb = synthetic.f32_to_bf16_bits(np.array([[1.0]], np.float32))
    np.testing.assert_allclose(oracle.fwd(Ob, Wb, [100], THETA, nope, pe)[0, 0], expect,
                               rtol=0, atol=1e-13)


def test_hand_worked_rope_direction():
    """RoPE (the backward's rotation) multiplies by e^{+j phi}: with W = [[1]],
    dO = rope(dY).  pe=2: one pair turned by exactly p rad; p=1."""
    nope, pe = 0, 2
    dY = np.array([[[0.25, -1.5]]])
    dO = oracle.bwd_dx(dY, np.array([[1.0]]), [1], THETA, nope, pe)[0, 0]
    c, s = taylor_cos_sin(1.0)
    z = complex(0.25, -1.5) * complex(c, s)
    np.testing.assert_allclose(dO, [z.real, z.imag], rtol=0, atol=1e-15)


def test_angles_match_textbook_ladder_and_taylor_trig():
    pe, pos = 8, np.array([0, 1, 7, 32767], np.int32)
    C, S = oracle.rope_angles(THETA, pe, pos)
    inv = textbook_inv_freq(THETA, pe)
    for si, p in enumerate(pos):
        for i in range(pe // 2):
            phi = float(p) * inv[i]
            c, s = taylor_cos_sin(phi)
            # the two fp64 angle evaluations may differ by a few ulp of phi
            tol = 1e-15 * max(1.0, phi) + 1e-15
            assert abs(C[si, i] - c) < tol and abs(S[si, i] - s) < tol


# --------------------------------------------------------------------------
# rotation invariants and brute force with explicit rotation matrices
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nope,pe", [(0, 2), (6, 4), (48, 16), (8, 64)])
def test_inv_rope_after_rope_is_identity(nope, pe):
    sq, nh = 5, 3
    X = rand((sq, nh, nope + pe), 11)
    pos = np.array([0, 3, 99, 4097, 32767], np.int32)
    back = oracle.inv_rope(oracle.rope(X, pos, THETA, nope, pe), pos, THETA, nope, pe)
    np.testing.assert_allclose(back, X, rtol=0, atol=1e-13)
    fwd_back = oracle.rope(oracle.inv_rope(X, pos, THETA, nope, pe), pos, THETA, nope, pe)
    np.testing.assert_allclose(fwd_back, X, rtol=0, atol=1e-13)


def test_rotation_keeps_pair_norms_and_nope_channels():
    nope, pe, sq, nh = 6, 10, 4, 2
    X = rand((sq, nh, nope + pe), 12)
    pos = np.array([1, 10, 100, 1000], np.int32)
    Y = oracle.inv_rope(X, pos, THETA, nope, pe)
    np.testing.assert_array_equal(Y[..., :nope], X[..., :nope])
    h2 = pe // 2
    nx = X[..., nope:nope + h2] ** 2 + X[..., nope + h2:] ** 2
    ny = Y[..., nope:nope + h2] ** 2 + Y[..., nope + h2:] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13)


@pytest.mark.parametrize("nh,nope,pe,theta", [(4, 48, 16, THETA), (3, 6, 4, 500.0),
                                               (5, 0, 8, THETA), (2, 8, 2, 77.0)])
def test_forward_brute_force_with_rotation_matrices(nh, nope, pe, theta):
    """Y[s] = W @ (O[s] @ R_s^T) with R_s = expm(-sum phi_i J_i) built from the
    textbook frequency ladder; no oracle code involved."""
    sq, d = 6, nope + pe
    O, W = rand((sq, nh, d), 21), wmat(nh, 22)
    pos = np.array([0, 1, 2, 63, 1000, 16384], np.int32)
    Y = oracle.fwd(O, W, pos, theta, nope, pe)
    inv = textbook_inv_freq(theta, pe)
    for s in range(sq):
        R = rotation_matrix_expm(pos[s] * inv, nope, pe, -1)
        ref = W @ (O[s] @ R.T)
        np.testing.assert_allclose(Y[s], ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("nh,nope,pe", [(4, 48, 16), (3, 6, 4)])
def test_backward_brute_force_with_rotation_matrices(nh, nope, pe):
    """dO[s] = (W^T @ dY[s]) @ R_s^{+} ^T and dW = sum_s dY[s] @ (O[s] @ R_s^-T)^T,
    with R^{+} = expm(+sum phi J) (the adjoint of the inverse rotation)."""
    sq, d = 5, nope + pe
    O, dY, W = rand((sq, nh, d), 31), rand((sq, nh, d), 32), wmat(nh, 33)
    pos = np.array([0, 7, 100, 2048, 32000], np.int32)
    dO = oracle.bwd_dx(dY, W, pos, THETA, nope, pe)
    dW = oracle.bwd_dw(dY, O, pos, THETA, nope, pe)
    inv = textbook_inv_freq(THETA, pe)
    dW_ref = np.zeros((nh, nh))
    for s in range(sq):
        Rm = rotation_matrix_expm(pos[s] * inv, nope, pe, -1)
        Rp = rotation_matrix_expm(pos[s] * inv, nope, pe, +1)
        np.testing.assert_allclose(Rp, Rm.T, atol=1e-14)  # inverse is the transpose
        np.testing.assert_allclose(dO[s], (W.T @ dY[s]) @ Rp.T, rtol=0, atol=1e-11)
        dW_ref += dY[s] @ (O[s] @ Rm.T).T
    np.testing.assert_allclose(dW, dW_ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("nh,nope,pe", [(4, 48, 16), (3, 6, 4), (1, 8, 8)])
def test_dw_term_magnitudes_brute_force(nh, nope, pe):
    """A[g,h] = sum_{s,c} |dY[s,g,c] X[s,h,c]| with X = O rotated by the
    expm matrices (numpy only), and A >= |dW| entry by entry."""
    sq, d = 5, nope + pe
    to_bits = synthetic.f32_to_bf16_bits
    O = to_bits(rand((sq, nh, d), 41).astype(np.float32))
    dY = to_bits(rand((sq, nh, d), 42).astype(np.float32))
    pos = np.array([0, 3, 99, 4000, 31000], np.int32)
    A = oracle.bwd_dw_abs(dY, O, pos, THETA, nope, pe)
    Of, dYf = synthetic.bf16_bits_to_f32(O).astype(np.float64), synthetic.bf16_bits_to_f32(dY).astype(np.float64)
    inv = textbook_inv_freq(THETA, pe)
    A_ref = np.zeros((nh, nh))
    for s in range(sq):
        X = Of[s] @ rotation_matrix_expm(pos[s] * inv, nope, pe, -1).T
        A_ref += np.abs(dYf[s]) @ np.abs(X).T
    np.testing.assert_allclose(A, A_ref, rtol=1e-12, atol=1e-12)
    dW = oracle.bwd_dw(dY, O, pos, THETA, nope, pe)
    assert np.all(A >= np.abs(dW) * (1 - 1e-12))


def test_dw_term_magnitudes_equal_dw_for_nonnegative_terms():
    """With zero positions (X = O) and non-negative dY and O, every term is
    non-negative, so A equals dW itself."""
    sq, nh, nope, pe = 6, 3, 16, 16
    to_bits = synthetic.f32_to_bf16_bits
    O = to_bits(np.abs(rand((sq, nh, nope + pe), 43)).astype(np.float32))
    dY = to_bits(np.abs(rand((sq, nh, nope + pe), 44)).astype(np.float32))
    pos = np.zeros(sq, np.int32)
    np.testing.assert_array_equal(oracle.bwd_dw_abs(dY, O, pos, THETA, nope, pe),
                                  oracle.bwd_dw(dY, O, pos, THETA, nope, pe))


# --------------------------------------------------------------------------
# special cases that reduce to the textbook batched GEMM
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nope,pe,pos", [(48, 16, 0), (64, 0, 123)])
def test_reduces_to_batched_gemm(nope, pe, pos):
    """Zero positions (no rotation) or pe = 0: Y = einsum('gh,shc->sgc', W, O),
    dO = einsum('gh,sgc->shc', W, dY), dW = einsum('sgc,shc->gh', dY, O)."""
    sq, nh, d = 7, 5, nope + pe
    O, dY, W = rand((sq, nh, d), 41), rand((sq, nh, d), 42), wmat(nh, 43)
    positions = np.full(sq, pos, np.int32)
    np.testing.assert_allclose(oracle.fwd(O, W, positions, THETA, nope, pe),
                               np.einsum("gh,shc->sgc", W, O), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.bwd_dx(dY, W, positions, THETA, nope, pe),
                               np.einsum("gh,sgc->shc", W, dY), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.bwd_dw(dY, O, positions, THETA, nope, pe),
                               np.einsum("sgc,shc->gh", dY, O), rtol=0, atol=1e-11)


def test_identity_mix_returns_inverse_rotation():
    sq, nh, nope, pe = 4, 3, 8, 8
    O = rand((sq, nh, nope + pe), 51)
    pos = np.array([2, 20, 200, 2000], np.int32)
    np.testing.assert_allclose(oracle.fwd(O, np.eye(nh), pos, THETA, nope, pe),
                               oracle.inv_rope(O, pos, THETA, nope, pe), rtol=0, atol=1e-14)


def test_channel_axis_is_a_pure_n_dimension():
    """Perturbing input channel c moves only output channel c (nope) or the
    pair {c, partner} (pe) -- the split-N property the fusion relies on."""
    sq, nh, nope, pe = 2, 3, 6, 8
    d, h2 = nope + pe, pe // 2
    O, W = rand((sq, nh, d), 61), wmat(nh, 62)
    pos = np.array([5, 77], np.int32)
    base = oracle.fwd(O, W, pos, THETA, nope, pe)
    for c in range(d):
        P = O.copy()
        P[1, 2, c] += 1.0
        diff = np.abs(oracle.fwd(P, W, pos, THETA, nope, pe) - base)
        moved = set(np.nonzero(diff.max(axis=(0, 1)) > 1e-12)[0].tolist())
        if c < nope:
            assert moved == {c}
        else:
            i = (c - nope) % h2
            assert moved == {nope + i, nope + h2 + i}
        assert diff[0].max() == 0.0  # other tokens untouched


# --------------------------------------------------------------------------
# adjoint identities and finite differences
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nh,nope,pe", [(4, 48, 16), (3, 10, 6), (1, 0, 2)])
def test_adjoint_identities(nh, nope, pe):
    sq, d = 9, nope + pe
    O, dY, W = rand((sq, nh, d), 71), rand((sq, nh, d), 72), wmat(nh, 73)
    pos = np.arange(1000, 1000 + sq, dtype=np.int32)
    Y = oracle.fwd(O, W, pos, THETA, nope, pe)
    dO = oracle.bwd_dx(dY, W, pos, THETA, nope, pe)
    dW = oracle.bwd_dw(dY, O, pos, THETA, nope, pe)
    L = float(np.sum(dY * Y))
    assert abs(float(np.sum(dO * O)) - L) <= 1e-12 * max(1.0, abs(L)) * sq * nh * d
    assert abs(float(np.sum(dW * W)) - L) <= 1e-12 * max(1.0, abs(L)) * sq * nh * d


def test_central_finite_differences():
    """L(O, W) = <dY, Y(O, W)> is linear in O and in W, so a central difference
    with step 1 is exact up to rounding."""
    sq, nh, nope, pe = 3, 4, 6, 6
    d = nope + pe
    O, dY, W = rand((sq, nh, d), 81), rand((sq, nh, d), 82), wmat(nh, 83)
    pos = np.array([3, 30, 300], np.int32)

    def L(O_, W_):
        return float(np.sum(dY * oracle.fwd(O_, W_, pos, THETA, nope, pe)))

    dO = oracle.bwd_dx(dY, W, pos, THETA, nope, pe)
    dW = oracle.bwd_dw(dY, O, pos, THETA, nope, pe)
    rng = np.random.default_rng(84)
    for _ in range(12):
        s, h, c = rng.integers(sq), rng.integers(nh), rng.integers(d)
        Op, Om = O.copy(), O.copy()
        Op[s, h, c] += 1.0
        Om[s, h, c] -= 1.0
        assert abs((L(Op, W) - L(Om, W)) / 2.0 - dO[s, h, c]) < 1e-11
    for g in range(nh):
        for h in range(nh):
            Wp, Wm = W.copy(), W.copy()
            Wp[g, h] += 1.0
            Wm[g, h] -= 1.0
            assert abs((L(O, Wp) - L(O, Wm)) / 2.0 - dW[g, h]) < 1e-11


# --------------------------------------------------------------------------
# entry-point consistency: bf16 decoding, threads, one-by-one evaluators
# --------------------------------------------------------------------------

def test_bf16_entry_points_match_widened_fp64():
    c = synthetic.case(13, 5, 24, 8, seed=91, pos_offset=40)
    O, W, dY, pos = c.O(), c.W(), c.dY(), c.positions()
    f = synthetic.bf16_bits_to_f32
    O64, W64, dY64 = (f(x).astype(np.float64) for x in (O, W, dY))
    np.testing.assert_array_equal(oracle.fwd(O, W, pos, THETA, c.nope, c.pe),
                                  oracle.fwd(O64, W64, pos, THETA, c.nope, c.pe))
    np.testing.assert_array_equal(oracle.bwd_dx(dY, W, pos, THETA, c.nope, c.pe),
                                  oracle.bwd_dx(dY64, W64, pos, THETA, c.nope, c.pe))
    np.testing.assert_allclose(oracle.bwd_dw(dY, O, pos, THETA, c.nope, c.pe),
                               oracle.bwd_dw(dY64, O64, pos, THETA, c.nope, c.pe),
                               rtol=1e-14, atol=1e-12)


def test_thread_count_does_not_change_results_beyond_rounding():
    c = synthetic.case(37, 4, 48, 16, seed=101)
    O, W, dY, pos = c.O(), c.W(), c.dY(), c.positions()
    y1 = oracle.fwd(O, W, pos, THETA, c.nope, c.pe, nthreads=1)
    y5 = oracle.fwd(O, W, pos, THETA, c.nope, c.pe, nthreads=5)
    np.testing.assert_array_equal(y1, y5)
    w1 = oracle.bwd_dw(dY, O, pos, THETA, c.nope, c.pe, nthreads=1)
    w5 = oracle.bwd_dw(dY, O, pos, THETA, c.nope, c.pe, nthreads=5)
    np.testing.assert_allclose(w1, w5, rtol=1e-13, atol=1e-11)


@pytest.mark.parametrize("sq,nh,nope,pe", [(19, 4, 48, 16), (11, 3, 24, 8), (6, 64, 448, 64)])
def test_one_by_one_evaluators_match_full(sq, nh, nope, pe):
    c = synthetic.case(sq, nh, nope, pe, seed=111, pos_offset=16384)
    O, W, dY, pos = c.O(), c.W(), c.dY(), c.positions()
    Y = oracle.fwd(O, W, pos, THETA, nope, pe)
    dO = oracle.bwd_dx(dY, W, pos, THETA, nope, pe)
    dW = oracle.bwd_dw(dY, O, pos, THETA, nope, pe)
    rng = np.random.default_rng(112)
    idx = rng.integers(0, Y.size, 200)
    idx[:3] = [0, Y.size - 1, Y.size - pe // 2]  # include ends and a pe channel
    np.testing.assert_allclose(oracle.fwd_at(O, W, pos, THETA, nope, pe, idx),
                               Y.reshape(-1)[idx], rtol=1e-14, atol=1e-13)
    np.testing.assert_allclose(oracle.bwd_dx_at(dY, W, pos, THETA, nope, pe, idx),
                               dO.reshape(-1)[idx], rtol=1e-14, atol=1e-13)
    widx = np.arange(nh * nh) if nh * nh <= 64 else rng.integers(0, nh * nh, 64)
    np.testing.assert_allclose(oracle.bwd_dw_at(dY, O, pos, THETA, nope, pe, widx),
                               dW.reshape(-1)[widx], rtol=1e-12, atol=1e-10)


def test_empty_token_range():
    O = np.zeros((0, 4, 64), np.float64)
    W = np.eye(4)
    pos = np.zeros(0, np.int32)
    assert oracle.fwd(O, W, pos, THETA, 48, 16).shape == (0, 4, 64)
    np.testing.assert_array_equal(oracle.bwd_dw(O, O, pos, THETA, 48, 16), np.zeros((4, 4)))


def test_rejects_odd_pe():
    with pytest.raises(ValueError):
        oracle.fwd(np.zeros((1, 1, 5)), np.eye(1), [0], THETA, 2, 3)


# --------------------------------------------------------------------------
# regression guard: the stored oracle outputs (written by tests/golden/make_golden.py)
# --------------------------------------------------------------------------

def test_golden_tiny_case_reproduces():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    with open(path) as f:
        g = json.load(f)
    sh = g["shape"]
    sq, nh, nope, pe = sh["sq"], sh["nh"], sh["nope"], sh["pe"]
    d = nope + pe

    def bits(key, shape):
        return np.array([int(v, 16) for v in g[key]], np.uint16).reshape(shape)

    O, W, dY = bits("O_bf16_hex", (sq, nh, d)), bits("W_bf16_hex", (nh, nh)), bits("dY_bf16_hex", (sq, nh, d))
    pos = np.array(g["positions"], np.int32)
    want = {k: np.array([float(v) for v in g[k]]) for k in ("Y", "dO", "dW")}
    np.testing.assert_allclose(oracle.fwd(O, W, pos, sh["theta"], nope, pe).reshape(-1), want["Y"],
                               rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(oracle.bwd_dx(dY, W, pos, sh["theta"], nope, pe).reshape(-1),
                               want["dO"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(oracle.bwd_dw(dY, O, pos, sh["theta"], nope, pe).reshape(-1),
                               want["dW"], rtol=1e-14, atol=1e-14)
