"""Pins for the oracle's output epilogue (y = aux_op(act(Y*c + b), a)): checks
against closed forms, identities and orderings fixed by mathematics, so that a
wrong step (order of scale and bias, activation before the bias, the auxiliary
operand before the activation, a wrong SiLU) fails one of them.  CPU only.
"""
import math

import numpy as np
import pytest

import w4a16_synth as synth

F16_ONE, BF16_ONE = 0x3C00, 0x3F80
F16_TWO, BF16_TWO = 0x4000, 0x4000


def one_bits(dtype):
    return F16_ONE if dtype == "fp16" else BF16_ONE


def small_gemm(oracle_mod, dtype, seed=3, M=5, K=256, N=128, G=64, sym=False):
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=seed)
    Y, B = oracle_mod.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, sym)
    return p, Y, B


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_identity_epilogue_is_the_plain_product(oracle_mod, dtype):
    _, Y, B = small_gemm(oracle_mod, dtype)
    Yo, Bo = oracle_mod.epilogue(Y, B, *Y.shape, dtype)
    assert np.array_equal(Yo, Y) and np.array_equal(Bo, B)


def test_relu_is_max_with_zero(oracle_mod):
    _, Y, B = small_gemm(oracle_mod, "fp16")
    Yo, _ = oracle_mod.epilogue(Y, B, *Y.shape, "fp16", activation="relu")
    assert np.array_equal(Yo, np.where(Y > 0, Y, 0.0))
    assert np.any(Y < 0) and np.any(Y > 0)


def test_silu_closed_form_points(oracle_mod):
    # sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4, so silu(+-ln 3) = +-ln 3 * (3/4 or 1/4)
    l3 = math.log(3.0)
    Y = np.array([[0.0, l3, -l3, 40.0, -40.0]])
    Yo, _ = oracle_mod.epilogue(Y, np.abs(Y), 1, 5, "fp16", activation="silu")
    expect = [0.0, 0.75 * l3, -0.25 * l3, 40.0, 0.0]
    assert np.allclose(Yo[0], expect, rtol=1e-15, atol=1e-15)


def test_silu_odd_part_is_identity(oracle_mod):
    # silu(t) - silu(-t) = t (sigma(t) + sigma(-t) = 1); -X gives exactly -Y
    p, Y, B = small_gemm(oracle_mod, "bf16", seed=7)
    Xn = p.X ^ np.uint16(0x8000)
    Yn, _ = oracle_mod.gemm(Xn, p.qweight, p.scales, p.zeros, p.M, p.N, p.K, p.G, "bf16", False)
    assert np.array_equal(Yn, -Y)
    a, _ = oracle_mod.epilogue(Y, B, *Y.shape, "bf16", activation="silu")
    b, _ = oracle_mod.epilogue(Yn, B, *Y.shape, "bf16", activation="silu")
    assert np.allclose(a - b, Y, rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_scale_then_bias_then_activation_then_aux(oracle_mod, dtype):
    one, two = one_bits(dtype), (F16_TWO if dtype == "fp16" else BF16_TWO)
    Y = np.array([[1.0, -1.0, -0.5]])
    B = np.abs(Y)
    cs = np.array([2.0, 2.0, 1.0])
    bias = np.array([one, one, one], dtype=np.uint16)
    # scale before bias: 1*2 + 1 = 3 (not (1 + 1)*2 = 4)
    Yo, _ = oracle_mod.epilogue(Y, B, 1, 3, dtype, col_scale=cs, bias=bias)
    assert list(Yo[0]) == [3.0, -1.0, 0.5]
    # bias before the activation: relu(-0.5 + 1) = 0.5 (not relu(-0.5) + 1 = 1)
    Yo, _ = oracle_mod.epilogue(Y, B, 1, 3, dtype, col_scale=cs, bias=bias, activation="relu")
    assert list(Yo[0]) == [3.0, 0.0, 0.5]
    # the auxiliary operand after the activation: relu(-1) + 2 = 2 (not relu(1) = 1)
    aux = np.full((1, 3), two, dtype=np.uint16)
    Yo, _ = oracle_mod.epilogue(Y, B, 1, 3, dtype, activation="relu", aux=aux)
    assert list(Yo[0]) == [3.0, 2.0, 2.0]
    Yo, _ = oracle_mod.epilogue(Y, B, 1, 3, dtype, activation="relu", aux=aux, aux_op="mul")
    assert list(Yo[0]) == [2.0, 0.0, 0.0]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_unit_operands_leave_the_product(oracle_mod, dtype):
    _, Y, B = small_gemm(oracle_mod, dtype, seed=11)
    M, N = Y.shape
    ones = np.full((M, N), one_bits(dtype), dtype=np.uint16)
    zeros = np.zeros((M, N), dtype=np.uint16)
    Yo, Bo = oracle_mod.epilogue(Y, B, M, N, dtype, col_scale=np.ones(N), aux=ones, aux_op="mul")
    assert np.array_equal(Yo, Y) and np.array_equal(Bo, B)
    Yo, _ = oracle_mod.epilogue(Y, B, M, N, dtype, bias=np.zeros(N, np.uint16), aux=zeros)
    assert np.array_equal(Yo, Y)
    Yo, _ = oracle_mod.epilogue(Y, B, M, N, dtype, aux=zeros, aux_op="mul")
    assert np.all(Yo == 0)


def test_bias_and_aux_decode_their_dtype(oracle_mod):
    Y = np.zeros((1, 2))
    # fp16 0x3555 = 0.333251953125; bf16 0x3EAB = 0.333984375
    Yo, _ = oracle_mod.epilogue(Y, Y, 1, 2, "fp16", bias=np.array([0x3555, 0xC000], np.uint16))
    assert list(Yo[0]) == [0.333251953125, -2.0]
    Yo, _ = oracle_mod.epilogue(Y, Y, 1, 2, "bf16", aux=np.array([[0x3EAB, 0xC000]], np.uint16))
    assert list(Yo[0]) == [0.333984375, -2.0]


def test_silu_slope_stays_below_the_bound_constant(oracle_mod):
    """The error bound carries a perturbation of t through SiLU with L = 1.1.
    SiLU's slope sigma(t) (1 + t (1 - sigma(t))) peaks near t = 2.3994 at about
    1.0998 and dips to about -0.0998 near t = -2.3994, so |silu'| < 1.1: every
    difference quotient of the oracle's SiLU over a dense grid stays inside
    (-1.1, 1.1), and the extremes come within 1e-3 of those values (a looser
    L would hide nothing, a SiLU with the wrong slope fails)."""
    t = np.linspace(-30.0, 30.0, 600001)
    Yo, _ = oracle_mod.epilogue(t[None, :], np.abs(t)[None, :], 1, t.size, "fp16",
                                activation="silu")
    q = np.diff(Yo[0]) / np.diff(t)
    assert q.max() < 1.1 and q.min() > -1.1
    assert abs(q.max() - 1.0998) < 1e-3 and abs(q.min() + 0.0998) < 1e-3
    assert abs(t[np.argmax(q)] - 2.3994) < 1e-2
    # far from 0 the slope tends to 1 on the right and 0 on the left
    assert abs(q[-1] - 1.0) < 1e-9 and abs(q[0]) < 1e-9


@pytest.mark.parametrize("act", ["none", "relu", "silu"])
@pytest.mark.parametrize("aux_op", ["add", "mul"])
def test_bound_covers_the_output(oracle_mod, act, aux_op):
    p, Y, B = small_gemm(oracle_mod, "fp16", seed=5)
    M, N = Y.shape
    rng = np.random.default_rng(0)
    cs = rng.uniform(-2.0, 2.0, N)
    bias = np.asarray(synth.to_dtype_bits(rng.normal(0, 1, N), "fp16"), dtype=np.uint16)
    aux = np.asarray(synth.to_dtype_bits(rng.normal(0, 1, (M, N)), "fp16"), dtype=np.uint16)
    Yo, Bo = oracle_mod.epilogue(Y, B, M, N, "fp16", col_scale=cs, bias=bias, aux=aux,
                                 activation=act, aux_op=aux_op)
    assert np.all(np.abs(Yo) <= Bo * (1 + 1e-12))


def test_sampled_elements_match_full(oracle_mod):
    p, Y, B = small_gemm(oracle_mod, "bf16", seed=9)
    M, N = Y.shape
    rng = np.random.default_rng(1)
    cs = rng.uniform(0.5, 1.5, N)
    aux = np.asarray(synth.to_dtype_bits(rng.normal(0, 1, (M, N)), "bf16"), dtype=np.uint16)
    full, fb = oracle_mod.epilogue(Y, B, M, N, "bf16", col_scale=cs, aux=aux, activation="silu")
    ms = np.array([0, 4, 2, 1]); ns = np.array([5, 127, 0, 64])
    part, pb = oracle_mod.epilogue(Y[ms, ns], B[ms, ns], M, N, "bf16", col_scale=cs, aux=aux,
                                   activation="silu", ms=ms, ns=ns)
    assert np.array_equal(part, full[ms, ns]) and np.array_equal(pb, fb[ms, ns])
