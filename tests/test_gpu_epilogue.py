"""GPU parity of the fused output epilogue (w4a16_gemm_ex, through the C ABI):
y = aux_op(act(X.deq * col_scale + bias), aux), against the CPU oracle's
epilogue on the oracle's product.  Every kernel path that stores Y is covered:
the decode kernel (one workgroup per tile, and one workgroup running many
items in turn), the wide kernel (whole blocks, and blocks split into parts
that meet in the workspace), split-K whole blocks, split-K blocks shared inside a workgroup
and between workgroups, the tiled kernel with and without a split of K.

Bar: max |Y - Y_ref| / Bo <= 2e-3 (fp16) or 1e-2 (bf16), where Bo carries the
product's bound B through the epilogue (see the oracle).
"""
import numpy as np
import pytest

import oracle
import w4a16_synth as synth
from gpu_helpers import TOL, OnDevice, lib, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lib()


# (label, M, K, N, G, plan hint)
PATHS = [
    ("decode-m1", 1, 2048, 512, 128, "decode"),
    ("decode-m8-one-wg", 8, 1024, 768, 64, ("decode", 1)),
    ("decode-m7-split", 7, 1024, 384, 32, ("decode", 5)),
    ("wide-m64", 64, 2048, 512, 128, "wide"),
    ("wide-m100-parts", 100, 1024, 256, 64, ("wide", 16)),
    ("splitk-whole-blocks", 3, 2048, 512, 128, "splitk"),
    ("splitk-shared-blocks", 5, 1024, 256, 64, ("splitk", 3)),
    ("splitk-m32", 32, 1024, 384, 32, ("splitk", 2)),
    ("tiled-mt2-split", 40, 2048, 512, 128, "tiled"),
    ("tiled-mt4", 150, 512, 1024, 64, ("tiled", 1)),
    ("tiled-mt4-split", 70, 4096, 256, 128, ("tiled", 4)),
]

# (label, use col_scale, use bias, aux: None | "add" | "mul" | "inplace", activation)
EPILOGUES = [
    ("scale-bias-silu-add", True, True, "add", "silu"),
    ("relu-mul", False, False, "mul", "relu"),
    ("bias-only", False, True, None, "none"),
    ("scale-relu", True, False, None, "relu"),
    ("inplace-residual", False, True, "inplace", "silu"),
    ("empty", False, False, None, "none"),
]


def operands(p, seed):
    rng = np.random.default_rng(seed)
    cs = rng.uniform(-1.5, 1.5, p.N).astype(np.float32)
    bias = synth.to_dtype_bits(rng.normal(0.0, 0.5, p.N), p.dtype).astype(np.uint16)
    aux = synth.to_dtype_bits(rng.normal(0.0, 1.0, (p.M, p.N)), p.dtype).astype(np.uint16)
    return cs, bias, aux


def run_case(path, epi, dtype):
    _, M, K, N, G, plan = path
    elabel, use_cs, use_bias, aux_mode, act = epi
    sym = dtype == "bf16"
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=M + K + N)
    d = OnDevice(p)
    w4 = d.w4
    cs, bias, aux = operands(p, seed=N)
    tdt = w4.torch_dtype(d.flags)
    dev = d.X.device
    cs_t = torch.from_numpy(cs).to(dev) if use_cs else None
    bias_t = torch.from_numpy(bias.view(np.int16)).view(tdt).to(dev) if use_bias else None
    aux_t = torch.from_numpy(aux.view(np.int16)).view(tdt).to(dev) if aux_mode else None
    say(f"epilogue {path[0]} / {elabel} / {dtype}: M={M} K={K} N={N} G={G}")
    if aux_mode == "inplace":
        Y = aux_t.clone().reshape(M, N)
        w4.w4a16_gemm_ex(d.X, d.packed, Y=Y, col_scale=cs_t, bias=bias_t, aux=Y,
                         activation=act, aux_op="add", plan=plan)
    else:
        Y = w4.w4a16_gemm_ex(d.X, d.packed, col_scale=cs_t, bias=bias_t, aux=aux_t,
                             activation=act, aux_op=aux_mode or "add", plan=plan)
    torch.cuda.synchronize()
    Yg = d.y_float(Y)
    Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, sym)
    Yo, Bo = oracle.epilogue(Yref, B, M, N, dtype, col_scale=cs if use_cs else None,
                             bias=bias if use_bias else None,
                             aux=aux if aux_mode else None, activation=act,
                             aux_op="mul" if aux_mode == "mul" else "add")
    rel, zero_ok = oracle.max_rel_error(Yg, Yo, Bo)
    assert zero_ok, "an output with bound 0 is not 0"
    assert rel <= TOL[dtype], f"max|Y-Yref|/Bo = {rel:.3e} > {TOL[dtype]}"
    return rel


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("epi", EPILOGUES, ids=[e[0] for e in EPILOGUES])
@pytest.mark.parametrize("path", PATHS, ids=[q[0] for q in PATHS])
def test_epilogue_matches_oracle(path, epi, dtype):
    run_case(path, epi, dtype)


def test_empty_epilogue_equals_plain_gemm():
    p = synth.make_problem(9, 2048, 768, G=128, dtype="fp16", sym=False, seed=4)
    d = OnDevice(p)
    Y0 = d.gemm()
    Y1 = d.w4.w4a16_gemm_ex(d.X, d.packed)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)


def test_epilogue_rejects_bad_arguments():
    w4 = lib()
    p = synth.make_problem(2, 256, 128, G=128, dtype="fp16", sym=False, seed=1)
    d = OnDevice(p)
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_gemm_ex(d.X, d.packed, activation="gelu")
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_gemm_ex(d.X, d.packed, bias=torch.zeros(64, dtype=torch.float16, device="cuda"))
    # an aux that overlaps Y without being Y
    Y = torch.zeros((2, 128 + 8), dtype=torch.float16, device="cuda")
    Yv = Y.view(-1)[: 2 * 128].view(2, 128)
    aux = Y.view(-1)[8: 8 + 2 * 128]
    lib_ = w4.load_library()
    ep = w4.Epilogue(None, None, aux.data_ptr(), 0, 0)
    import ctypes
    st = lib_.w4a16_gemm_ex(ctypes.c_void_p(d.X.data_ptr()), ctypes.c_void_p(d.packed.data.data_ptr()),
                            d.packed.data.numel(), ctypes.c_void_p(Yv.data_ptr()), 2, 128, 256, 128,
                            d.flags, ctypes.byref(ep), None, 0, None)
    assert st == w4.W4A16_ERR_INVALID_ARG


# Full-size shapes of a decoder FFN block, as the fused-block benchmark runs them:
# (workload, epilogue), every output element against the oracle.
FULL = [
    ("decode_m1_k8192_n28672_fp16_asym_g128_outliers", "silu", None),
    ("decode_m8_k8192_n28672_fp16_asym_g128_outliers", "none", "mul"),
    ("transition_m16_k28672_n8192_bf16_sym_g128", "none", "add"),
    ("batch_m64_k8192_n28672_fp16_asym_g64", "silu", "add"),
]


@pytest.mark.parametrize("name,act,aux_op", FULL, ids=[f[0] for f in FULL])
def test_full_size_epilogue(name, act, aux_op):
    w4 = lib()
    p = synth.workload(name)
    say(f"full-size epilogue {name}: act={act} aux={aux_op}")
    d = OnDevice(p)
    cs, bias, aux = operands(p, seed=3)
    tdt = w4.torch_dtype(d.flags)
    dev = d.X.device
    cs_t = torch.from_numpy(cs).to(dev)
    bias_t = torch.from_numpy(bias.view(np.int16)).view(tdt).to(dev)
    aux_t = torch.from_numpy(aux.view(np.int16)).view(tdt).to(dev) if aux_op else None
    Y = w4.w4a16_gemm_ex(d.X, d.packed, col_scale=cs_t, bias=bias_t, aux=aux_t,
                         activation=act, aux_op=aux_op or "add")
    torch.cuda.synchronize()
    Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, p.M, p.N, p.K, p.G, p.dtype, p.sym)
    Yo, Bo = oracle.epilogue(Yref, B, p.M, p.N, p.dtype, col_scale=cs, bias=bias,
                             aux=aux if aux_op else None, activation=act,
                             aux_op=aux_op or "add")
    rel, zero_ok = oracle.max_rel_error(d.y_float(Y), Yo, Bo)
    assert zero_ok and rel <= TOL[p.dtype], f"{name}: max|Y-Yref|/Bo = {rel:.3e}"


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=[q[0] for q in PATHS])
def test_neutral_epilogue_is_bitwise_the_plain_product(path, dtype):
    """Column scale 1 and bias 0 run the epilogue kernels through every step
    (t = v*1 + 0, identity) and must store exactly what the plain kernels
    store (up to the sign of zero)."""
    from gpu_helpers import same_bits
    _, M, K, N, G, plan = path
    sym = dtype == "bf16"
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=7 * M + N)
    d = OnDevice(p)
    w4 = d.w4
    ones = torch.ones(N, dtype=torch.float32, device=d.X.device)
    zeros = torch.zeros(N, dtype=w4.torch_dtype(d.flags), device=d.X.device)
    say(f"neutral epilogue {path[0]} / {dtype}")
    Y0 = w4.w4a16_gemm(d.X, d.packed, plan=plan)
    Y1 = w4.w4a16_gemm_ex(d.X, d.packed, col_scale=ones, bias=zeros, plan=plan)
    torch.cuda.synchronize()
    assert same_bits(w4.bits_of(Y0), w4.bits_of(Y1))


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("M,Hd,F", [(1, 8192, 28672), (8, 1024, 2048), (40, 1024, 2048)])
def test_ffn_chain_matches_oracle(M, Hd, F):
    """A decoder FFN block as three fused calls, Gt = silu(X Wg),
    Ht = (X Wu) * Gt, Y = Ht Wd + X (fp16, G = 128).

    Each call is compared with the oracle fed the same operands the GPU call
    read (the GPU's own Gt and Ht), every output element, to the product's bar
    tol * Bo.  The chain's end is then compared with the oracle chain (the
    oracle's own intermediates, rounded to fp16 as the library stores them).
    First-order propagation bounds their difference: |Gt - G_or| <= 2 tol Bo1
    (the call's error plus the oracle's rounding), so
    |Ht - H_or| <= tol (Bo2 + Bo2_or + 2 Bu Bo1) =: tol D with Bu the bound of
    X Wu, and |Y - Y_or| <= tol (Bo3 + sum_k D[m][k] |Wd[k][n]|)."""
    w4 = lib()
    G, dt = 128, "fp16"
    tol = TOL[dt]
    flags = w4.flags_of(dt, False)
    dev = torch.device("cuda")
    say(f"ffn chain M={M} H={Hd} F={F}")
    probs = [synth.make_problem(1, K, N, G=G, dtype=dt, sym=False, seed=seed)
             for seed, (K, N) in ((31, (Hd, F)), (32, (Hd, F)), (33, (F, Hd)))]
    blobs = []
    for p in probs:
        _, qw, sc, zr = w4.to_device(p, dev)
        blobs.append(w4.w4a16_repack(qw, sc, zr, p.K, p.N, G, flags))
    Xb = synth.make_activations(M, Hd, dt, seed=9)
    X = torch.from_numpy(Xb.view(np.int16)).view(torch.float16).to(dev)
    Gt = w4.w4a16_gemm_ex(X, blobs[0], activation="silu")
    Ht = w4.w4a16_gemm_ex(X, blobs[1], aux=Gt, aux_op="mul")
    Y = w4.w4a16_gemm_ex(Ht, blobs[2], aux=X, aux_op="add")
    torch.cuda.synchronize()
    Gb, Hb, Yb = _bits(Gt), _bits(Ht), _bits(Y)
    pg, pu, pd = probs

    def product(p, Xin):
        return oracle.gemm(Xin, p.qweight, p.scales, p.zeros, M, p.N, p.K, G, dt, False)

    def f(b):
        return oracle.bits_to_float(b, dt)

    yg, bg = product(pg, Xb)
    yu, bu = product(pu, Xb)
    g_ref, g_bo = oracle.epilogue(yg, bg, M, F, dt, activation="silu")
    h_ref, h_bo = oracle.epilogue(yu, bu, M, F, dt, aux=Gb, aux_op="mul")
    yd, bd = product(pd, Hb)
    y_ref, y_bo = oracle.epilogue(yd, bd, M, Hd, dt, aux=Xb, aux_op="add")
    # stage by stage, on the GPU's own operands
    for name, got, ref, bo in (("gate", Gb, g_ref, g_bo), ("up*gate", Hb, h_ref, h_bo),
                               ("down+res", Yb, y_ref, y_bo)):
        rel, zero_ok = oracle.max_rel_error(f(got), ref, bo)
        assert zero_ok and rel <= tol, f"{name}: max|Y-Yref|/Bo = {rel:.3e}"
    # the oracle's own chain
    g_or = synth.to_dtype_bits(g_ref, dt)
    h_or, h_or_bo = oracle.epilogue(yu, bu, M, F, dt, aux=g_or, aux_op="mul")
    yo, bo = product(pd, synth.to_dtype_bits(h_or, dt))
    y_or, y_or_bo = oracle.epilogue(yo, bo, M, Hd, dt, aux=Xb, aux_op="add")
    # sum_k D[m][k] |Wd[k][n]| is the bound column of a product whose
    # activations are D (rounded up to fp16, scaled by a power of two to fit)
    D = (h_bo + h_or_bo + 2.0 * bu * g_bo) * (1 + 2.0 ** -9)
    sc = 2.0 ** max(0, int(np.ceil(np.log2(max(float(D.max()), 1.0) / 16384.0))))
    _, carried = product(pd, synth.to_dtype_bits(D / sc, dt))
    bound = tol * (np.maximum(y_bo, y_or_bo) + sc * carried)
    err = np.abs(f(Yb) - y_or)
    worst = float(np.max(err / np.where(bound > 0, bound, np.inf)))
    assert np.all(err <= bound), f"chain end: max err/bound = {worst:.3f}"
