"""GPU parity of the fused output epilogue (w4a16_gemm_ex, through the C ABI):
y = aux_op(act(X.deq * col_scale + bias), aux), against the CPU oracle's
epilogue on the oracle's product.  Every kernel path that stores Y is covered:
split-K whole blocks, split-K blocks shared inside a workgroup and between
workgroups, the tiled kernel with and without a split of K.

Bar: max |Y - Y_ref| / Bo <= 2e-3 (fp16) or 1e-2 (bf16), where Bo carries the
product's bound B through the epilogue (see the oracle).
"""
import numpy as np
import pytest

import oracle
import w4a16_synth as synth
from gpu_helpers import TOL, OnDevice, env, lib, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lib()


# (label, M, K, N, G, variant, environment overrides)
PATHS = [
    ("splitk-whole-blocks", 3, 2048, 512, 128, "splitk", {}),
    ("splitk-shared-blocks", 5, 1024, 256, 64, "splitk", {"W4A16_SPLITK_WGS": 3}),
    ("splitk-m32", 32, 1024, 384, 32, "splitk", {"W4A16_SPLITK_WGS": 2}),
    ("tiled-mt2-split", 40, 2048, 512, 128, "tiled", {}),
    ("tiled-mt4", 150, 512, 1024, 64, "tiled", {"W4A16_SPLITS": 1}),
    ("tiled-mt4-split", 70, 4096, 256, 128, "tiled", {"W4A16_SPLITS": 4}),
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
    _, M, K, N, G, variant, extra = path
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
    with env(W4A16_FORCE_VARIANT=variant, **extra):
        if aux_mode == "inplace":
            Y = aux_t.clone().reshape(M, N)
            w4.w4a16_gemm_ex(d.X, d.packed, Y=Y, col_scale=cs_t, bias=bias_t, aux=Y,
                             activation=act, aux_op="add")
        else:
            Y = w4.w4a16_gemm_ex(d.X, d.packed, col_scale=cs_t, bias=bias_t, aux=aux_t,
                                 activation=act, aux_op=aux_mode or "add")
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
# (workload, epilogue) with sampled outputs against the oracle.
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
    rng = np.random.default_rng(2)
    ms = np.concatenate([rng.integers(0, p.M, 256), np.full(16, p.M - 1)])
    ns = np.concatenate([rng.integers(0, p.N, 256), np.arange(16) + p.N - 16])
    Yref, B = oracle.gemm_at(p.X, p.qweight, p.scales, p.zeros, p.M, p.N, p.K, p.G, p.dtype,
                             p.sym, ms, ns)
    Yo, Bo = oracle.epilogue(Yref, B, p.M, p.N, p.dtype, col_scale=cs, bias=bias,
                             aux=aux if aux_op else None, activation=act,
                             aux_op=aux_op or "add", ms=ms, ns=ns)
    Yg = d.y_float(Y)[ms, ns]
    rel, zero_ok = oracle.max_rel_error(Yg, Yo, Bo)
    assert zero_ok and rel <= TOL[p.dtype], f"{name}: max|Y-Yref|/Bo = {rel:.3e}"


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=[q[0] for q in PATHS])
def test_neutral_epilogue_is_bitwise_the_plain_product(path, dtype):
    """Column scale 1 and bias 0 run the epilogue kernels through every step
    (t = v*1 + 0, identity) and must store exactly what the plain kernels
    store (up to the sign of zero)."""
    from gpu_helpers import same_bits
    _, M, K, N, G, variant, extra = path
    sym = dtype == "bf16"
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=7 * M + N)
    d = OnDevice(p)
    w4 = d.w4
    ones = torch.ones(N, dtype=torch.float32, device=d.X.device)
    zeros = torch.zeros(N, dtype=w4.torch_dtype(d.flags), device=d.X.device)
    say(f"neutral epilogue {path[0]} / {dtype}")
    with env(W4A16_FORCE_VARIANT=variant, **extra):
        Y0 = w4.w4a16_gemm(d.X, d.packed)
        Y1 = w4.w4a16_gemm_ex(d.X, d.packed, col_scale=ones, bias=zeros)
    torch.cuda.synchronize()
    assert same_bits(w4.bits_of(Y0), w4.bits_of(Y1))
