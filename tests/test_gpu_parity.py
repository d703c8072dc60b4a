"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bars (from the statement of the problem):
  * quantizer: signs identical, scales bit-identical in their dtype;
  * pack: the oracle's own unpacker reads back exactly the signs and scales;
  * product, exact regime (integer x in [-8, 8], scales 2^-e, e in 4..8):
    equal values;
  * product, general inputs: |y - y_ref| <= 1e-3 * sum_j |W_hat_ij| |x_j| for
    every output, with fp32 accumulation on the device.
Full-size layers are checked on sampled output rows that the oracle computes
on its own from the same seeded W and x.
"""
import os

import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, alpha_enum, gemm, gemv, np_alpha, pack_on_gpu, say, to_dev, x_to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


GEMV_VARIANTS = {
    "rows16": {"MBOK_GEMV_VARIANT": "rows", "MBOK_GEMV_R": "16"},
    "rows32": {"MBOK_GEMV_VARIANT": "rows", "MBOK_GEMV_R": "32"},
    "rows64": {"MBOK_GEMV_VARIANT": "rows", "MBOK_GEMV_R": "64", "MBOK_GEMV_NW": "4"},
    "split": {"MBOK_GEMV_VARIANT": "split"},
    "fullrow": {"MBOK_GEMV_VARIANT": "fullrow"},
    "direct": {"MBOK_GEMV_VARIANT": "direct"},
    "stream": {"MBOK_GEMV_VARIANT": "stream"},
    # fp4 x fp8 matrix-core kernel (bf16 x only; fp32 x keeps the table kernels)
    "f4": {"MBOK_GEMV_VARIANT": "f4"},
    # matrix-core kernel of the few-token product at one token (bf16 x only;
    # fp32 x keeps the table kernels)
    "skinny": {"MBOK_GEMV_VARIANT": "skinny"},
    "skinny_blocks_nw3": {"MBOK_GEMV_VARIANT": "skinny", "MBOK_SKINNY_VARIANT": "blocks",
                          "MBOK_SKINNY_NW": "3"},
}

ENV_KEYS = ("MBOK_GEMV_VARIANT", "MBOK_GEMV_R", "MBOK_GEMV_NW", "MBOK_SKINNY_NW",
            "MBOK_SKINNY_VARIANT")


def _swap_env(new: dict) -> dict:
    old = {k: os.environ.get(k) for k in ENV_KEYS}
    for k in ENV_KEYS:
        os.environ.pop(k, None)
    os.environ.update(new)
    return old


def _restore_env(old: dict):
    for k, v in old.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


@pytest.fixture(params=list(GEMV_VARIANTS))
def gemv_variant(request):
    old = _swap_env(GEMV_VARIANTS[request.param])
    yield request.param
    _restore_env(old)


# the few-token kernels: the streaming default, and the per-tile "blocks"
# form with several wavefronts per workgroup (uneven group ranges when NW
# does not divide G, one wavefront doing every group)
SKINNY_SHAPES = {
    "default": {},
    "stream": {"MBOK_SKINNY_VARIANT": "stream"},
    "blocks_nw3": {"MBOK_SKINNY_VARIANT": "blocks", "MBOK_SKINNY_NW": "3"},
    "blocks_nw7": {"MBOK_SKINNY_VARIANT": "blocks", "MBOK_SKINNY_NW": "7"},
    "blocks_nw1": {"MBOK_SKINNY_VARIANT": "blocks", "MBOK_SKINNY_NW": "1"},
}


@pytest.fixture(params=list(SKINNY_SHAPES))
def skinny_shape(request):
    old = _swap_env(SKINNY_SHAPES[request.param])
    yield request.param
    _restore_env(old)


def quantize_on_gpu(W: np.ndarray, K: int, dt: str):
    m, n = W.shape
    d = bw.mbok_desc_init(m, n, K, alpha_enum(dt))
    Wt = to_dev(W)
    signs = torch.empty((K, m, n), dtype=torch.int8, device=DEV)
    alpha = torch.empty((K, m, n // 128), dtype=bw.alpha_torch_dtype(d.alpha_dtype), device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    bw.mbok_residual_binarize(d, Wt, signs, alpha, flag)
    packed = torch.empty(bw.mbok_packed_bytes(d), dtype=torch.uint8, device=DEV)
    bw.mbok_pack(d, signs, alpha, packed)
    return d, signs, alpha, packed, int(flag.item())


def sample_rows(m: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, size=min(count, m), replace=False).tolist())
    rows |= {0, m - 1, min(63, m - 1), min(64, m - 1)}
    return np.array(sorted(rows))


# ----------------------------------------------------------------- quantizer

@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_quantizer_bit_exact_small(K, dt):
    say(f"quantizer small K={K} {dt}")
    W = syn.weight(100, 384, seed=300 + K)
    W[3, :9] = 0.0
    W[4, 5:11] = -0.0
    W[7, 128:256] = 0.0          # a whole zero group
    S, A, R = oracle.residual_binarize(W, K, alpha_dtype=dt)
    d, signs, alpha, packed, flag = quantize_on_gpu(W, K, dt)
    assert flag == 0
    assert np.array_equal(signs.cpu().numpy(), S)
    assert np.array_equal(alpha.cpu().numpy().view(np.uint8), A.view(np.uint8))
    S2, A2, clean = oracle.unpack(packed.cpu().numpy(), 100, 384, K, dt)
    assert np.array_equal(S2, S) and np.array_equal(A2.view(np.uint8), A.view(np.uint8)) and clean
    assert np.array_equal(packed.cpu().numpy(), oracle.pack(S, A, dt))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_quantizer_bit_exact_workloads_sampled(cfg):
    w = syn.WORKLOADS[cfg]
    dt = w["alpha_dtype"]
    for li, (name, m, n) in enumerate(w["linears"]):
        say(f"quantizer config {cfg} {name} {m}x{n} K={w['K']}")
        W = syn.weight(m, n, syn.weight_seed(cfg, li))
        d, signs, alpha, packed, flag = quantize_on_gpu(W, w["K"], dt)
        assert flag == 0
        rows = sample_rows(m, 128, cfg * 10 + li)
        S, A, _ = oracle.residual_binarize(W[rows], w["K"], alpha_dtype=dt)
        assert np.array_equal(signs.cpu().numpy()[:, rows], S), name
        assert np.array_equal(alpha.cpu().numpy()[:, rows].view(np.uint8), A.view(np.uint8)), name
        del signs, alpha, packed
        torch.cuda.empty_cache()


def test_quantizer_flags_non_finite():
    say("quantizer non-finite flag")
    W = syn.weight(64, 256, seed=7)
    W[10, 20] = np.nan
    d, signs, alpha, packed, flag = quantize_on_gpu(W, 2, "f16")
    assert flag == 1
    W[10, 20] = np.inf
    assert quantize_on_gpu(W, 2, "f16")[4] == 1
    W[10, 20] = 0.5
    assert quantize_on_gpu(W, 2, "f16")[4] == 0


def test_quantizer_row_stride():
    say("quantizer with ldw > n")
    W = syn.weight(70, 512, seed=8)
    Wbig = np.zeros((70, 640), dtype=np.float32)
    Wbig[:, :512] = W
    Wbig[:, 512:] = np.nan  # must never be read
    d = bw.mbok_desc_init(70, 512, 3, bw.MBOK_F16)
    signs = torch.empty((3, 70, 512), dtype=torch.int8, device=DEV)
    alpha = torch.empty((3, 70, 4), dtype=torch.float16, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    bw.mbok_residual_binarize(d, to_dev(Wbig), signs, alpha, flag)
    S, A, _ = oracle.residual_binarize(W, 3, alpha_dtype="f16")
    assert int(flag.item()) == 0
    assert np.array_equal(signs.cpu().numpy(), S)
    assert np.array_equal(alpha.cpu().numpy(), A)


# --------------------------------------------------------------------- pack

@pytest.mark.parametrize("K,m,n,dt", [(1, 1, 128, "f32"), (2, 63, 256, "f16"), (3, 65, 384, "f16"),
                                      (4, 130, 512, "f32"), (3, 256, 128, "f16")])
def test_pack_matches_oracle_layout(K, m, n, dt):
    say(f"pack K={K} m={m} n={n} {dt}")
    S = syn.random_signs(K, m, n, seed=K * 1000 + m)
    A = syn.exact_alpha(K, m, n // 128, seed=m).astype(np_alpha(dt))
    d, packed = pack_on_gpu(S, A, dt)
    buf = packed.cpu().numpy()
    assert np.array_equal(buf, oracle.pack(S, A, dt))
    S2, A2, clean = oracle.unpack(buf, m, n, K, dt)
    assert np.array_equal(S2, S) and np.array_equal(A2, A) and clean


# ------------------------------------------------------------ decode GEMV

EXACT_SHAPES = [(1, 128), (63, 256), (64, 128), (65, 384), (100, 512), (130, 1024),
                (256, 4096), (200, 5120), (70, 13824)]


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("m,n", EXACT_SHAPES)
def test_gemv_exact_regime(m, n, K, gemv_variant):
    for dt, xdt in (("f16", "bf16"), ("f32", "f32")):
        say(f"gemv exact {gemv_variant} m={m} n={n} K={K} {dt}/{xdt}")
        S = syn.random_signs(K, m, n, seed=m * 7 + n + K)
        A = syn.exact_alpha(K, m, n // 128, seed=m + K).astype(np_alpha(dt))
        x = syn.exact_activations(1, n, seed=n + K)[0]
        d, packed = pack_on_gpu(S, A, dt)
        y = gemv(d, packed, x, xdt, guard=17)
        want = oracle.product(S, A, x)
        assert np.array_equal(y, want), np.max(np.abs(y - want))


# The streaming kernel walks 16-row tiles (up to 8 per persistent workgroup)
# over column slabs of at most 64 groups.  These layers take two or three
# slabs with 1 to 4 tiles per workgroup (odd and even counts), or one slab
# (n <= 4096) with 2 to 5 tiles per workgroup.  Sampled rows include the
# whole last row block.
@pytest.mark.parametrize("K,m,n", [(2, 4200, 8320), (3, 8400, 8320), (1, 12400, 16512),
                                   (4, 4300, 8320), (2, 12000, 4096), (3, 16384, 4096),
                                   (3, 16400, 4096), (1, 5000, 2048)])
def test_gemv_stream_slabs_exact(K, m, n):
    say(f"gemv stream slabs m={m} n={n} K={K}")
    S = syn.random_signs(K, m, n, seed=m + n + K)
    A = syn.exact_alpha(K, m, n // 128, seed=m + 3 * K).astype(np.float16)
    x = syn.exact_activations(1, n, seed=n + 5 * K)[0]
    d, packed = pack_on_gpu(S, A, "f16")
    y = gemv(d, packed, x, "bf16", guard=17)
    rows = np.unique(np.r_[np.arange(0, m, 13), np.arange(m - 70, m)])
    want = oracle.product(S[:, rows], A[:, rows], x)
    assert np.array_equal(y[rows], want), np.max(np.abs(y[rows] - want))


def test_gemv_one_hot_and_all_ones(gemv_variant):
    say(f"gemv one-hot {gemv_variant}")
    K, m, n = 3, 70, 384
    S = syn.random_signs(K, m, n, seed=5)
    A = syn.exact_alpha(K, m, 3, seed=6).astype(np.float16)
    d, packed = pack_on_gpu(S, A, "f16")
    for j in (0, 1, 4, 31, 32, 127, 128, 200, 383):
        x = np.zeros(n, dtype=np.float32)
        x[j] = 1.0
        y = gemv(d, packed, x, "bf16")
        want = np.array([sum(float(A[k, i, j // 128]) * int(S[k, i, j]) for k in range(K))
                         for i in range(m)])
        assert np.array_equal(y, want), j
    for g in range(3):
        x = np.zeros(n, dtype=np.float32)
        x[128 * g:128 * g + 128] = 1.0
        y = gemv(d, packed, x, "bf16")
        want = [sum(float(A[k, i, g]) * (2 * int(np.count_nonzero(S[k, i, 128 * g:128 * g + 128] > 0)) - 128)
                    for k in range(K)) for i in range(m)]
        assert np.array_equal(y, np.array(want)), g


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_gemv_workloads_tolerance(cfg):
    """Full pipeline on the device (quantize, pack, gemv) at the workload
    shapes; the oracle quantizes and multiplies sampled rows on its own."""
    w = syn.WORKLOADS[cfg]
    dt, xdt = w["alpha_dtype"], w["x_dtype"]
    for li, (name, m, n) in enumerate(w["linears"]):
        say(f"gemv config {cfg} {name} {m}x{n} K={w['K']}")
        W = syn.weight(m, n, syn.weight_seed(cfg, li))
        x = syn.activations(1, n, syn.act_seed(cfg, li), xdt)[0]
        d, signs, alpha, packed, flag = quantize_on_gpu(W, w["K"], dt)
        del signs, alpha
        y = gemv(d, packed, x, xdt, guard=5)
        rows = sample_rows(m, 256, li)
        S, A, _ = oracle.residual_binarize(W[rows], w["K"], alpha_dtype=dt)
        want, E = oracle.product(S, A, x), oracle.bound(S, A, x)
        ratio = oracle.max_error_ratio(y[rows], want, E)
        assert ratio <= TOL, (name, ratio)
        # determinism: a second call gives the same bits
        y2 = gemv(d, packed, x, xdt)
        assert np.array_equal(y, y2)
        del packed
        torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("K", [1, 2, 3])
def test_gemv_k_sweep_first_linear(cfg, K):
    w = syn.WORKLOADS[cfg]
    dt = w["alpha_dtype"]
    xdt = w["x_dtype"]
    name, m, n = w["linears"][0]
    say(f"gemv K sweep config {cfg} {name} K={K}")
    W = syn.weight(m, n, syn.weight_seed(cfg, 0))
    x = syn.activations(1, n, syn.act_seed(cfg, 0), xdt)[0]
    d, signs, alpha, packed, flag = quantize_on_gpu(W, K, dt)
    y = gemv(d, packed, x, xdt)
    rows = sample_rows(m, 128, 100 + K)
    S, A, _ = oracle.residual_binarize(W[rows], K, alpha_dtype=dt)
    ratio = oracle.max_error_ratio(y[rows], oracle.product(S, A, x), oracle.bound(S, A, x))
    assert ratio <= TOL, ratio


def test_gemv_workspace_shared_across_shapes_and_garbage():
    """The column-split kernel: one workspace serves every shape, whatever it
    holds beforehand; the default kernel asks for none."""
    say("gemv shared workspace")
    shapes = [(4096, 4096, 2), (300, 11008, 3), (11008, 4096, 3), (64, 13824, 1)]
    assert all(bw.mbok_gemv_workspace_bytes(bw.mbok_desc_init(m, n, K, bw.MBOK_F16)) == 0
               for m, n, K in shapes)
    old = _swap_env({"MBOK_GEMV_VARIANT": "split"})
    try:
        need = max(bw.mbok_gemv_workspace_bytes(bw.mbok_desc_init(m, n, K, bw.MBOK_F16))
                   for m, n, K in shapes)
        assert need > 0
        ws = torch.full((need + 4096,), 0x7f, dtype=torch.uint8, device=DEV)
        for rep in range(2):
            for (m, n, K) in shapes:
                S = syn.random_signs(K, m, n, seed=m + n)
                A = syn.exact_alpha(K, m, n // 128, seed=K).astype(np.float16)
                x = syn.exact_activations(1, n, seed=n)[0]
                d, packed = pack_on_gpu(S, A, "f16")
                y = torch.empty(m, dtype=torch.float32, device=DEV)
                bw.mbok_gemv(d, packed, x_to_dev(x, "bf16"), y, workspace=ws)
                assert np.array_equal(y.cpu().numpy().astype(np.float64),
                                      oracle.product(S, A, x)), (m, n, K)
    finally:
        _restore_env(old)


def test_gemv_without_workspace_matches():
    say("gemv without workspace")
    K, m, n = 3, 500, 4096
    S = syn.random_signs(K, m, n, seed=3)
    A = syn.exact_alpha(K, m, n // 128, seed=4).astype(np.float16)
    x = syn.exact_activations(1, n, seed=5)[0]
    d, packed = pack_on_gpu(S, A, "f16")
    y = torch.empty(m, dtype=torch.float32, device=DEV)
    bw.mbok_gemv(d, packed, x_to_dev(x, "bf16"), y, workspace=None)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.product(S, A, x))


def test_gemv_config1_full_oracle():
    """Config 1 is small enough for the oracle to do every row."""
    say("gemv config 1 full")
    w = syn.WORKLOADS[1]
    W = syn.weight(256, 512, syn.weight_seed(1))
    x = syn.activations(1, 512, syn.act_seed(1), "f32")[0]
    S, A, _ = oracle.residual_binarize(W, 2, alpha_dtype="f32")
    d, signs, alpha, packed, flag = quantize_on_gpu(W, 2, "f32")
    y = gemv(d, packed, x, "f32")
    assert oracle.max_error_ratio(y, oracle.product(S, A, x), oracle.bound(S, A, x)) <= TOL


# ---------------------------------------------------------- multi-token GEMM

@pytest.mark.parametrize("T", [1, 3, 4, 16, 17, 40])
@pytest.mark.parametrize("K", [1, 2, 3])
def test_gemm_exact_regime(T, K):
    m, n = 130, 512
    say(f"gemm exact T={T} K={K}")
    S = syn.random_signs(K, m, n, seed=T * 10 + K)
    A = syn.exact_alpha(K, m, n // 128, seed=T + K).astype(np.float16)
    X = syn.exact_activations(T, n, seed=T + 50 * K)
    d, packed = pack_on_gpu(S, A, "f16")
    Y = gemm(d, packed, X, ldx=n + 8, ldy=m + 3)
    assert np.array_equal(Y, oracle.product(S, A, X))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("T,m,n", [(2, 1, 128), (5, 65, 384), (8, 130, 1152), (16, 200, 640),
                                   (13, 64, 2048), (3, 65, 5120), (16, 70, 11008),
                                   (5, 4160, 128)])
@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_gemm_skinny_exact(T, m, n, K, dt, skinny_shape):
    """Few-token kernel in the exact regime (integer x, power-of-two scales):
    every launch shape gives the fp64 definition bit for bit, including
    ragged rows, uneven group ranges and row/column leading dimensions."""
    say(f"gemm skinny exact T={T} m={m} n={n} K={K} {dt} {skinny_shape}")
    S = syn.random_signs(K, m, n, seed=T * 7 + m + K)
    A = syn.exact_alpha(K, m, n // 128, seed=T + 3 * K).astype(np_alpha(dt))
    X = syn.exact_activations(T, n, seed=T * 5 + K)
    d, packed = pack_on_gpu(S, A, dt)
    Y = gemm(d, packed, X, ldx=n + 24, ldy=m + 7)
    assert np.array_equal(Y, oracle.product(S, A, X))


def test_gemm_skinny_matches_fp64_closely():
    """Random (non-exact) bf16 activations and fp16 scales: the few-token
    kernel rounds nothing but the fp32 accumulation, so its error stays below
    1% of the 1e-3 tolerance; rounding W_hat to bf16 (2^-9 relative, random
    signs over n = 4096 columns) would land near 10% of it."""
    T, m, n, K = 16, 512, 4096, 3
    say("gemm skinny closeness")
    W = syn.weight(m, n, 77)
    X = syn.activations(T, n, 78, "bf16")
    d, signs, alpha, packed, flag = quantize_on_gpu(W, K, "f16")
    del signs, alpha
    Y = gemm(d, packed, X)
    S, A, _ = oracle.residual_binarize(W, K, alpha_dtype="f16")
    ratio = oracle.max_error_ratio(Y, oracle.product(S, A, X), oracle.bound(S, A, X))
    assert ratio <= 1e-2 * TOL, ratio


@pytest.mark.parametrize("K", [1, 2, 3])
@pytest.mark.parametrize("T", [4, 16])
def test_gemm_config3_tolerance(T, K):
    w = syn.WORKLOADS[3]
    for li, (name, m, n) in enumerate(w["linears"]):
        say(f"gemm config 3 {name} T={T} K={K}")
        W = syn.weight(m, n, syn.weight_seed(3, li))
        X = syn.activations(T, n, syn.act_seed(3, li), "bf16")
        d, signs, alpha, packed, flag = quantize_on_gpu(W, K, "f16")
        del signs, alpha
        Y = gemm(d, packed, X)
        rows = sample_rows(m, 128, li)
        S, A, _ = oracle.residual_binarize(W[rows], K, alpha_dtype="f16")
        ratio = oracle.max_error_ratio(Y[:, rows], oracle.product(S, A, X), oracle.bound(S, A, X))
        assert ratio <= TOL, (name, ratio)


PREFILL_VARIANTS = {
    "8": {"MBOK_GEMM_WAVES": "8"},
    "8_token_order": {"MBOK_GEMM_WAVES": "8", "MBOK_GEMM_ORDER": "token"},
    "4": {"MBOK_GEMM_WAVES": "4"},
}


@pytest.fixture(params=list(PREFILL_VARIANTS))
def prefill_waves(request):
    """Prefill kernel with 8 wavefronts per workgroup (default; XCD-blocked
    or token-major tile order) or 4."""
    keys = ("MBOK_GEMM_WAVES", "MBOK_GEMM_ORDER")
    old = {k: os.environ.get(k) for k in keys}
    for k in keys:
        os.environ.pop(k, None)
    os.environ.update(PREFILL_VARIANTS[request.param])
    yield request.param
    for k, v in old.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("T,m,n", [(2, 65, 128), (33, 300, 384), (257, 256, 256), (300, 513, 640)])
def test_gemm_prefill_exact_ragged(T, m, n, K, prefill_waves):
    say(f"gemm prefill exact T={T} m={m} n={n} K={K}")
    S = syn.random_signs(K, m, n, seed=T + m + K)
    A = syn.exact_alpha(K, m, n // 128, seed=T + K).astype(np.float16)
    X = syn.exact_activations(T, n, seed=T * 3 + K)
    d, packed = pack_on_gpu(S, A, "f16")
    Y = gemm(d, packed, X, ldx=n + 16, ldy=m + 5)
    assert np.array_equal(Y, oracle.product(S, A, X))


def test_gemm_prefill_exact_whole_and_half_tiles(prefill_waves):
    """More 256 x 256 tiles than compute units (20 x 13 = 260 tiles on 256):
    the last round's tiles run as 128-row halves; exact regime, every element."""
    T, m, n, K = 3328, 5120, 256, 3
    say("gemm prefill whole and half tiles")
    S = syn.random_signs(K, m, n, seed=91)
    A = syn.exact_alpha(K, m, n // 128, seed=92).astype(np.float16)
    X = syn.exact_activations(T, n, seed=93)
    d, packed = pack_on_gpu(S, A, "f16")
    Y = gemm(d, packed, X)
    assert np.array_equal(Y, oracle.product(S, A, X))


def test_gemm_maximum_tokens():
    """T = MBOK_MAX_T tokens, every element (exact regime).  With ldx = n the
    activation offsets fit in 32 bits and the 8-wavefront kernel runs; with
    ldx = 65536, T * ldx reaches 2^32 elements (an 8 GiB activation buffer)
    and the kernel with 64-bit offsets runs instead."""
    K, m, n = 2, 70, 256
    T = bw.MBOK_MAX_T
    say(f"gemm maximum tokens T={T} m={m} n={n} K={K}")
    S = syn.random_signs(K, m, n, seed=61)
    A = syn.exact_alpha(K, m, n // 128, seed=62).astype(np.float16)
    X = syn.exact_activations(T, n, seed=63)
    want = oracle.product(S, A, X)
    d, packed = pack_on_gpu(S, A, "f16")
    Xn = x_to_dev(X, "bf16")
    for ldx in (n, 65536):
        say(f"gemm maximum tokens ldx={ldx}")
        if ldx == n:
            Xd = Xn
        else:
            Xd = torch.zeros((T, ldx), dtype=torch.bfloat16, device=DEV)
            Xd[:, :n] = Xn
        Y = torch.full((T, m), -777.25, dtype=torch.float32, device=DEV)
        bw.mbok_gemm(d, packed, Xd, Y)
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), want), ldx
        del Xd, Y
    torch.cuda.empty_cache()


def test_maximum_rows():
    """m = 2^24 rows (the maximum), n = 128, K = 1, exact regime, through the
    decode (T = 1), few-token (T = 2: two tokens per matrix-core product;
    T = 4: one product per group; T = 7: bf16 +-1) and prefill (T = 17)
    kernels: sampled
    rows (every 4099th and the last 70) against the oracle, and no output
    left unwritten.  This runs the tile and chunk index arithmetic over its
    whole range."""
    K, m, n = 1, 1 << 24, 128
    say(f"maximum rows m={m} n={n} K={K}")
    S = syn.random_signs(K, m, n, seed=71)
    A = syn.exact_alpha(K, m, n // 128, seed=72).astype(np.float16)
    d, packed = pack_on_gpu(S, A, "f16")
    rows = np.unique(np.r_[np.arange(0, m, 4099), np.arange(m - 70, m)])
    Ss, As = S[:, rows].copy(), A[:, rows].copy()
    del S
    rows_t = torch.from_numpy(rows).to(DEV)
    canary = -777.25  # |y| <= 128 * 8 * 2^-4 in this regime, so never equal
    for T in (1, 2, 4, 7, 17):
        say(f"maximum rows T={T}")
        X = syn.exact_activations(T, n, seed=73 + T)
        Xd = x_to_dev(X, "bf16")
        Y = torch.full((T, m), canary, dtype=torch.float32, device=DEV)
        if T == 1:
            bw.mbok_gemv(d, packed, Xd[0], Y[0])
        else:
            bw.mbok_gemm(d, packed, Xd, Y)
        assert not bool((Y == canary).any()), T
        got = Y[:, rows_t].cpu().numpy().astype(np.float64)
        assert np.array_equal(got, oracle.product(Ss, As, X)), T
        del Y
    torch.cuda.empty_cache()


def test_gemm_identity_activations_give_the_weights(prefill_waves):
    """X = identity rows (T = n) in the exact regime: Y = W_hat^T exactly,
    which pins the operand orientation, k order and bf16 rounding of W_hat."""
    say("gemm identity")
    K, m, n = 3, 200, 384
    S = syn.random_signs(K, m, n, seed=41)
    A = syn.exact_alpha(K, m, n // 128, seed=42).astype(np.float16)
    d, packed = pack_on_gpu(S, A, "f16")
    Y = gemm(d, packed, np.eye(n, dtype=np.float32))
    assert np.array_equal(Y, oracle.dequantize(S, A).T)


def test_gemm_prefill_config5_tolerance(prefill_waves):
    """Config 5 at full size (11008 x 4096, K = 3, 2048 tokens) on the device;
    the oracle quantizes and multiplies sampled output rows for every token."""
    w = syn.WORKLOADS[5]
    name, m, n = w["linears"][0]
    T = w["T"][0]
    say(f"gemm config 5 {m}x{n} T={T}")
    W = syn.weight(m, n, syn.weight_seed(5))
    X = syn.activations(T, n, syn.act_seed(5), "bf16")
    d, signs, alpha, packed, flag = quantize_on_gpu(W, 3, "f16")
    del signs, alpha
    Y = gemm(d, packed, X)
    rows = sample_rows(m, 128, 5)
    S, A, _ = oracle.residual_binarize(W[rows], 3, alpha_dtype="f16")
    ratio = oracle.max_error_ratio(Y[:, rows], oracle.product(S, A, X), oracle.bound(S, A, X))
    assert ratio <= TOL, ratio
    # determinism
    Y2 = gemm(d, packed, X)
    assert np.array_equal(Y, Y2)


@pytest.mark.parametrize("K", [1, 2])
def test_gemm_prefill_config5_k_sweep(K):
    """Config 5's shape (11008 x 4096, 2048 tokens) with K = 1 and 2 kernels
    through the default prefill kernel; sampled rows for every token."""
    w = syn.WORKLOADS[5]
    name, m, n = w["linears"][0]
    T = w["T"][0]
    say(f"gemm config 5 {m}x{n} T={T} K={K}")
    W = syn.weight(m, n, syn.weight_seed(5))
    X = syn.activations(T, n, syn.act_seed(5), "bf16")
    d, signs, alpha, packed, flag = quantize_on_gpu(W, K, "f16")
    del signs, alpha
    Y = gemm(d, packed, X)
    rows = sample_rows(m, 128, 50 + K)
    S, A, _ = oracle.residual_binarize(W[rows], K, alpha_dtype="f16")
    ratio = oracle.max_error_ratio(Y[:, rows], oracle.product(S, A, X), oracle.bound(S, A, X))
    assert ratio <= TOL, ratio
