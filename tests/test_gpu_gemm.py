"""GPU parity of the projection GEMM (isd_gemm) at the Qwen3-8B decode shapes and at edge
shapes, against float64 dot products of the same bf16 / fp32 values on sampled outputs.

Tolerance (bf16 path): |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), i.e. the bf16 rounding of
the stored output plus fp32 accumulation error; fp32 outputs: 1e-4 rms(ref) relative.
Row invariance: the rows a smaller batch shares with a larger one come out bit-identical.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rand(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV, dtype=torch.float32) * scale).to(dtype)


def _pk(W):
    """bf16 weights go to the library in the packed operand layout."""
    from strided_decoding_amd import pack_weight
    return pack_weight(W) if W.dtype == torch.bfloat16 else W


def _ref(X, W, rows, cols):
    x = X.float().cpu().numpy().astype(np.float64)
    w = W.float().cpu().numpy().astype(np.float64)
    return np.einsum("ik,ik->i", x[rows], w[cols])


def _pick(M, N, n, seed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([[0, M - 1], rng.integers(0, M, n)])
    cols = np.concatenate([[0, N - 1], rng.integers(0, N, n)])
    return rows, cols


def _check(got, ref, bf16=True):
    rms = np.sqrt(np.mean(ref ** 2)) + 1e-12
    tol = (2.0 ** -7) * np.abs(ref) + 1e-3 * rms if bf16 else 1e-4 * rms
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (np.abs(got - ref)[bad][:5], ref[bad][:5])


SHAPES_8B = [("qkv", 448, 6144, 4096), ("o", 448, 4096, 4096), ("down", 448, 4096, 12288),
             ("lm_head", 448, 151936, 4096)]
# the 32B shape: 64 x 128 query heads and 8 KV heads over d_model 5120, d_ffn 25600
SHAPES_32B = [("qkv", 448, 10240, 5120), ("o", 448, 5120, 8192), ("down", 448, 5120, 25600),
              ("qkv", 112, 10240, 5120), ("down", 112, 5120, 25600)]


@pytest.mark.parametrize("name,M,N,K", SHAPES_8B + SHAPES_32B)
def test_gemm_decode_shapes(name, M, N, K):
    from strided_decoding_amd import gemm
    print(f"gemm {name} {M}x{N}x{K}", flush=True)
    X = _rand((M, K), 1, 1.0)
    W = _rand((N, K), 2, 0.02)
    Y = gemm(X, _pk(W), "store_f32" if name == "lm_head" else "store")
    torch.cuda.synchronize()
    rows, cols = _pick(M, N, 400, 3)
    got = Y.float().cpu().numpy()[rows, cols]
    _check(got, _ref(X, W, rows, cols), bf16=(name != "lm_head"))


@pytest.mark.parametrize("M,F,K", [(448, 12288, 4096), (448, 25600, 5120)])
def test_gemm_swiglu_and_residual(M, F, K):
    from strided_decoding_amd import gemm
    X = _rand((M, K), 4, 1.0)
    Wg = _rand((F, K), 5, 0.02)
    Wu = _rand((F, K), 6, 0.02)
    H = gemm(X, _pk(Wg), "swiglu", W2=_pk(Wu))
    torch.cuda.synchronize()
    rows, cols = _pick(M, F, 400, 7)
    g = _ref(X, Wg, rows, cols)
    u = _ref(X, Wu, rows, cols)
    _check(H.float().cpu().numpy()[rows, cols], g / (1 + np.exp(-g)) * u)
    # residual: R += X W^T in fp32
    Wd = _rand((K, F), 8, 0.02)
    R0 = _rand((M, K), 9, 1.0, torch.float32)
    R = R0.clone()
    gemm(H, _pk(Wd), "resid", R=R)
    torch.cuda.synchronize()
    rows, cols = _pick(M, K, 400, 10)
    ref = R0.cpu().numpy().astype(np.float64)[rows, cols] + _ref(H, Wd, rows, cols)
    _check(R.cpu().numpy()[rows, cols], ref, bf16=False)


@pytest.mark.parametrize("M,N,K,splits", [(1, 256, 32, 0), (225, 4100, 96, 0), (64, 512, 4096, 8),
                                          (700, 1024, 1024, 2), (448, 128, 4096, 8), (3, 4, 64, 1)])
def test_gemm_edge_shapes(M, N, K, splits):
    from strided_decoding_amd import gemm
    X = _rand((M, K), 11, 1.0)
    W = _rand((N, K), 12, 0.05)
    Y = gemm(X, _pk(W), "store_f32", splits=splits)
    torch.cuda.synchronize()
    ref = X.double() @ W.double().T
    err = (Y.double() - ref).abs().max().item()
    assert err <= 1e-4 * ref.abs().max().item(), err


def test_gemm_row_invariance():
    """Rows shared by a 64-row and a 448-row call come out bit-identical (same split rule)."""
    from strided_decoding_amd import gemm
    K, N = 4096, 6144
    X = _rand((448, K), 13, 1.0)
    W = _rand((N, K), 14, 0.02)
    Wp = _pk(W)
    big = gemm(X, Wp, "store")
    small = gemm(X[:64].contiguous(), Wp, "store")
    one = gemm(X[5:6].contiguous(), Wp, "store")
    torch.cuda.synchronize()
    assert torch.equal(big[:64], small)
    assert torch.equal(big[5:6], one)


@pytest.mark.parametrize("splits", [0, 1])
def test_gemm_residual_with_fused_rmsnorm(splits):
    """R += H Wd^T, then y = RMSNorm(R) * g (fused into the split-K reduction when split)."""
    from strided_decoding_amd import gemm
    M, d, F = 448, 4096, 12288
    H = _rand((M, F), 17, 1.0)
    Wd = _rand((d, F), 18, 0.02)
    R0 = _rand((M, d), 19, 1.0, torch.float32)
    g = (1.0 + 0.1 * _rand((d,), 20, 1.0, torch.float32)).to(torch.bfloat16)
    R = R0.clone()
    y = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    gemm(H, _pk(Wd), "resid", R=R, splits=splits, norm_g=g, norm_out=y, norm_eps=1e-6)
    torch.cuda.synchronize()
    rows, cols = _pick(M, d, 400, 21)
    ref = R0.cpu().numpy().astype(np.float64)[rows, cols] + _ref(H, Wd, rows, cols)
    _check(R.cpu().numpy()[rows, cols], ref, bf16=False)
    Rg = R.double().cpu().numpy()
    yref = Rg / np.sqrt((Rg ** 2).mean(axis=1, keepdims=True) + 1e-6) * g.double().cpu().numpy()
    _check(y.float().cpu().numpy().ravel(), yref.ravel())


@pytest.mark.parametrize("M", [7, 200])
@pytest.mark.parametrize("S,K", [(3, 1536), (5, 1280), (6, 1536), (12, 1536), (16, 2048)])
def test_gemm_split_counts(M, S, K):
    """Split counts that are not powers of two, and the largest (16), on the skinny (7 rows) and
    tiled (200 rows) kernels: the ordered reductions (plain, the SwiGLU pair, residual + RMSNorm)
    issue the split loads together in a group of the next power of two, the slots past S
    re-reading the last split and left out of the sum."""
    from strided_decoding_amd import gemm
    print(f"gemm splits S={S} M={M} K={K}", flush=True)
    N = 512
    X = _rand((M, K), 60 + S, 1.0)
    W = _rand((N, K), 61, 0.05)
    W2 = _rand((N, K), 62, 0.05)
    Wp, W2p = _pk(W), _pk(W2)
    Y = gemm(X, Wp, "store_f32", splits=S)
    torch.cuda.synchronize()
    ref = X.double() @ W.double().T
    assert (Y.double() - ref).abs().max().item() <= 1e-4 * ref.abs().max().item()
    H = gemm(X, Wp, "swiglu", W2=W2p, splits=S)
    torch.cuda.synchronize()
    rows, cols = _pick(M, N, 300, 63)
    g, u = _ref(X, W, rows, cols), _ref(X, W2, rows, cols)
    _check(H.float().cpu().numpy()[rows, cols], g / (1 + np.exp(-g)) * u)
    R0 = _rand((M, N), 64, 1.0, torch.float32)
    R = R0.clone()
    gn = (1.0 + 0.1 * _rand((N,), 65, 1.0, torch.float32)).to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    gemm(X, Wp, "resid", R=R, splits=S, norm_g=gn, norm_out=y, norm_eps=1e-6)
    torch.cuda.synchronize()
    Rref = R0.double() + ref
    assert (R.double() - Rref).abs().max().item() <= 1e-4 * Rref.abs().max().item()
    Rg = R.double().cpu().numpy()
    yref = Rg / np.sqrt((Rg ** 2).mean(axis=1, keepdims=True) + 1e-6) * gn.double().cpu().numpy()
    _check(y.float().cpu().numpy().ravel(), yref.ravel())


SKINNY_ROWS = [1, 7, 28, 32, 33, 56, 64, 65, 112, 128]


@pytest.mark.parametrize("M", SKINNY_ROWS)
@pytest.mark.parametrize("mode,N,K", [("store", 6144, 4096), ("store_f32", 2048, 4096), ("resid", 4096, 4096),
                                      ("swiglu", 1536, 4096), ("resid", 512, 12288), ("store", 200, 96)])
def test_skinny_path_bit_identical_to_tiled(M, mode, N, K):
    """The two bf16 kernels accumulate every output in the same order: bit-identical results."""
    from strided_decoding_amd import gemm
    print(f"skinny vs tiled {mode} M={M} N={N} K={K}", flush=True)
    X = _rand((M, K), 30 + M, 1.0)
    W = _rand((N, K), 31, 0.02)
    W2 = _rand((N, K), 32, 0.02) if mode == "swiglu" else None
    outs = []
    for path in ("tiled", "skinny"):
        if mode == "resid":
            R = _rand((M, N), 33, 1.0, torch.float32)
            outs.append(gemm(X, _pk(W), mode, R=R, path=path))
        else:
            outs.append(gemm(X, _pk(W), mode, W2=None if W2 is None else _pk(W2), path=path))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    if M in (7, 56, 112):
        rows, cols = _pick(M, N, 300, 34)
        ref = _ref(X, W, rows, cols)
        if mode == "swiglu":
            u = _ref(X, W2, rows, cols)
            ref = ref / (1 + np.exp(-ref)) * u
        if mode == "resid":
            ref = ref + _rand((M, N), 33, 1.0, torch.float32).cpu().numpy().astype(np.float64)[rows, cols]
        _check(outs[1].float().cpu().numpy()[rows, cols], ref, bf16=mode in ("store", "swiglu"))


@pytest.mark.parametrize("M", [224, 300, 448])
@pytest.mark.parametrize("mode,N,K", [("swiglu", 12288, 4096), ("store", 6144, 4096), ("resid", 4096, 12288),
                                      ("store_f32", 2048, 4096), ("store", 200, 96)])
def test_tiled_wave_counts_bit_identical(M, mode, N, K):
    """The tiled kernel with 4, 3 or 2 waves per workgroup (and the automatic choice) runs the
    same per-wave pipeline over different column groupings: bit-identical results, and the
    8B gate/up product (the one the automatic choice runs with 3 waves at 448 rows) on sampled
    outputs against fp64."""
    from strided_decoding_amd import gemm
    print(f"tiled wave counts {mode} M={M} N={N} K={K}", flush=True)
    X = _rand((M, K), 40 + M, 1.0)
    W = _rand((N, K), 41, 0.02)
    W2 = _rand((N, K), 42, 0.02) if mode == "swiglu" else None
    Wp, W2p = _pk(W), None if W2 is None else _pk(W2)
    outs = []
    for path in ("tiled4", "tiled3", "tiled2", "auto"):
        if mode == "resid":
            R = _rand((M, N), 43, 1.0, torch.float32)
            outs.append(gemm(X, Wp, mode, R=R, path=path))
        else:
            outs.append(gemm(X, Wp, mode, W2=W2p, path=path))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0], o)
    if mode == "swiglu" and M == 448:
        rows, cols = _pick(M, N, 300, 44)
        g, u = _ref(X, W, rows, cols), _ref(X, W2, rows, cols)
        _check(outs[1].float().cpu().numpy()[rows, cols], g / (1 + np.exp(-g)) * u)


@pytest.mark.parametrize("splits", [0, 1])
def test_skinny_fused_rmsnorm_and_row_gather(splits):
    """Skinny path with the fused residual + RMSNorm, and equal to the tiled path bit for bit."""
    from strided_decoding_amd import gemm
    M, d, F = 56, 4096, 12288
    H = _rand((M, F), 40, 1.0)
    Wd = _rand((d, F), 41, 0.02)
    g = (1.0 + 0.1 * _rand((d,), 42, 1.0, torch.float32)).to(torch.bfloat16)
    res = []
    for path in ("tiled", "skinny"):
        R = _rand((M, d), 43, 1.0, torch.float32)
        y = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
        gemm(H, _pk(Wd), "resid", R=R, splits=splits, norm_g=g, norm_out=y, norm_eps=1e-6, path=path)
        res.append((R, y))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_gemm_fp32_path():
    from strided_decoding_amd import gemm
    X = _rand((37, 200), 15, 1.0, torch.float32)
    W = _rand((300, 200), 16, 0.1, torch.float32)
    Y = gemm(X, W, "store")
    torch.cuda.synchronize()
    ref = X.double() @ W.double().T
    assert (Y.double() - ref).abs().max().item() <= 1e-5 * ref.abs().max().item()


@pytest.mark.parametrize("rows,cols", [(1, 16), (33, 48), (64, 4096), (200, 96)])
def test_pack_weights_layout(rows, cols):
    """The packed operand layout: block (nb, kb), lane l holds row 32 nb + l%32, k = 16 kb +
    8 (l/32) .. + 7; rows padded with zeros to a multiple of 32."""
    from strided_decoding_amd import pack_weight
    W = _rand((rows, cols), 50 + rows, 1.0)
    got = pack_weight(W).data.view(torch.int16).cpu().numpy()
    w = W.view(torch.int16).cpu().numpy()
    rp = -(-rows // 32) * 32
    wp = np.zeros((rp, cols), np.int16)
    wp[:rows] = w
    want = wp.reshape(rp // 32, 32, cols // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert np.array_equal(got, want)
