"""GPU parity of the decoded-weight matmul (needs an MI355X).

qamw_rotate_activations against the oracle's rotation rounded to bf16: the
GPU rotates in fp32 and rounds once, so it can land on the other bf16
neighbour only when a rounding midpoint lies between its value and the fp64
one; every element must be within one bf16 ulp and at least 99.9% identical.

qamw_decode_matmul against the oracle's decode-then-multiply in fp64.  The
GPU multiplies bf16-rounded operands (rotated activations and looked-up
pairs, each within 2^-9 relative) and accumulates in fp32, so each output
is within 2^-7 * S of the exact value, S[t][n] = rho^_n sum_k |Xr[t][k]
y^_n[k]| (the bound of two 2^-9 roundings with margin for fp32 sums).
"""
import sys
import zlib

import numpy as np
import pytest

import workloads
from oracle import qamw_ref as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vector_codebook_codec_amd as pkg
    from vector_codebook_codec_amd import _lib

    _lib.load()
    return pkg


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-38)))
    return 2.0 ** (e - 7)


def encode_gpu(q, W, r, alpha, b, seed, C, wdtype="f32"):
    Wt = torch.from_numpy(W).to(DEV)
    if wdtype == "bf16":
        Wt = Wt.to(torch.bfloat16)
    s, sigma = q.qamw_calibrate(Wt, torch.from_numpy(r).to(DEV), alpha, b, seed)
    Ct = torch.from_numpy(C).to(DEV)
    packed, rn = q.qamw_encode(Wt, s, sigma, b, seed, Ct, plan=q.qamw_build_plan(Ct))
    torch.cuda.synchronize()
    return dict(s=s, sigma=sigma, C=Ct, packed=packed, rn=rn)


def check_matmul(q, X, g, b, seed, C, d, rows=None, use_s=True, out_dtype=torch.float32):
    Xt = torch.from_numpy(X).to(DEV)
    s = g["s"] if use_s else None
    Xr = q.qamw_rotate_activations(Xt, s, b, seed)
    Y = q.qamw_decode_matmul(Xr, g["packed"], g["rn"], g["sigma"], g["C"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    packed = g["packed"].cpu().numpy().view(np.uint32)
    rn = g["rn"].cpu().numpy().view(np.uint16)
    if rows is None:
        rows = np.arange(packed.shape[0])
    s_np = g["s"].cpu().numpy() if use_s else None
    sig = g["sigma"].cpu().numpy()
    Yref = O.decode_matmul(X, packed[rows], rn[rows], s_np, sig, b, seed, C, d)
    Xr_ex = O.rotate_activations(X, s_np, b, seed)
    Yh = O.lookup_pairs(packed[rows], sig, C, d)
    S = (np.abs(Xr_ex) @ np.abs(Yh).T) * O.f16_bits_to_f64(rn[rows])[None, :]
    got = Y[:, torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - Yref)
    tol = 2.0 ** -7 * S
    if out_dtype == torch.bfloat16:
        tol = tol + 0.5 * bf16_ulp(Yref) * (1 + 2.0 ** -7)
    worst = float(np.max(err / np.maximum(S, 1e-300)))
    say(f"  T={X.shape[0]} rows={len(rows)}: max |err|/S = {worst:.3e}, "
        f"rel rms {float(np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(Yref ** 2))):.3e}")
    assert np.all(err <= tol + 1e-30)
    return Y, Xr


@pytest.mark.parametrize("T,d,b,wdtype", [(5, 512, 128, "f32"), (3, 1088, 64, "bf16"), (2, 96, 32, "f32")])
def test_rotate_activations(q, T, d, b, wdtype):
    rng = np.random.default_rng(T * 1000 + d)
    X = rng.standard_normal((T, d)).astype(np.float32)
    s = rng.lognormal(0, 0.7, d).astype(np.float32)
    Xt = torch.from_numpy(X).to(DEV)
    if wdtype == "bf16":
        Xt = Xt.to(torch.bfloat16)
        X = Xt.float().cpu().numpy()
    Xr = q.qamw_rotate_activations(Xt, torch.from_numpy(s).to(DEV), b, 77)
    torch.cuda.synchronize()
    ref = O.rotate_activations(X.astype(np.float64), s.astype(np.float64), b, 77)
    got_bits = Xr.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_bits = O.to_bf16_bits(ref)
    same = float((got_bits == ref_bits).mean())
    got = O.bf16_bits_to_f64(got_bits)
    say(f"case rotate T={T} d={d} b={b} {wdtype}: identical {same:.5f}")
    assert np.all(np.abs(got - ref) <= bf16_ulp(ref) * 1.0001)
    assert same >= 0.999


@pytest.mark.parametrize("N,d,b,K,T", [
    (37, 512, 128, 256, 1), (37, 512, 128, 256, 16), (16, 1088, 64, 2048, 17), (20, 96, 32, 16, 40),
    (9, 48, 16, 4, 65), (33, 3072, 256, 4096, 64), (8, 2048, 1024, 1024, 7),
    # one token (the GEMV kernel): B = 12, a ragged single slice with B = 2, B = 10,
    # more slices than wavefronts (d / 2 = 18432 pairs = 36 slices of 512)
    (33, 3072, 256, 4096, 1), (9, 48, 16, 4, 1), (8, 2048, 1024, 1024, 1), (5, 36864, 256, 256, 1),
])
def test_decode_matmul_shapes(q, N, d, b, K, T):
    rng = np.random.default_rng(N * 7 + d + T)
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    r = rng.lognormal(0, 1.0, d).astype(np.float32)
    C = q.load_codebook(K)
    g = encode_gpu(q, W, r, 0.5, b, 11, C)
    X = rng.standard_normal((T, d)).astype(np.float32)
    say(f"case matmul N={N} d={d} b={b} K={K} T={T}")
    check_matmul(q, X, g, b, 11, C, d)


def test_decode_matmul_without_s_and_bf16_out(q):
    rng = np.random.default_rng(5)
    N, d, b, K = 24, 768, 256, 256
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    r = rng.lognormal(0, 1.0, d).astype(np.float32)
    C = q.load_codebook(K)
    g = encode_gpu(q, W, r, 0.5, b, 3, C)
    X = rng.standard_normal((10, d)).astype(np.float32)
    say("case matmul s=None")
    check_matmul(q, X, g, b, 3, C, d, use_s=False)
    say("case matmul bf16 out")
    check_matmul(q, X, g, b, 3, C, d, out_dtype=torch.bfloat16)
    say("case matmul one token, s=None and bf16 out")
    check_matmul(q, X[:1], g, b, 3, C, d, use_s=False)
    check_matmul(q, X[:1], g, b, 3, C, d, out_dtype=torch.bfloat16)


def test_decode_matmul_full_size_sampled(q):
    """4096 x 11008 (K = 2048, block 256), 16 tokens, 96 sampled output channels."""
    wl = workloads.get("c3t_4096x11008")
    C = q.load_codebook(wl.K)
    g = encode_gpu(q, wl.W_f32(), wl.r, wl.alpha, wl.block, wl.sign_seed, C, wdtype="bf16")
    rng = np.random.default_rng(zlib.crc32(b"matmul"))
    X = rng.standard_normal((16, wl.d)).astype(np.float32)
    rows = np.sort(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 94, replace=False)]))
    say("case matmul c3t 4096x11008 T=16")
    Y1, _ = check_matmul(q, X, g, wl.block, wl.sign_seed, C, wl.d, rows=rows)
    Xt = torch.from_numpy(X).to(DEV)
    Y2 = q.qamw_decode_matmul(q.qamw_rotate_activations(Xt, g["s"], wl.block, wl.sign_seed), g["packed"], g["rn"],
                              g["sigma"], g["C"])
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)              # deterministic


def test_decode_matmul_full_size_one_token(q):
    """4096 x 11008 (K = 2048, block 256), one token (GEMV kernel), 96 sampled channels, deterministic."""
    wl = workloads.get("c3t_4096x11008")
    C = q.load_codebook(wl.K)
    g = encode_gpu(q, wl.W_f32(), wl.r, wl.alpha, wl.block, wl.sign_seed, C, wdtype="bf16")
    rng = np.random.default_rng(zlib.crc32(b"gemv"))
    X = rng.standard_normal((1, wl.d)).astype(np.float32)
    rows = np.sort(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 94, replace=False)]))
    say("case matmul c3t 4096x11008 T=1")
    Y1, Xr = check_matmul(q, X, g, wl.block, wl.sign_seed, C, wl.d, rows=rows)
    Y2 = q.qamw_decode_matmul(Xr, g["packed"], g["rn"], g["sigma"], g["C"])
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
