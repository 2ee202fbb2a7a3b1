"""The no-allocation encode (qamw_encode_noalloc, the library's own per-GPU
workspace) against qamw_encode with a caller workspace, through the C ABI:
identical packed words and row norms, with and without a search plan, on two
calls in a row, the second with a smaller matrix (the shared array keeps the
first call's contents, which the second must not depend on)."""
import numpy as np
import pytest

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


def _case(q, N, d, b, K, seed, dtype):
    rng = np.random.default_rng(seed)
    W = torch.from_numpy((rng.standard_normal((N, d)) * 0.02).astype(np.float32)).to(DEV).to(dtype)
    r = torch.from_numpy(rng.lognormal(0.0, 1.0, d).astype(np.float32)).to(DEV)
    C = torch.from_numpy(q.load_codebook(K)).to(DEV)
    s, sigma = q.qamw_calibrate(W, r, 0.5, b, seed)
    return W, s, sigma, C


@pytest.mark.parametrize("use_plan", [False, True])
def test_noalloc_matches_encode_twice(q, use_plan):
    out = []
    for (N, d, b, K, seed, dtype) in ((512, 11008, 256, 2048, 5, torch.bfloat16), (37, 1024, 128, 256, 6, torch.float32)):
        print(f"case noalloc N={N} d={d} b={b} K={K} plan={use_plan}", flush=True)
        W, s, sigma, C = _case(q, N, d, b, K, seed, dtype)
        plan = q.qamw_build_plan(C) if use_plan else None
        ref_p, ref_r = q.qamw_encode(W, s, sigma, b, seed, C, plan=plan)
        rw = q.qamw_packed_row_words(d, K)
        packed = torch.full((N, rw), -1, dtype=torch.int32, device=DEV)
        rn = torch.full((N,), -1, dtype=torch.int16, device=DEV)
        q.qamw_encode_noalloc(W, s, sigma, b, seed, C, plan=plan, packed=packed, rownorm_f16=rn)
        torch.cuda.synchronize()
        assert torch.equal(packed, ref_p) and torch.equal(rn, ref_r)
        out.append(packed.cpu())
    assert out[0].shape != out[1].shape


def test_noalloc_rejects_oversize(q):
    from vector_codebook_codec_amd import _lib

    lib = _lib.load()
    assert lib.qamw_encode_noalloc_scratch_bytes() == 1 << 20
    # 2^17 rows need 1 MiB of fp64 row norms alone: refused before any launch
    rc = lib.qamw_encode_noalloc(1 << 20, 1, 1 << 17, 16, 16, 1 << 20, 1 << 20, 16, 0, 1 << 20, 256, None, 0,
                                 1 << 20, 1 << 20, None)
    assert rc == _lib.QAMW_EUNSUPPORTED and b"no-allocation" in lib.qamw_last_error()
