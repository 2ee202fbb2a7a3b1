"""GPU parity of the QAM-W kernels against the CPU oracle (needs an MI355X).

Criteria (the tolerances the codec's target sets, written out here):
  * s_j: relative error <= 5e-7 (fp32 powf vs fp64 r^alpha).
  * sigma_k: relative error <= 1e-5 (fp32 amplitudes, fp64 tile sums).
  * row norms (fp16 bits): identical, except a one-ulp difference where the
    oracle's norm lies within 1e-9 (relative) of an fp16 rounding boundary.
  * indices: identical, except near-ties -- pairs where the GPU's centroid is
    within 1e-6 |z~|^2 of the oracle's in fp64 squared distance; near-ties are
    counted and printed.
    "mode C": the oracle encodes with the GPU's s and sigma (isolates the
    per-row rotation and the nearest-centroid search);
    "mode I": the oracle uses its own s and sigma (fully independent).
  * decode: max |GPU - oracle| <= 1e-5 in fp32 output; fp16/bf16 outputs
    within half an output ulp of the oracle's fp64 value plus 2e-6.  The
    GPU rounds its fp32 value, so it lands on the other neighbour whenever a
    rounding midpoint lies between that value and the fp64 one: with a
    relative decode error of ~2e-6 that happens for ~2e-6 * 2^10 = 0.2% of
    fp16 outputs; at least 99% must be identical to the oracle's rounding.
Full-size workloads are checked on sampled rows (sigma always over all rows).
"""
import math
import sys
import zlib

import numpy as np
import pytest

import workloads
from oracle import qamw_ref as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vector_codebook_codec_amd as pkg
    from vector_codebook_codec_amd import _lib

    _lib.load()
    return pkg


DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(W, wdtype):
    if wdtype == "bf16":
        return torch.from_numpy(W.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(W).to(DEV)


def f16_boundary_ok(gpu_bits, ora_bits, rho):
    """Equal, or one ulp apart with rho within 1e-9 of a rounding boundary."""
    gpu_bits = gpu_bits.astype(np.int64)
    ora_bits = ora_bits.astype(np.int64)
    same = gpu_bits == ora_bits
    lo = np.minimum(gpu_bits, ora_bits).astype(np.uint16)
    hi = np.maximum(gpu_bits, ora_bits).astype(np.uint16)
    mid = (O.f16_bits_to_f64(lo) + O.f16_bits_to_f64(hi)) / 2
    near = (np.abs(gpu_bits - ora_bits) == 1) & (np.abs(rho - mid) <= 1e-9 * np.abs(rho))
    return same | near


def encode_both(q, W, s, sigma, block, seed, Ct):
    """Encode with the exhaustive search and with a search plan; the two must
    agree bit for bit (packed words and row norms)."""
    packed, rn = q.qamw_encode(W, s, sigma, block, seed, Ct)
    plan = q.qamw_build_plan(Ct)
    packed_p, rn_p = q.qamw_encode(W, s, sigma, block, seed, Ct, plan=plan)
    torch.cuda.synchronize()
    n_bad = int((packed_p != packed).sum())
    assert n_bad == 0, f"planned encode differs from exhaustive in {n_bad} words"
    assert torch.equal(rn_p, rn)
    return packed, rn


def run_gpu(q, wl, C):
    W = to_dev(wl.W, wl.wdtype)
    r = torch.from_numpy(wl.r).to(DEV)
    Ct = torch.from_numpy(C).to(DEV)
    s, sigma = q.qamw_calibrate(W, r, wl.alpha, wl.block, wl.sign_seed)
    packed, rn = encode_both(q, W, s, sigma, wl.block, wl.sign_seed, Ct)
    return dict(W=W, r=r, C=Ct, s=s, sigma=sigma, packed=packed, rn=rn)


def check_encode_rows(wl, C, g, rows, mode, s_ref=None, sig_ref=None):
    """Compare GPU indices / row norms of ``rows`` with the oracle."""
    Wf = wl.W_f32()
    s_g = g["s"].cpu().numpy()
    sig_g = g["sigma"].cpu().numpy()
    s_use, sig_use = (s_g, sig_g) if mode == "C" else (s_ref, sig_ref)
    enc = O.encode(Wf, s_use, sig_use, wl.block, wl.sign_seed, C, rows=rows)
    K = C.shape[0]
    packed = g["packed"].cpu().numpy().view(np.uint32)[rows]
    idx_g = O.unpack(packed, K, wl.d)
    ok = O.accept_index(enc["zt"].reshape(-1, 2), C, enc["idx"].reshape(-1), idx_g.reshape(-1))
    n_diff = int((idx_g != enc["idx"]).sum())
    say(f"  mode {mode}: {len(rows)} rows, {idx_g.size} pairs, {n_diff} differ, "
        f"{int((~ok).sum())} beyond near-tie tolerance")
    assert ok.all(), f"{int((~ok).sum())} indices differ beyond the near-tie tolerance"
    rn = g["rn"].cpu().numpy().view(np.uint16)[rows]
    if mode == "C":
        assert f16_boundary_ok(rn, enc["rho_hat_bits"], enc["rho"]).all()
    # padding words after the last index are zero
    B = O.index_bits(K)
    used = (wl.d // 2) * B
    if used % 32:
        assert not (packed[:, used // 32] >> np.uint32(used % 32)).any()
    assert not packed[:, -(-used // 32):].any()
    return enc, idx_g


def check_decode_rows(q, wl, C, g, rows, out_dtype=torch.float32, use_s=True):
    s_g = g["s"].cpu().numpy()
    sig_g = g["sigma"].cpu().numpy()
    Wh = q.qamw_decode(g["packed"], g["rn"], wl.d, g["s"] if use_s else None, g["sigma"], wl.block,
                       wl.sign_seed, g["C"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    packed = g["packed"].cpu().numpy().view(np.uint32)[rows]
    rn = g["rn"].cpu().numpy().view(np.uint16)[rows]
    ref = O.decode(packed, rn, s_g if use_s else None, sig_g, wl.block, wl.sign_seed, C, wl.d)
    got = Wh[rows].float().cpu().numpy().astype(np.float64)
    if out_dtype == torch.float32:
        err = float(np.max(np.abs(got - ref)))
        say(f"  decode fp32 rows={len(rows)} max abs err {err:.3e}")
        assert err <= 1e-5
    else:
        if out_dtype == torch.float16:
            ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
            bits_ref = O.to_f16_bits(ref)
            bits_got = Wh[rows].cpu().view(torch.int16).numpy().view(np.uint16)
        else:
            e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-38)))
            ulp = 2.0 ** (e - 7)
            bits_ref = O.to_bf16_bits(ref)
            bits_got = Wh[rows].cpu().view(torch.int16).numpy().view(np.uint16)
        err = np.abs(got - ref)
        assert np.all(err <= 0.5 * ulp + 2e-6), float(np.max(err - 0.5 * ulp))
        same = float((bits_ref == bits_got).mean())
        say(f"  decode {out_dtype} identical to oracle rounding: {same:.6f}")
        assert same >= 0.99
    return Wh


# ---------------------------------------------------------------- full c1
def test_c1_full(q):
    wl = workloads.get("c1_256x512")
    C = q.load_codebook(wl.K)
    say(f"case c1 {wl.N}x{wl.d} K={wl.K} b={wl.block}: calibrate/encode")
    g = run_gpu(q, wl, C)
    s_o, sig_o, _ = O.calibrate(wl.W_f32(), wl.r, wl.alpha, wl.block, wl.sign_seed)
    s_g, sig_g = g["s"].cpu().numpy(), g["sigma"].cpu().numpy()
    assert np.max(np.abs(s_g / s_o - 1)) <= 5e-7
    assert np.max(np.abs(sig_g / sig_o - 1)) <= 1e-5
    rows = np.arange(wl.N)
    check_encode_rows(wl, C, g, rows, "C")
    check_encode_rows(wl, C, g, rows, "I", s_o, sig_o)
    say("case c1: decode")
    check_decode_rows(q, wl, C, g, rows)
    check_decode_rows(q, wl, C, g, rows, torch.float16)
    check_decode_rows(q, wl, C, g, rows, torch.bfloat16)
    check_decode_rows(q, wl, C, g, rows, use_s=False)


# ---------------------------------------------------------------- shapes, blocks, K
SHAPES = [
    # (N, d, block, K, wdtype, alpha, seed)
    (3, 16, 16, 2, "f32", 0.5, 1),          # one chunk, one lane, binary codebook
    (5, 48, 16, 4, "bf16", 0.0, 2),          # ragged window, alpha = 0
    (7, 96, 32, 16, "f32", 1.0, 3),
    (9, 1088, 64, 128, "bf16", 0.5, 4),      # two windows, second ragged
    (17, 2560, 128, 1024, "f32", 0.5, 5),
    (6, 3072, 256, 2048, "bf16", 0.5, 6),
    (4, 1536, 512, 4096, "f32", 0.5, 7),
    (3, 2048, 1024, 256, "bf16", 0.5, 8),
    (1, 1024, 1024, 2048, "f32", 0.5, 9),    # a single row
    (3, 17408, 128, 256, "bf16", 0.5, 10),   # 17 windows: row norms and amplitudes in two passes
    (4, 64, 2, 16, "f32", 0.5, 11),          # blocks of 2, 4, 8: the rotation stays inside a lane
    (5, 272, 4, 200, "bf16", 0.5, 12),       # K not a power of two (B = 8), 17 chunks
    (6, 1040, 8, 1000, "f32", 0.5, 13),      # two windows, the second one chunk wide; B = 10
    (3, 2048, 128, 3000, "bf16", 0.5, 14),   # K = 3000: the uniform grid of per-cell records, B = 12
    (2, 262144, 256, 256, "bf16", 0.5, 15),  # 256 windows per row: the widest rows tested
    (20000, 32, 16, 16, "f32", 0.5, 16),     # 20000 one-window rows: every grid walks many rows
]


def codebook_for(q, K):
    """The stored codebook of K centroids, or the first K centroids of the
    next larger stored one (any codebook serves the parity checks)."""
    for k in (2, 4, 16, 128, 256, 1024, 2048, 4096):
        if k == K:
            return q.load_codebook(K)
        if k > K:
            return q.load_codebook(k)[:K].copy()
    raise ValueError(K)


@pytest.mark.parametrize("N,d,block,K,wdtype,alpha,seed", SHAPES)
def test_shapes(q, N, d, block, K, wdtype, alpha, seed):
    rng = np.random.default_rng(1000 + seed)
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    r = rng.lognormal(0.0, 1.0, d).astype(np.float32)
    if wdtype == "bf16":
        W = workloads.bf16_bits_from_f32(W)
    wl = workloads.Workload(f"shape{seed}", W, wdtype, r, alpha, block, seed * 12345, K)
    C = codebook_for(q, K)
    say(f"case shapes N={N} d={d} b={block} K={K} {wdtype} alpha={alpha}")
    g = run_gpu(q, wl, C)
    s_o, sig_o, _ = O.calibrate(wl.W_f32(), wl.r, alpha, block, wl.sign_seed)
    assert np.max(np.abs(g["s"].cpu().numpy() / s_o - 1)) <= 5e-7
    assert np.max(np.abs(g["sigma"].cpu().numpy() / sig_o - 1)) <= 1e-5
    rows = np.arange(N)
    check_encode_rows(wl, C, g, rows, "C")
    check_decode_rows(q, wl, C, g, rows)


def test_strided_rows(q):
    """ldw > d on input and ldo > d on output."""
    rng = np.random.default_rng(77)
    N, d, ld, K, b = 10, 512, 640, 256, 128
    big = (rng.standard_normal((N, ld)) * 0.02).astype(np.float32)
    r = rng.lognormal(0, 1, d).astype(np.float32)
    C = q.load_codebook(K)
    Wbig = torch.from_numpy(big).to(DEV)
    W = Wbig[:, :d]
    s, sigma = q.qamw_calibrate(W, torch.from_numpy(r).to(DEV), 0.5, b, 3)
    packed, rn = q.qamw_encode(W, s, sigma, b, 3, torch.from_numpy(C).to(DEV))
    Wc = W.contiguous()
    s2, sigma2 = q.qamw_calibrate(Wc, torch.from_numpy(r).to(DEV), 0.5, b, 3)
    packed2, rn2 = q.qamw_encode(Wc, s2, sigma2, b, 3, torch.from_numpy(C).to(DEV))
    out_big = torch.zeros((N, ld), device=DEV)
    q.qamw_decode(packed, rn, d, s, sigma, b, 3, torch.from_numpy(C).to(DEV), out=out_big[:, :d])
    ref = q.qamw_decode(packed2, rn2, d, s2, sigma2, b, 3, torch.from_numpy(C).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(s, s2) and torch.equal(sigma, sigma2)
    assert torch.equal(packed, packed2) and torch.equal(rn, rn2)
    assert torch.equal(out_big[:, :d], ref)
    assert torch.count_nonzero(out_big[:, d:]) == 0


@pytest.mark.parametrize("N,d,block,K,wdtype,alpha,seed", SHAPES)
def test_decode_16bit_is_rounded_fp32(q, N, d, block, K, wdtype, alpha, seed):
    """bf16 output = the fp32 decode rounded to nearest even, bit for bit; fp16
    output within one unit in the last place of it (the last scale and the
    rounding are one fused step); columns past d of a strided output untouched.
    Covers every block size, ragged windows and single rows for the 16-bit
    stores (the fp32 decode of the same shapes is checked against the oracle)."""
    rng = np.random.default_rng(2000 + seed)
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    r = rng.lognormal(0.0, 1.0, d).astype(np.float32)
    if wdtype == "bf16":
        W = workloads.bf16_bits_from_f32(W)
    wl = workloads.Workload(f"shape16_{seed}", W, wdtype, r, alpha, block, seed * 7919, K)
    say(f"case decode16 N={N} d={d} b={block} K={K}")
    g = run_gpu(q, wl, codebook_for(q, K))
    args = (g["packed"], g["rn"], d, g["s"], g["sigma"], block, wl.sign_seed, g["C"])
    ref32 = q.qamw_decode(*args)
    pad = 40
    for dt in (torch.bfloat16, torch.float16):
        big = torch.full((N, d + pad), -3.0, dtype=dt, device=DEV)
        q.qamw_decode(*args, out=big[:, :d])
        torch.cuda.synchronize()
        got = big[:, :d].contiguous().view(torch.int16).cpu().numpy().astype(np.int32)
        want = ref32.to(dt).view(torch.int16).cpu().numpy().astype(np.int32)
        if dt == torch.bfloat16:
            assert np.array_equal(got, want)
        else:
            assert int(np.max(np.abs(got - want))) <= 1
        assert torch.all(big[:, d:] == -3.0)


# ---------------------------------------------------------------- degenerate inputs
def test_zero_rows_and_zero_sigma(q):
    rng = np.random.default_rng(5)
    N, d, b, K = 8, 256, 128, 256
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    W[3] = 0.0
    C = q.load_codebook(K)
    Wt = torch.from_numpy(W).to(DEV)
    s = torch.ones(d, device=DEV)
    sig_np = (np.abs(rng.standard_normal(d // 2)) * 0.05 + 0.01).astype(np.float32)
    sig_np[[0, 17, 127]] = 0.0
    sigma = torch.from_numpy(sig_np).to(DEV)
    Ct = torch.from_numpy(C).to(DEV)
    say("case degenerate: zero row, sigma_k = 0")
    packed, rn = encode_both(q, Wt, s, sigma, b, 9, Ct)
    Wh = q.qamw_decode(packed, rn, d, s, sigma, b, 9, Ct)
    torch.cuda.synchronize()
    enc = O.encode(W, np.ones(d), sig_np, b, 9, C)
    idx_g = O.unpack(packed.cpu().numpy().view(np.uint32), K, d)
    ok = O.accept_index(enc["zt"].reshape(-1, 2), C, enc["idx"].reshape(-1), idx_g.reshape(-1))
    assert ok.all()
    origin, *_ = O.nearest_centroid(np.zeros((1, 2)), C)
    assert np.all(idx_g[:, [0, 17, 127]] == origin[0])
    assert np.all(idx_g[3] == origin[0])
    assert rn.cpu().numpy()[3] == 0
    assert torch.count_nonzero(Wh[3]) == 0


def test_all_zero_matrix(q):
    N, d, b, K = 4, 128, 128, 16
    Wt = torch.zeros((N, d), device=DEV)
    C = q.load_codebook(K)
    s, sigma = q.qamw_calibrate(Wt, torch.ones(d, device=DEV), 0.5, b, 0)
    packed, rn = encode_both(q, Wt, s, sigma, b, 0, torch.from_numpy(C).to(DEV))
    Wh = q.qamw_decode(packed, rn, d, s, sigma, b, 0, torch.from_numpy(C).to(DEV))
    torch.cuda.synchronize()
    assert torch.count_nonzero(sigma) == 0
    assert torch.count_nonzero(rn) == 0 and torch.count_nonzero(Wh) == 0
    origin, *_ = O.nearest_centroid(np.zeros((1, 2)), C)
    assert np.all(O.unpack(packed.cpu().numpy().view(np.uint32), K, d) == origin[0])


@pytest.mark.parametrize("K", [5, 200, 1000])   # B = 3 (width at run time), 8 and 10 (compile time)
def test_out_of_range_indices_clamp(q, K):
    """A hand-made stream with indices >= K decodes as K - 1."""
    N, d, b = 2, 64, 32
    C = q.load_codebook(1024 if K > 16 else 16)[:K].copy()
    B = O.index_bits(K)
    rng = np.random.default_rng(3 + K)
    idx = rng.integers(0, 1 << B, size=(N, d // 2))
    idx[:, :4] = (1 << B) - 1                                # the largest index is always present
    packed = O.pack(idx, K, d)
    rn = O.to_f16_bits(np.array([1.0, 0.5]))
    sig = np.full(d // 2, 0.1, np.float32)
    s = np.ones(d, np.float32)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    Wh = q.qamw_decode(dev(packed.view(np.int32)), dev(rn.view(np.int16)), d, dev(s), dev(sig), b, 4, dev(C))
    torch.cuda.synchronize()
    ref = O.decode(packed, rn, s, sig, b, 4, C, d)
    assert float(np.max(np.abs(Wh.cpu().numpy() - ref))) <= 1e-6
    # the one-token product reads the same stream: indices >= K act as K - 1
    x = rng.standard_normal(d).astype(np.float32)
    Xr = q.qamw_rotate_activations(dev(np.ascontiguousarray(x[None, :])), dev(s), b, 4)
    y = q.qamw_decode_matmul(Xr, dev(packed.view(np.int32)), dev(rn.view(np.int16)), dev(sig), dev(C))
    torch.cuda.synchronize()
    y_ref = Wh.double() @ torch.from_numpy(x.astype(np.float64)).to(DEV)
    S = float((Wh.abs().double() @ torch.from_numpy(np.abs(x).astype(np.float64)).to(DEV)).max())
    assert float((y[0].double() - y_ref).abs().max()) <= 2.0 ** -7 * S + 1e-6


@pytest.mark.parametrize("Kb", [4, 16, 32])
def test_exact_ties_lowest_index(q, Kb):
    """Duplicated centroids: every index must be the first copy.  The
    exhaustive kernel's MFMA tiles hold 32 centroids, rows 8 g + 4 h + k in
    half-wave h: copies 4 apart tie across the half-waves of one tile, 16
    apart inside one half-wave, 32 apart across tiles."""
    rng = np.random.default_rng(11)
    N, d, b = 4, 256, 64
    base = q.load_codebook(4) if Kb == 4 else (q.load_codebook(16) if Kb == 16 else q.load_codebook(256)[:32].copy())
    C = np.concatenate([base, base]).astype(np.float32)          # K = 2 Kb, second half duplicates
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    s, sigma = q.qamw_calibrate(dev(W), dev(np.ones(d, np.float32)), 0.0, b, 1)
    packed, rn = encode_both(q, dev(W), s, sigma, b, 1, dev(C))
    torch.cuda.synchronize()
    idx = O.unpack(packed.cpu().numpy().view(np.uint32), 2 * Kb, d)
    assert idx.max() < Kb
    enc = O.encode(W, s.cpu().numpy(), sigma.cpu().numpy(), b, 1, C)
    assert O.accept_index(enc["zt"].reshape(-1, 2), C, enc["idx"].reshape(-1), idx.reshape(-1)).all()


# ---------------------------------------------------------------- non-finite weights, dead channels
def test_non_finite_weights(q):
    """Rows holding NaN or +-Inf weights (outside the codec's contract, which
    leaves their indices unspecified): every encode kernel completes, the
    planned and exhaustive searches give the same words, every index is in
    range, and the finite rows still match the oracle.  s and sigma come from
    the finite matrix."""
    rng = np.random.default_rng(31)
    N, d, b, K, seed = 8, 1024, 128, 2048, 17
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    r = rng.lognormal(0.0, 1.0, d).astype(np.float32)
    C = q.load_codebook(K)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    s, sigma = q.qamw_calibrate(dev(W), dev(r), 0.5, b, seed)
    Wb = W.copy()
    Wb[1, 5] = np.nan
    Wb[3, 700] = np.inf
    Wb[5, 130] = -np.inf
    Wb[6, :] = np.nan
    say("case non-finite weights")
    packed, rn = encode_both(q, dev(Wb), s, sigma, b, seed, dev(C))
    idx = O.unpack(packed.cpu().numpy().view(np.uint32), K, d)
    assert idx.max() < K
    finite = [0, 2, 4, 7]
    enc = O.encode(Wb[finite], s.cpu().numpy(), sigma.cpu().numpy(), b, seed, C)
    assert O.accept_index(enc["zt"].reshape(-1, 2), C, enc["idx"].reshape(-1), idx[finite].reshape(-1)).all()
    # calibrate_encode on this matrix (its own, non-finite calibration): with
    # and without a plan, the same words
    s2, sig2, packed2, rn2 = q.qamw_calibrate_encode(dev(Wb), dev(r), 0.5, b, seed, dev(C),
                                                     plan=q.qamw_build_plan(dev(C)))
    packed3, _ = q.qamw_encode(dev(Wb), s2, sig2, b, seed, dev(C))
    torch.cuda.synchronize()
    assert torch.equal(packed2, packed3)


def test_dead_channel(q):
    """r_j = 0 for one input channel: s_j = 0 (alpha = 1/2), the channel is
    zeroed before quantisation and decodes as 0 (the oracle's reading), every
    other column matches the oracle, and the one-token product drops it."""
    rng = np.random.default_rng(32)
    N, d, b, K, seed, j = 16, 512, 128, 256, 3, 77
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    r = rng.lognormal(0.0, 1.0, d).astype(np.float32)
    r[j] = 0.0
    wl = workloads.Workload("dead", W, "f32", r, 0.5, b, seed, K)
    C = q.load_codebook(K)
    say("case dead channel")
    g = run_gpu(q, wl, C)
    s_g = g["s"].cpu().numpy()
    assert s_g[j] == 0.0 and np.all(np.isfinite(g["sigma"].cpu().numpy()))
    check_encode_rows(wl, C, g, np.arange(N), "C")
    Wh = check_decode_rows(q, wl, C, g, np.arange(N))
    assert torch.all(Wh[:, j] == 0) and bool(torch.isfinite(Wh).all())
    # the one-token product (rotated activations, bf16) drops the channel too
    x = rng.standard_normal(d).astype(np.float32)
    xt = torch.from_numpy(x).to(DEV)[None, :]
    Xr = q.qamw_rotate_activations(xt, g["s"], b, seed)
    y = q.qamw_decode_matmul(Xr, g["packed"], g["rn"], g["sigma"], g["C"])[0]
    torch.cuda.synchronize()
    y_ref = Wh.double() @ torch.from_numpy(x.astype(np.float64)).to(DEV)
    S = float((Wh.abs().double() @ torch.from_numpy(np.abs(x).astype(np.float64)).to(DEV)).max())
    assert bool(torch.isfinite(y).all()) and float((y.double() - y_ref).abs().max()) <= 2.0 ** -7 * S


# ---------------------------------------------------------------- determinism
def test_repeatable_bitwise(q):
    wl = workloads.get("c1_256x512")
    C = q.load_codebook(wl.K)
    outs = []
    for _ in range(3):
        g = run_gpu(q, wl, C)
        Wh = q.qamw_decode(g["packed"], g["rn"], wl.d, g["s"], g["sigma"], wl.block, wl.sign_seed, g["C"])
        torch.cuda.synchronize()
        outs.append((g["s"].cpu(), g["sigma"].cpu(), g["packed"].cpu(), g["rn"].cpu(), Wh.cpu()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


# ---------------------------------------------------------------- full-size workloads
FULL = ["c2_4096x4096", "c3_11008x4096", "c3t_4096x11008"] + \
    [f"c4_5120x13824_K{K}_a{a}" for K in (256, 1024, 2048, 4096) for a in ("0", "0.5")] + \
    ["c5_l0_q", "c5_l5_k", "c5_l9_v", "c5_l13_o", "c5_l31_gate", "c5_l22_up", "c5_l17_down"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(q, name):
    wl = workloads.get(name)
    C = q.load_codebook(wl.K)
    say(f"case {name} {wl.N}x{wl.d} K={wl.K} b={wl.block}: GPU calibrate/encode")
    g = run_gpu(q, wl, C)
    s_o, sig_o, _ = O.calibrate(wl.W_f32(), wl.r, wl.alpha, wl.block, wl.sign_seed)
    s_g, sig_g = g["s"].cpu().numpy(), g["sigma"].cpu().numpy()
    assert np.max(np.abs(s_g / s_o - 1)) <= 5e-7
    err = np.max(np.abs(sig_g / sig_o - 1))
    say(f"  sigma max rel err {err:.3e}")
    assert err <= 1e-5
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    # the headline matrix gets a larger sample (48 rows) than the other shapes (12)
    extra = 46 if name == "c3t_4096x11008" else 10
    rows = np.sort(np.concatenate([[0, wl.N - 1], rng.choice(np.arange(1, wl.N - 1), extra, replace=False)]))
    check_encode_rows(wl, C, g, rows, "C")
    check_encode_rows(wl, C, g, rows, "I", s_o, sig_o)
    # the stored fp16 row norm of every row, against the oracle's rho with the
    # GPU's s (the products formed in fp64: fp32 products would round them)
    rho_all = O.row_split(wl.W_f32().astype(np.float64) * s_g.astype(np.float64)[None, :])[0]
    rn_all = g["rn"].cpu().numpy().view(np.uint16)
    ok_rn = f16_boundary_ok(rn_all, O.to_f16_bits(rho_all), rho_all)
    say(f"  row norms: {int((~ok_rn).sum())} of {wl.N} rows differ")
    assert ok_rn.all()
    say(f"case {name}: GPU decode, every row")
    every = np.arange(wl.N)
    check_decode_rows(q, wl, C, g, every)
    if name.startswith("c3"):
        check_decode_rows(q, wl, C, g, every, torch.float16)
    if name == "c3t_4096x11008":
        check_decode_rows(q, wl, C, g, every, torch.bfloat16)


# ---------------------------------------------------------------- search plan
PLAN_OVERFLOW = 255
U32 = 2.0 ** -24


def _uniform_records(raw, off, G, lmax):
    """Per-cell records of a uniform grid: entry i is 16 c_i | nibble_i with
    nibble_0 = count - 1 and nibble_1 = overflow."""
    rec = raw[off:off + G * G * lmax * 2].view(np.uint16).reshape(G * G, lmax).astype(np.int64)
    nib = rec & 15
    assert np.all(nib[:, 1] <= 1) and np.all(nib[:, 2:] == 0)
    counts = np.where(nib[:, 1] == 1, PLAN_OVERFLOW, nib[:, 0] + 1)
    lists = rec >> 4
    ok = counts != PLAN_OVERFLOW
    assert np.all(counts[ok] <= lmax) and np.all(counts[ok] >= 1)
    used = np.arange(lmax)[None, :] < counts[:, None]
    last = lists[np.arange(len(counts)), np.clip(counts, 1, lmax) - 1]
    assert np.all((lists == last[:, None])[ok][~used[ok]])
    return counts, lists


def _lds_records(img, G, cells_off, lists_off, cap, nlists, K):
    """Cell entries of the LDS table: 16 c (one candidate), 0x8000 | r (list
    record r: 4 x 16 c ascending, tail repeating the last, the top bit of the
    fourth entry continuing in record r + 1) or 0xFFFF (scan all)."""
    cells = img[cells_off:cells_off + 2 * G * G].view(np.uint16).astype(np.int64)
    recs = img[lists_off:lists_off + 8 * cap].view(np.uint16).reshape(cap, 4).astype(np.int64)
    counts = np.full(G * G, PLAN_OVERFLOW, np.int64)
    lists = np.zeros((G * G, 8), np.int64)
    single = cells < 0x8000
    assert np.all(cells[single] & 15 == 0)
    counts[single] = 1
    lists[single] = (cells[single] >> 4)[:, None]
    for c in np.nonzero((cells >= 0x8000) & (cells != 0xFFFF))[0]:
        r = cells[c] & 0x7FFF
        assert r < nlists
        ent = list(recs[r])
        more = ent[3] >> 15
        ent[3] &= 0x7FFF
        if more:
            assert r + 1 < nlists
            ent += list(recs[r + 1])
        ent = np.array(ent)
        assert np.all(ent & 15 == 0)
        ent >>= 4
        uniq = np.unique(ent)
        assert np.all(np.diff(ent) >= 0) and np.all(ent < K), "lists ascend, tails repeat the last entry"
        assert 2 <= len(uniq) <= 8
        counts[c] = len(uniq)
        lists[c, :len(uniq)] = uniq
        lists[c, len(uniq):] = uniq[-1]
    return counts, lists


def read_plan(q, C):
    """Build the plan on the GPU and decode its grids: {"inner": ..., "outer":
    ...}, each (kind, geometry, counts, lists of centroid indices)."""
    K = C.shape[0]
    plan = q.qamw_build_plan(torch.from_numpy(C).to(DEV))
    torch.cuda.synchronize()
    raw = plan.cpu().numpy()
    assert raw.size == q.qamw_plan_bytes(K)
    hdr_f = raw[:64].view(np.float32)
    hdr_i = raw[:64].view(np.int32)
    lmax = 8 if K <= 2048 else 16
    assert hdr_f[0] == 5.0 and hdr_i[3] == lmax and hdr_i[4] == K
    assert hdr_f[5] == 20.0 and hdr_f[6] == np.float32(128 / 40.0) and hdr_i[7] == 128
    grids = {}
    if K <= 2048:
        G, bins, cap, nlists, ib, co, lo, io = (int(v) for v in hdr_i[8:16])
        assert bins == 2048 and 1 <= G <= 256 and 0 <= nlists <= cap and hdr_i[2] == 0
        img = raw[io:io + ib]
        bmap = img[:bins].astype(np.int64)
        assert bmap[0] == 0 and bmap[-1] == G - 1 and np.all(np.diff(bmap) >= 0) and np.all(np.diff(bmap) <= 1)
        counts, lists = _lds_records(img, G, co, lo, cap, nlists, K)
        grids["inner"] = ("lds", (bmap, G), counts, lists)
        outer_off = 256
    else:
        assert hdr_i[2] == 512 and hdr_f[1] == np.float32(512 / 10.0) and hdr_i[8] == 0
        counts, lists = _uniform_records(raw, 256, 512, lmax)
        grids["inner"] = ("uniform", (512, 5.0), counts, lists)
        outer_off = 256 + 512 * 512 * lmax * 2
    counts, lists = _uniform_records(raw, outer_off, 128, lmax)
    grids["outer"] = ("uniform", (128, 20.0), counts, lists)
    return grids, lmax


def cell_of(z, grid):
    """Cell index of points inside the grid, from fp32 coordinates as the kernel forms them."""
    kind, geom = grid[0], grid[1]
    zf = z.astype(np.float32).astype(np.float64)
    if kind == "lds":
        bmap, G = geom
        kb = np.float64(np.float32(2048 / 10.0))
        t = (zf * kb + 1024.0).astype(np.float32)
        bx = np.minimum(t[:, 0].astype(np.int64), 2047)
        by = np.minimum(t[:, 1].astype(np.int64), 2047)
        return bmap[bx] * G + bmap[by]
    G, R = geom
    cpu = np.float32(G / (2 * R))
    zf32 = z.astype(np.float32)
    ix = np.minimum(((zf32[:, 0] + np.float32(R)) * cpu).astype(np.int64), G - 1)
    iy = np.minimum(((zf32[:, 1] + np.float32(R)) * cpu).astype(np.int64), G - 1)
    return ix * G + iy


def grid_of(z):
    """Which grid the encode kernel consults for each point (None: full scan)."""
    zf = z.astype(np.float32)
    fine = (zf >= -5).all(1) & (zf < 5).all(1)
    outer = (zf >= -20).all(1) & (zf < 20).all(1)
    return fine, outer & ~fine


def fp32_candidates(z, Cd):
    """Centroids that can be the fp32 nearest one of fp32 point z: the fp32
    score of c is within 2^-24 (2.5 |c|^2 + 2 |z| |c|) of |c|^2/2 - z.c, so
    the winner's squared distance exceeds the minimum by at most
    4 2^-24 (2.5 m^2 + 2 |z| m), m the larger centroid radius (fp64, z as the kernel has it)."""
    zf = z.astype(np.float32).astype(np.float64)
    D = ((zf[:, None, :] - Cd[None, :, :]) ** 2).sum(-1)
    best = D.argmin(1)
    rc = np.sqrt((Cd ** 2).sum(1))
    m = np.maximum(rc[None, :], rc[best][:, None])
    rz = np.sqrt((zf ** 2).sum(1))[:, None]
    return D <= D.min(1, keepdims=True) + 4 * U32 * (2.5 * m * m + 2 * rz * m) * 1.0001


@pytest.mark.parametrize("K", [2, 16, 256, 1000, 2048, 4096])
def test_plan_lists_cover_near_minimisers(q, K):
    """Every centroid that can be the fp32 nearest one of a point (within the
    fp32 scores' error bound of its minimum squared distance, fp64 brute
    force) is in the list of the cell the encode kernel consults for that
    point; lists are ascending and in range (checked while decoding)."""
    C = q.load_codebook(K) if K != 1000 else q.load_codebook(1024)[:1000].copy()
    grids, lmax = read_plan(q, C)
    # the outer cells tiling the inner grid's square [-5, 5)^2 are never
    # consulted (points there take the inner grid): "scan all" records
    G2 = 128
    lo = (G2 - G2 * 10 // 40) // 2
    assert np.all(grids["outer"][2].reshape(G2, G2)[lo:G2 - lo, lo:G2 - lo] == PLAN_OVERFLOW)
    for name, (kind, geom, counts, lists) in grids.items():
        ok_cells = counts != PLAN_OVERFLOW
        say(f"case plan K={K} {name} ({kind}): {int((~ok_cells).sum())} scan-all cells of {counts.size}, "
            f"max count {int(counts[ok_cells].max())}")
        assert np.all(lists[ok_cells] < K)
    rng = np.random.default_rng(K)
    fine_edges = -5 + np.arange(2048) * (10 / 2048)
    outer_edges = -20 + np.arange(128) * (40 / 128)
    z = np.concatenate([
        rng.uniform(-5, 5, (30000, 2)),
        rng.standard_normal((30000, 2)),
        rng.standard_normal((10000, 2)) * 0.05,
        np.stack([rng.choice(fine_edges, 6000), rng.choice(fine_edges, 6000)], 1),
        np.stack([np.full(200, 5 - 1e-6), rng.uniform(-5, 5, 200)], 1),
        rng.uniform(-20, 20, (20000, 2)),
        rng.standard_normal((10000, 2)) * 8,
        np.stack([rng.choice(outer_edges, 4000), rng.choice(outer_edges, 4000)], 1),
    ])
    # the centroids themselves and the midpoints of close pairs: exact and near ties
    z = np.concatenate([z, C.astype(np.float64), (C[:-1] + C[1:]).astype(np.float64) / 2])
    fine, outer = grid_of(z)
    Cd = C.astype(np.float64)
    gauss = np.zeros(len(z), bool)
    gauss[30000:60000] = True
    for name, sel in (("inner", fine), ("outer", outer)):
        grid = grids[name]
        counts, lists = grid[2], grid[3]
        zs = z[sel]
        total, npts = 0.0, 0
        for lo_ in range(0, len(zs), 4000):
            zz = zs[lo_:lo_ + 4000]
            near = fp32_candidates(zz, Cd)
            cells = cell_of(zz, grid)
            listed = np.zeros_like(near)
            rows = np.repeat(np.arange(len(zz)), lists.shape[1])
            cols = lists[cells].reshape(-1)
            listed[rows, cols] = True
            listed[counts[cells] == PLAN_OVERFLOW] = True
            assert not (near & ~listed).any(), f"a possible fp32 winner is missing from a {name} cell list"
        if name == "inner":
            cg = cell_of(z[gauss & fine], grid)
            mean = float(np.where(counts[cg] == PLAN_OVERFLOW, K, counts[cg]).mean())
            say(f"  mean candidates per N(0, I) point: {mean:.2f}")


def test_plan_overflow_and_outside_grid(q):
    """Clustered centroids overflow their cells' lists, moderately small
    sigma_k put pairs on the outer grid and tiny ones beyond it: every case is
    bit-identical to the exhaustive search and accepted by the oracle."""
    rng = np.random.default_rng(21)
    base = q.load_codebook(16)
    ang = rng.uniform(0, 2 * np.pi, 48)
    cluster = np.stack([0.3 + 1e-3 * np.cos(ang), -0.2 + 1e-3 * np.sin(ang)], 1)
    C = np.concatenate([base, cluster]).astype(np.float32)          # K = 64
    grids, _ = read_plan(q, C)
    counts = grids["inner"][2]
    assert (counts == PLAN_OVERFLOW).any()
    N, d, b = 64, 4096, 256
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    s, sigma = q.qamw_calibrate(dev(W), dev(np.ones(d, np.float32)), 0.0, b, 5)
    sig_np = sigma.cpu().numpy().copy()
    sig_np[::7] *= 1e-3                                                  # |z~| ~ 1e3: beyond both grids
    sig_np[3::7] *= 0.15                                                 # |z~| ~ 5..30: outer grid, some beyond
    sigma = dev(sig_np)
    say("case plan overflow / outer grid / outside")
    packed, rn = encode_both(q, dev(W), s, sigma, b, 5, dev(C))
    enc = O.encode(W, s.cpu().numpy(), sig_np, b, 5, C)
    zt = enc["zt"].reshape(-1, 2)
    fine, outer = grid_of(zt)
    in_overflow = fine.copy()
    in_overflow[fine] = counts[cell_of(zt[fine], grids["inner"])] == PLAN_OVERFLOW
    say(f"  {int(outer.sum())} pairs on the outer grid, {int((~fine & ~outer).sum())} beyond it, "
        f"{int(in_overflow.sum())} in overflow cells")
    assert outer.sum() > 1000 and (~fine & ~outer).sum() > 1000 and in_overflow.sum() > 0
    idx = O.unpack(packed.cpu().numpy().view(np.uint32), C.shape[0], d)
    assert O.accept_index(zt, C, enc["idx"].reshape(-1), idx.reshape(-1)).all()


@pytest.mark.parametrize("K_plan,K_use", [(2048, 1024), (4096, 2048), (4096, 3000)])
def test_plan_built_for_another_k(q, K_plan, K_use):
    """A plan built for another codebook size (its buffer at least as large as
    qamw_plan_bytes of the K in use, so the host accepts it) is detected on
    the device: every pair then scans the whole codebook, and the words equal
    the exhaustive search's bit for bit.  A plan buffer smaller than
    qamw_plan_bytes(K) is refused before any launch."""
    assert q.qamw_plan_bytes(K_plan) >= q.qamw_plan_bytes(K_use)
    rng = np.random.default_rng(K_plan + K_use)
    N, d, b = 48, 2048, 128
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    s, sigma = q.qamw_calibrate(dev(W), dev(rng.lognormal(0.0, 1.0, d).astype(np.float32)), 0.5, b, 9)
    C_plan, C_use = dev(codebook_for(q, K_plan)), dev(codebook_for(q, K_use))
    plan = q.qamw_build_plan(C_plan)
    say(f"case plan built for K={K_plan} used with K={K_use}")
    ref, rn_ref = q.qamw_encode(dev(W), s, sigma, b, 9, C_use)
    got, rn = q.qamw_encode(dev(W), s, sigma, b, 9, C_use, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(got, ref) and torch.equal(rn, rn_ref)
    # the other way round the buffer is too small: refused on the host
    small = q.qamw_build_plan(C_use)
    if q.qamw_plan_bytes(K_use) < q.qamw_plan_bytes(K_plan):
        with pytest.raises(ValueError):
            q.qamw_encode(dev(W), s, sigma, b, 9, C_plan, plan=small)


def test_encode_phases_match_encode(q):
    """qamw_encode_prepare + qamw_encode_indices give qamw_encode's outputs,
    with and without a plan, and the workspace is reusable across codebooks."""
    wl = workloads.get("c1_256x512")
    W = to_dev(wl.W, wl.wdtype)
    s, sigma = q.qamw_calibrate(W, torch.from_numpy(wl.r).to(DEV), wl.alpha, wl.block, wl.sign_seed)
    rn, ws = q.qamw_encode_prepare(W, s, sigma, wl.block, wl.sign_seed)
    for K in (wl.K, 16):
        Ct = torch.from_numpy(q.load_codebook(K)).to(DEV)
        packed, rn_ref = q.qamw_encode(W, s, sigma, wl.block, wl.sign_seed, Ct)
        for plan in (None, q.qamw_build_plan(Ct)):
            got = q.qamw_encode_indices(W, wl.block, Ct, ws, plan=plan)
            torch.cuda.synchronize()
            assert torch.equal(got, packed)
        assert torch.equal(rn, rn_ref)


# ---------------------------------------------------------------- calibrate + encode in one call
@pytest.mark.parametrize("name", ["c1_256x512", "c3t_4096x11008"])
def test_calibrate_encode_matches_separate_calls(q, name):
    wl = workloads.get(name)
    say(f"case calibrate_encode {name}")
    W = to_dev(wl.W, wl.wdtype)
    r = torch.from_numpy(wl.r).to(DEV)
    Ct = torch.from_numpy(q.load_codebook(wl.K)).to(DEV)
    plan = q.qamw_build_plan(Ct)
    s, sigma = q.qamw_calibrate(W, r, wl.alpha, wl.block, wl.sign_seed)
    packed, rn = q.qamw_encode(W, s, sigma, wl.block, wl.sign_seed, Ct, plan=plan)
    for p in (plan, None):
        s2, sig2, packed2, rn2 = q.qamw_calibrate_encode(W, r, wl.alpha, wl.block, wl.sign_seed, Ct, plan=p)
        torch.cuda.synchronize()
        assert torch.equal(s2, s) and torch.equal(sig2, sigma)
        assert torch.equal(packed2, packed) and torch.equal(rn2, rn)
    # the calibration half, then qamw_encode_indices on its workspace (the
    # plan built on another stream meanwhile, joined before the encode)
    side = torch.cuda.Stream()
    plan2 = torch.empty_like(plan)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.qamw_build_plan(Ct, plan2)
    s3, sig3, rn3, ws = q.qamw_calibrate_prepare(W, r, wl.alpha, wl.block, wl.sign_seed)
    torch.cuda.current_stream().wait_stream(side)
    packed3 = q.qamw_encode_indices(W, wl.block, Ct, ws, plan=plan2)
    torch.cuda.synchronize()
    assert torch.equal(s3, s) and torch.equal(sig3, sigma) and torch.equal(rn3, rn)
    assert torch.equal(packed3, packed)
    # the same plan: header fields, outer grid and table image (the build's
    # scratch after the image, and the header block's unused tail, are not
    # part of it)
    hdr = plan[:64].cpu().numpy().view(np.int32)
    end = int(hdr[15]) + int(hdr[12])
    assert torch.equal(plan2[:64], plan[:64]) and torch.equal(plan2[256:end], plan[256:end])
