"""GPU parity of the polar-code encode (qamw_encode_polar) against the oracle
(oracle/polar.py); needs an MI355X.

Criteria:
  * amplitude and phase indices identical to the oracle's fp32 decisions
    on the GPU's z~, except near-ties (``accept_polar``: fp64 |r - a| or the
    fp64 inner product within 1e-6 |z~| of the oracle choice's); near-ties
    are counted and printed.  The oracle encodes with the GPU's s and sigma
    (it isolates the per-row transform and the quantiser).
  * row norms: identical fp16 bits (same rule as the joint encode).
  * decode through the joint decoder with the product table: max |GPU -
    oracle| <= 1e-5 in fp32.
  * the pages' ablation at 8 bits per pair: the joint K = 256 codebook
    reconstructs the synthetic matrix with less error than the 8 x 32 polar code.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import polar as P
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


def to_dev(W, wdtype):
    if wdtype == "bf16":
        return torch.from_numpy(W.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(W).to(DEV)


def run_polar(q, wl, Ka, Kp):
    lv, dr, tb = q.load_polar(Ka, Kp)
    W = to_dev(wl.W, wl.wdtype)
    s, sigma = q.qamw_calibrate(W, torch.from_numpy(wl.r).to(DEV), wl.alpha, wl.block, wl.sign_seed)
    packed, rn = q.qamw_encode_polar(W, s, sigma, wl.block, wl.sign_seed, torch.from_numpy(lv).to(DEV),
                                     torch.from_numpy(dr).to(DEV))
    torch.cuda.synchronize()
    return dict(W=W, s=s, sigma=sigma, packed=packed, rn=rn, lv=lv, dr=dr, tb=tb)


def check_rows(wl, g, rows, Ka, Kp):
    s_g = g["s"].cpu().numpy()
    sig_g = g["sigma"].cpu().numpy()
    enc = P.encode_polar(wl.W_f32(), s_g, sig_g, wl.block, wl.sign_seed, g["lv"], g["dr"], rows=rows)
    packed = g["packed"].cpu().numpy().view(np.uint32)[rows]
    idx = O.unpack(packed, Ka * Kp, wl.d)
    ia, ip = idx // Kp, idx % Kp
    ok = P.accept_polar(enc["zt"].reshape(-1, 2), g["lv"], g["dr"], enc["ia"], enc["ip"], ia, ip)
    n_diff = int((idx != enc["idx"]).sum())
    say(f"  polar {Ka}x{Kp}: {len(rows)} rows, {idx.size} pairs, {n_diff} differ, "
        f"{int((~ok).sum())} beyond near-tie tolerance")
    assert ok.all()
    assert n_diff <= max(2, idx.size // 100000)
    rn = g["rn"].cpu().numpy().view(np.uint16)[rows]
    assert np.array_equal(rn, enc["rho_hat_bits"]) or \
        np.max(np.abs(rn.astype(np.int64) - enc["rho_hat_bits"].astype(np.int64))) <= 1
    B = O.index_bits(Ka * Kp)
    used = (wl.d // 2) * B
    if used % 32:
        assert not (packed[:, used // 32] >> np.uint32(used % 32)).any()
    assert not packed[:, -(-used // 32):].any()
    return enc


SHAPES = [
    # (N, d, block, Ka, Kp, wdtype, alpha, seed)
    (5, 48, 16, 8, 32, "f32", 0.5, 1),        # one window, ragged chunk count
    (9, 1088, 64, 8, 16, "bf16", 0.5, 2),     # two windows, second ragged
    (17, 2560, 128, 32, 64, "f32", 0.0, 3),   # 11 bits
    (6, 3072, 256, 16, 256, "bf16", 1.0, 4),  # 12 bits, 256 directions
    (4, 512, 512, 1, 8, "f32", 0.5, 5),       # one amplitude level
    (4, 256, 128, 4, 1, "bf16", 0.5, 6),      # one direction
    (3, 64, 32, 2, 2, "f32", 0.5, 7),         # 2 bits
    (2, 1024, 1024, 4, 8, "bf16", 0.5, 8),
]


@pytest.mark.parametrize("N,d,block,Ka,Kp,wdtype,alpha,seed", SHAPES)
def test_polar_shapes(q, N, d, block, Ka, Kp, wdtype, alpha, seed):
    rng = np.random.default_rng(3000 + seed)
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    if N > 2:
        W[1] = 0.0                                    # a zero row codes z~ = 0
    r = rng.lognormal(0.0, 1.0, d).astype(np.float32)
    if wdtype == "bf16":
        W = workloads.bf16_bits_from_f32(W)
    wl = workloads.Workload(f"polar{seed}", W, wdtype, r, alpha, block, seed * 777, Ka * Kp)
    say(f"case polar shapes N={N} d={d} b={block} {Ka}x{Kp} {wdtype} alpha={alpha}")
    g = run_polar(q, wl, Ka, Kp)
    enc = check_rows(wl, g, np.arange(N), Ka, Kp)
    if N > 2:
        assert not enc["idx"][1].any()
    # decode with the product table through the joint decoder
    Ct = torch.from_numpy(g["tb"]).to(DEV)
    Wh = q.qamw_decode(g["packed"], g["rn"], d, g["s"], g["sigma"], block, wl.sign_seed, Ct)
    torch.cuda.synchronize()
    ref = O.decode(g["packed"].cpu().numpy().view(np.uint32), g["rn"].cpu().numpy().view(np.uint16),
                   g["s"].cpu().numpy(), g["sigma"].cpu().numpy(), block, wl.sign_seed, g["tb"], d)
    err = float(np.max(np.abs(Wh.cpu().numpy().astype(np.float64) - ref)))
    say(f"  decode fp32 max abs err {err:.3e}")
    assert err <= 1e-5


def test_polar_full_size_ablation(q):
    """4096 x 11008 bf16 at 8 bits per pair: sampled-row parity and the
    joint-versus-polar reconstruction error."""
    wl = workloads.get("c3t_4096x11008")
    Ka, Kp = 8, 32
    say(f"case polar full {wl.N}x{wl.d} {Ka}x{Kp}")
    g = run_polar(q, wl, Ka, Kp)
    rows = np.random.default_rng(41).choice(wl.N, 24, replace=False)
    rows[0] = wl.N - 1
    check_rows(wl, g, np.sort(rows), Ka, Kp)
    # joint K = 256 at the same rate
    C = q.load_codebook(Ka * Kp)
    Ct = torch.from_numpy(C).to(DEV)
    packed_j, rn_j = q.qamw_encode(g["W"], g["s"], g["sigma"], wl.block, wl.sign_seed, Ct)
    Wf = g["W"].float()
    Wh_j = q.qamw_decode(packed_j, rn_j, wl.d, g["s"], g["sigma"], wl.block, wl.sign_seed, Ct)
    Wh_p = q.qamw_decode(g["packed"], g["rn"], wl.d, g["s"], g["sigma"], wl.block, wl.sign_seed,
                         torch.from_numpy(g["tb"]).to(DEV))
    e_j = float(torch.linalg.norm(Wh_j - Wf) / torch.linalg.norm(Wf))
    e_p = float(torch.linalg.norm(Wh_p - Wf) / torch.linalg.norm(Wf))
    say(f"  relative error: joint K=256 {e_j:.5f}, polar 8x32 {e_p:.5f}")
    assert e_j < e_p


def test_polar_extreme_sigma(q):
    """Caller-supplied pair scales that make |z~| huge (past the threshold
    count's safe range: the kernel takes the definition itself) or tiny
    (scores could underflow: every direction is scanned)."""
    N, d, block, Ka, Kp = 6, 512, 128, 8, 32
    rng = np.random.default_rng(77)
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    s = np.ones(d, np.float32)
    sigma = np.full(d // 2, 0.05, np.float32)
    sigma[0::4] = 1e-9          # |z~| ~ 1e7
    sigma[1::4] = 1e15          # |z~| ~ 1e-16
    sigma[2::8] = 0.0           # codes z~ = 0
    lv, dr, tb = q.load_polar(Ka, Kp)
    seed = 4242
    say(f"case polar extreme sigma N={N} d={d} {Ka}x{Kp}")
    packed, rn = q.qamw_encode_polar(torch.from_numpy(W).to(DEV), torch.from_numpy(s).to(DEV),
                                     torch.from_numpy(sigma).to(DEV), block, seed,
                                     torch.from_numpy(lv).to(DEV), torch.from_numpy(dr).to(DEV))
    torch.cuda.synchronize()
    enc = P.encode_polar(W, s, sigma, block, seed, lv, dr)
    idx = O.unpack(packed.cpu().numpy().view(np.uint32), Ka * Kp, d)
    ia, ip = idx // Kp, idx % Kp
    ok = P.accept_polar(enc["zt"].reshape(-1, 2), lv, dr, enc["ia"], enc["ip"], ia, ip)
    big = np.repeat((sigma == np.float32(1e-9))[None, :], N, 0)
    say(f"  {int((idx != enc['idx']).sum())} differ of {idx.size}; huge pairs identical: "
        f"{bool(np.array_equal(idx[big], enc['idx'][big]))}")
    assert ok.all()
    tiny = np.repeat((sigma == np.float32(1e15))[None, :], N, 0)
    assert big.any() and tiny.any()
    assert np.array_equal(ip[tiny], enc["ip"][tiny])
    zero = np.repeat((sigma == 0.0)[None, :], N, 0)
    assert not idx[zero].any()
