"""GPU parity of the codebook refinement on a matrix's own pairs
(qamw_lloyd_update, qamw_learn_codebook) against the oracle
(oracle/lloyd.py: refine_on_pairs); needs an MI355X.

Criteria:
  * one update, on the GPU's own assignment: every centroid within
    1e-6 (1 + |c|) of the fp64 mean of its pairs (the GPU's z~ is fp32, its
    sums fixed point of 2^-28) -- an unused centroid keeps its value
    exactly -- and the distortion within 1e-5 relative; the GPU's assignment
    agrees with the oracle's up to near-ties.
  * several rounds: distortions within 1e-4 relative of the oracle's and the
    codebooks within 1e-4 (a near-tie reassignment moves a mean by at most
    |z~ - c| / count).
  * at the headline size: distortion falls round by round, the learned
    codebook reconstructs the matrix better than the Gaussian one, and two
    runs are bit-identical.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import lloyd
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


def prepare(q, wl, K):
    W = to_dev(wl.W, wl.wdtype)
    r = torch.from_numpy(wl.r).to(DEV)
    C = torch.from_numpy(q.load_codebook(K)).to(DEV)
    ws = torch.empty(q.qamw_calibrate_encode_workspace_bytes(wl.N, wl.d), dtype=torch.uint8, device=DEV)
    plan = q.qamw_build_plan(C)
    s, sigma, packed, rn = q.qamw_calibrate_encode(W, r, wl.alpha, wl.block, wl.sign_seed, C, plan=plan,
                                                   workspace=ws)
    return W, C, ws, s, sigma, packed


@pytest.mark.parametrize("K", [256, 4096])
def test_one_update(q, K):
    wl = workloads.get("c1_256x512")
    say(f"case lloyd update c1 K={K}")
    W, C, ws, s, sigma, packed = prepare(q, wl, K)
    C1, dist = q.qamw_lloyd_update(W, wl.block, packed, C, ws)
    torch.cuda.synchronize()
    Zt, _ = O.normalized_pairs(wl.W_f32(), s.cpu().numpy(), sigma.cpu().numpy(), wl.block, wl.sign_seed)
    Z = Zt.reshape(-1, 2)
    idx = O.unpack(packed.cpu().numpy().view(np.uint32), K, wl.d).reshape(-1)
    C0 = C.cpu().numpy()
    mean, cnt = lloyd.cell_means(Z, idx, K)
    ref = np.where(cnt[:, None] > 0, mean, C0.astype(np.float64))
    got = C1.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    say(f"  {int((cnt == 0).sum())} empty cells; max relative centroid error {err.max():.2e}")
    assert err.max() <= 1e-6
    assert np.array_equal(got[cnt == 0], C0[cnt == 0].astype(np.float64))
    d_ref = float(np.mean(np.sum((Z - C0.astype(np.float64)[idx]) ** 2, axis=1)))
    assert abs(float(dist.cpu()[0]) - d_ref) <= 1e-5 * d_ref
    own = np.concatenate([O.nearest_centroid(Z[a:a + 8192], C0)[0] for a in range(0, len(Z), 8192)])
    assert O.accept_index(Z, C0, own, idx).all()


def test_rounds_match_the_oracle(q):
    wl = workloads.get("c1_256x512")
    K, iters = 256, 4
    say(f"case learn_codebook c1 K={K} iters={iters}")
    W, C, ws, s, sigma, _ = prepare(q, wl, K)
    Cl, dist = q.qamw_learn_codebook(W, wl.block, ws, C, iters)
    torch.cuda.synchronize()
    Zt, _ = O.normalized_pairs(wl.W_f32(), s.cpu().numpy(), sigma.cpu().numpy(), wl.block, wl.sign_seed)
    Cref, hist = lloyd.refine_on_pairs(Zt.reshape(-1, 2), C.cpu().numpy(), iters)
    d = dist.cpu().numpy()
    say("  distortion gpu " + ", ".join(f"{v:.6g}" for v in d) + " / oracle " + ", ".join(f"{v:.6g}" for v in hist))
    assert np.all(np.abs(d - hist) <= 1e-4 * np.asarray(hist))
    assert float(np.max(np.abs(Cl.cpu().numpy() - Cref))) <= 1e-4


def test_headline_refinement(q):
    wl = workloads.get("c3t_4096x11008")
    iters = 3
    say(f"case learn_codebook {wl.name} K={wl.K} iters={iters}")
    W, C, ws, s, sigma, packed = prepare(q, wl, wl.K)
    Cl, dist = q.qamw_learn_codebook(W, wl.block, ws, C, iters)
    Cl2, dist2 = q.qamw_learn_codebook(W, wl.block, ws, C, iters)
    torch.cuda.synchronize()
    assert torch.equal(Cl, Cl2) and torch.equal(dist, dist2)
    d = dist.cpu().numpy()
    assert np.all(np.diff(d) < 0), d
    plan = q.qamw_build_plan(Cl)
    packed_l, rn_l = q.qamw_encode(W, s, sigma, wl.block, wl.sign_seed, Cl, plan=plan)
    rn = q.qamw_encode(W, s, sigma, wl.block, wl.sign_seed, C, plan=q.qamw_build_plan(C))[1]
    Wf = W.float()
    e0 = float(torch.linalg.norm(q.qamw_decode(packed, rn, wl.d, s, sigma, wl.block, wl.sign_seed, C) - Wf))
    e1 = float(torch.linalg.norm(q.qamw_decode(packed_l, rn_l, wl.d, s, sigma, wl.block, wl.sign_seed, Cl) - Wf))
    say(f"  distortion by round {d}; reconstruction error Gaussian codebook {e0:.5g}, learned {e1:.5g}")
    assert e1 < e0


def test_empty_cell_keeps_its_centroid(q):
    wl = workloads.get("c1_256x512")
    say("case lloyd update with an unused centroid")
    W = to_dev(wl.W, wl.wdtype)
    r = torch.from_numpy(wl.r).to(DEV)
    C0 = q.load_codebook(256).copy()
    C0[7] = (50.0, -50.0)                       # far from every pair
    C = torch.from_numpy(C0).to(DEV)
    ws = torch.empty(q.qamw_calibrate_encode_workspace_bytes(wl.N, wl.d), dtype=torch.uint8, device=DEV)
    s, sigma, packed, rn = q.qamw_calibrate_encode(W, r, wl.alpha, wl.block, wl.sign_seed, C, workspace=ws)
    C1, _ = q.qamw_lloyd_update(W, wl.block, packed, C, ws)
    torch.cuda.synchronize()
    assert not (O.unpack(packed.cpu().numpy().view(np.uint32), 256, wl.d) == 7).any()
    assert np.array_equal(C1.cpu().numpy()[7], C0[7])
