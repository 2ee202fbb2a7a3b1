"""GPU parity of the activation statistics and the layer-output error
(qamw_channel_rms, qamw_output_error) against the oracle
(oracle/output_error.py); needs an MI355X.

Criteria:
  * channel RMS: relative error <= 1e-5 (fp32 tile sums of squares, fp64
    across tiles); two calls bit-identical.
  * output error on the operands the kernel multiplies -- X and W - W^
    rounded to bf16 (test-side rounding of inputs) -- relative error
    <= 1e-5 (fp32 MFMA accumulation); against the exact fp64 error of the
    unrounded operands, <= 1e-2 (bf16 rounding of X and dW, ~2^-9 each).
  * the scaled codec's output error is smallest at alpha = 1/2 (the
    Cauchy-Schwarz optimum for i.i.d. weights), with the channel RMS from
    the GPU and every step of the codec on the GPU.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import output_error as E

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


def dev(a, dt):
    """fp32 numpy -> device tensor of dtype dt ('f32' or 'bf16', RNE), and the fp64 values it holds."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dt == "bf16":
        bits = workloads.bf16_bits_from_f32(a)
        return (torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16),
                workloads.bf16_bits_to_f32(bits).astype(np.float64))
    return torch.from_numpy(a).to(DEV), a.astype(np.float64)


def bf16_round(a):
    return workloads.bf16_bits_to_f32(workloads.bf16_bits_from_f32(np.asarray(a, np.float32))).astype(np.float64)


@pytest.mark.parametrize("T,d,dt", [(1, 8, "f32"), (63, 24, "bf16"), (1000, 4096, "f32"), (2048, 11008, "bf16")])
def test_channel_rms(q, T, d, dt):
    say(f"case channel_rms T={T} d={d} {dt}")
    r = workloads.channel_rms(d, sigma_log=1.2, seed=T + d)
    Xt, X64 = dev(workloads.activations(T, r, seed=5 + T), dt)
    got = q.qamw_channel_rms(Xt)
    got2 = q.qamw_channel_rms(Xt)
    torch.cuda.synchronize()
    assert torch.equal(got, got2)
    ref = E.channel_rms(X64)
    rel = float(np.max(np.abs(got.cpu().numpy() - ref) / ref))
    say(f"  max relative error {rel:.2e}")
    assert rel <= 1e-5


OE_CASES = [
    # (T, N, d, xdt, wdt, hdt)
    (1, 1, 16, "f32", "f32", "f32"),          # one token, one row, one 16-column group (zero tail of the step)
    (19, 37, 160, "bf16", "bf16", "f32"),     # ragged 128-blocks
    (130, 129, 48, "f32", "bf16", "bf16"),    # second token and row blocks hold one entry
    (300, 260, 1024, "bf16", "f32", "f32"),
]


@pytest.mark.parametrize("T,N,d,xdt,wdt,hdt", OE_CASES)
def test_output_error(q, T, N, d, xdt, wdt, hdt):
    say(f"case output_error T={T} N={N} d={d} X {xdt} W {wdt} W^ {hdt}")
    rng = np.random.default_rng(T * 1000 + N)
    r = workloads.channel_rms(d, sigma_log=1.0, seed=d)
    Xt, X64 = dev(workloads.activations(T, r, seed=T), xdt)
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    Wt, W64 = dev(W, wdt)
    Wh = (W64 + rng.standard_normal((N, d)) * 0.002).astype(np.float32)
    Wht, Wh64 = dev(Wh, hdt)
    got = float(q.qamw_output_error(Xt, Wt, Wht).cpu()[0])
    got2 = float(q.qamw_output_error(Xt, Wt, Wht).cpu()[0])
    assert got == got2
    # the operands the kernel multiplies: bf16(X), bf16(fp32(W - W^))
    dW_b = bf16_round(W64.astype(np.float32) - Wh64.astype(np.float32))
    ref_b = E.output_error(dW_b, np.zeros_like(dW_b), bf16_round(X64))
    ref = E.output_error(W64, Wh64, X64)
    say(f"  E={got:.6e}  vs rounded operands {abs(got - ref_b) / ref_b:.2e}, vs exact {abs(got - ref) / ref:.2e}")
    assert abs(got - ref_b) <= 1e-5 * ref_b
    assert abs(got - ref) <= 1e-2 * ref


def test_output_error_full_width_sampled_rows(q):
    """The headline shape's width (d = 11008) on 64 sampled rows and 256 tokens."""
    wl = workloads.get("c3t_4096x11008")
    rows = np.sort(np.random.default_rng(3).choice(wl.N, 64, replace=False))
    W = wl.W_f32()[rows]
    rng = np.random.default_rng(4)
    Wh = (W + rng.standard_normal(W.shape) * 0.001).astype(np.float32)
    Xt, X64 = dev(workloads.activations(256, wl.r, seed=8), "bf16")
    Wt, W64 = dev(W, "bf16")
    Wht, Wh64 = dev(Wh, "f32")
    say(f"case output_error sampled rows T=256 N=64 d={wl.d}")
    got = float(q.qamw_output_error(Xt, Wt, Wht).cpu()[0])
    dW_b = bf16_round(W64.astype(np.float32) - Wh64.astype(np.float32))
    ref_b = E.output_error(dW_b, np.zeros_like(dW_b), X64)
    say(f"  relative difference {abs(got - ref_b) / ref_b:.2e}")
    assert abs(got - ref_b) <= 1e-5 * ref_b


def test_alpha_sweep_on_gpu(q):
    N, d, b, K, T, seed = 512, 2048, 128, 256, 512, 31
    rng = np.random.default_rng(12)
    W = torch.from_numpy((rng.standard_normal((N, d)) * 0.02).astype(np.float32)).to(DEV)
    r_true = workloads.channel_rms(d, sigma_log=1.2, seed=13)
    X = torch.from_numpy(workloads.activations(T, r_true, seed=14)).to(DEV)
    r = q.qamw_channel_rms(X)
    C = torch.from_numpy(q.load_codebook(K)).to(DEV)
    plan = q.qamw_build_plan(C)
    err = {}
    for alpha in (0.0, 0.25, 0.5, 0.75, 1.0):
        s, sigma = q.qamw_calibrate(W, r, alpha, b, seed)
        packed, rn = q.qamw_encode(W, s, sigma, b, seed, C, plan=plan)
        Wh = q.qamw_decode(packed, rn, d, s, sigma, b, seed, C)
        err[alpha] = float(q.qamw_output_error(X, W, Wh).cpu()[0])
        ref = E.output_error(W.cpu().numpy(), Wh.cpu().numpy(), X.cpu().numpy())
        assert abs(err[alpha] - ref) <= 1e-2 * ref
    say("case alpha sweep N=512 d=2048 K=256 T=512: " + ", ".join(f"{a}: {e:.4g}" for a, e in err.items()))
    assert err[0.5] == min(err.values())
