"""C ABI checks that need no GPU: the library loads, exports every function
include/qamw.h declares, its host helpers return the documented values, and
invalid arguments are rejected on the host before anything is launched."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qamw.h")


@pytest.fixture(scope="module")
def lib():
    from vector_codebook_codec_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqamw.so not built")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qamw_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("qamw_calibrate", "qamw_encode", "qamw_decode", "qamw_packed_row_words"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from vector_codebook_codec_amd import _lib

    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no Python binding"



def lds_plan_layout(K):
    """The plan layout for K <= 2048, written out: cell edges on 2048 bins over
    [-5, 5) with widths round(7 sqrt(2048 / K) exp(t^2 / 8)) clamped to
    [1, 255] bins (t: the inner edge's coordinate), mirrored about 0; an image
    of the bin map, G x G 16-bit entries and as many 8-byte list records as fit
    160 KB - 1 KB of LDS next to the codebook (8 K bytes), 16 wavefronts'
    64 B-byte packing stages and the encode kernel's own copy of the map and
    cells (the map with a guard bin at each end, 2050 bytes padded to 2064;
    the cells with a guard row and column, (G + 1)^2 16-bit entries padded to
    16 bytes)."""
    h, w0 = 10 / 2048, 7 * math.sqrt(2048 / K)
    pos = [1024]
    while pos[-1] < 2048:
        t = (pos[-1] - 1024) * h
        w = min(255, max(1, math.floor(w0 * math.exp(t * t / 8) + 0.5)))
        pos.append(min(2048, pos[-1] + w))
    edges = [2048 - p for p in reversed(pos[1:])] + pos
    G = len(edges) - 1
    B = math.ceil(math.log2(K))
    up = lambda v, a: -(-v // a) * a
    lists_off = 2048 + up(2 * G * G, 16)
    cap = min((159 * 1024 - 8 * K - 16 * 64 * B - 2064 - up(2 * (G + 1) ** 2, 16)) // 8, 32767) & ~1
    image = lists_off + 8 * cap
    ns2 = (-(-G // 8)) * (-(-G // 4))       # 8 x 4-cell supercells
    scratch = up(G * G * 4, 256) + up(ns2 * 4, 256) + ns2 * 64 * 8
    return dict(G=G, edges=edges, cap=cap, image_bytes=image,
                plan_bytes=up(256 + 128 * 128 * 16 + image, 256) + scratch)

def test_host_helpers(lib):
    for K in (2, 3, 4, 256, 257, 2048, 4096):
        assert lib.qamw_index_bits(K) == math.ceil(math.log2(K))
    assert lib.qamw_index_bits(1) == -1 and lib.qamw_index_bits(4097) == -1
    assert lib.qamw_packed_row_words(11008, 2048) == 1892
    assert lib.qamw_packed_row_words(4096, 2048) == 704
    assert lib.qamw_packed_row_words(13824, 4096) == 2592
    assert lib.qamw_packed_row_words(12, 2048) == 4
    assert lib.qamw_packed_row_words(13, 2048) == -1
    # rho (fp64) + column factors (fp32) + 1 / sigma (fp32), each 256-byte padded
    assert lib.qamw_encode_workspace_bytes(4096, 11008) == 4096 * 8 + 11008 * 4 + 5504 * 4
    assert lib.qamw_encode_workspace_bytes(5, 16) == 3 * 256
    assert lib.qamw_encode_workspace_bytes(0, 16) == 0
    # rho (fp64) + column factors (fp32), each 256-byte padded, + ceil(N / 16) tiles x d/2 fp32
    assert lib.qamw_calibrate_workspace_bytes(4096, 11008, 256) == 4096 * 8 + 11008 * 4 + 256 * 5504 * 4
    # rows of 5 to 16 windows: tiles of ceil(N / 256) rows (a multiple of 4, at least 16)
    assert lib.qamw_calibrate_workspace_bytes(5120, 13824, 128) == 5120 * 8 + 13824 * 4 + 256 * 6912 * 4
    assert lib.qamw_calibrate_workspace_bytes(5000, 8192, 128) == 40192 + 8192 * 4 + 250 * 4096 * 4   # rho padded to 256 B
    # up to 4 windows, or more than 16: 16-row tiles
    assert lib.qamw_calibrate_workspace_bytes(11008, 4096, 128) == 11008 * 8 + 4096 * 4 + 688 * 2048 * 4
    assert lib.qamw_calibrate_workspace_bytes(0, 16, 16) == 0
    assert lib.qamw_status_string(-4) == b"workspace missing or too small"
    # K > 2048: header block + one uint16 record of 16 entries per cell of the
    # uniform 512 x 512 grid and of the outer 128 x 128 grid; K <= 2048:
    # header, outer grid (8 entries), the LDS table image and its build scratch
    assert lib.qamw_plan_bytes(4096) == 256 + (512 ** 2 + 128 ** 2) * 16 * 2
    for K in (2, 16, 256, 1000, 2048):
        assert lib.qamw_plan_bytes(K) == lds_plan_layout(K)["plan_bytes"], K
    g = lds_plan_layout(2048)
    # the encode kernel's LDS: map with guards, codebook (-cx, -cy), cells with
    # a guard row and column, records, 16 packing stages
    lds = 2064 + 8 * 2048 + -(-2 * 151 ** 2 // 16) * 16 + 8 * g["cap"] + 16 * 64 * 11
    assert g["G"] == 150 and lds <= 159 * 1024
    assert lib.qamw_plan_bytes(1) == 0 and lib.qamw_plan_bytes(4097) == 0


# Fake, never-dereferenced device addresses: every call below must fail in
# host-side validation, before any HIP call.
A = 1 << 20           # 16-byte aligned
MIS = A + 4           # misaligned
WS = 1 << 24


def _encode(lib, **kw):
    args = dict(W=A, wdt=1, N=8, d=256, ldw=256, s=A, sigma=A, block=128, seed=0, cb=A, K=256, plan=None,
                plan_size=1 << 26, packed=A, rn=A, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_encode(args["W"], args["wdt"], args["N"], args["d"], args["ldw"], args["s"], args["sigma"],
                           args["block"], args["seed"], args["cb"], args["K"], args["plan"], args["plan_size"],
                           args["packed"], args["rn"], args["ws"], args["ws_bytes"], args["stream"])


def _prepare(lib, **kw):
    args = dict(W=A, wdt=1, N=8, d=256, ldw=256, s=A, sigma=A, block=128, seed=0, rn=A, ws=WS,
                ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_encode_prepare(args["W"], args["wdt"], args["N"], args["d"], args["ldw"], args["s"],
                                   args["sigma"], args["block"], args["seed"], args["rn"], args["ws"],
                                   args["ws_bytes"], args["stream"])


def _indices(lib, **kw):
    args = dict(W=A, wdt=1, N=8, d=256, ldw=256, block=128, cb=A, K=256, plan=None, plan_size=1 << 26, packed=A,
                ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_encode_indices(args["W"], args["wdt"], args["N"], args["d"], args["ldw"], args["block"],
                                   args["cb"], args["K"], args["plan"], args["plan_size"], args["packed"], args["ws"],
                                   args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(block=1), -2), (dict(N=0), -1), (dict(W=MIS), -1), (dict(s=None), -1), (dict(sigma=MIS), -1),
    (dict(rn=None), -1), (dict(ws=None), -4), (dict(ws_bytes=8), -4), (dict(ws=WS + 16), -4), (dict(wdt=2), -2),
])
def test_encode_prepare_rejects(lib, kw, status):
    assert _prepare(lib, **kw) == status
    assert lib.qamw_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(block=1), -2), (dict(K=1), -2), (dict(cb=MIS), -1), (dict(packed=None), -1), (dict(packed=MIS), -1),
    (dict(plan=WS + 64), -1), (dict(ws=None), -4), (dict(ws_bytes=100), -4), (dict(ldw=100), -1),
    (dict(plan=WS, plan_size=1000), -4), (dict(plan=WS, K=2048, plan_size=1 << 19), -4),
])
def test_encode_indices_rejects(lib, kw, status):
    assert _indices(lib, **kw) == status
    assert lib.qamw_last_error()


def _polar(lib, **kw):
    args = dict(W=A, wdt=1, N=8, d=256, ldw=256, s=A, sigma=A, block=128, seed=0, lv=A, Ka=8, dirs=A, Kp=32,
                packed=A, rn=A, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_encode_polar(args["W"], args["wdt"], args["N"], args["d"], args["ldw"], args["s"],
                                 args["sigma"], args["block"], args["seed"], args["lv"], args["Ka"], args["dirs"],
                                 args["Kp"], args["packed"], args["rn"], args["ws"], args["ws_bytes"],
                                 args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(block=1), -2), (dict(Ka=0), -2), (dict(Kp=0), -2), (dict(Ka=1, Kp=1), -2), (dict(Ka=64, Kp=128), -2),
    (dict(lv=None), -1), (dict(dirs=None), -1), (dict(packed=MIS), -1), (dict(s=None), -1), (dict(rn=None), -1),
    (dict(ws=None), -4), (dict(ws_bytes=100), -4), (dict(ldw=100), -1), (dict(wdt=2), -2),
])
def test_encode_polar_rejects(lib, kw, status):
    assert _polar(lib, **kw) == status
    assert lib.qamw_last_error()


def _rms(lib, **kw):
    args = dict(X=A, xdt=1, T=100, d=64, ldx=64, r=A, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_channel_rms(args["X"], args["xdt"], args["T"], args["d"], args["ldx"], args["r"], args["ws"],
                                args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), -1), (dict(d=12, ldx=16), -1), (dict(X=None), -1), (dict(X=MIS), -1), (dict(ldx=60), -1),
    (dict(ldx=68), -1), (dict(xdt=2), -2), (dict(r=None), -1), (dict(r=MIS), -1), (dict(ws=None), -4),
    (dict(ws_bytes=16), -4), (dict(ws=WS + 32), -4),
])
def test_channel_rms_rejects(lib, kw, status):
    assert _rms(lib, **kw) == status
    assert lib.qamw_last_error()


def _oe(lib, **kw):
    args = dict(X=A, xdt=1, T=100, d=64, ldx=64, W=A, wdt=1, N=50, ldw=64, H=A, hdt=0, ldh=64, out=A,
                ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_output_error(args["X"], args["xdt"], args["T"], args["d"], args["ldx"], args["W"], args["wdt"],
                                 args["N"], args["ldw"], args["H"], args["hdt"], args["ldh"], args["out"],
                                 args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), -1), (dict(d=40, ldx=40, ldw=40, ldh=40), -1), (dict(W=None), -1), (dict(H=MIS), -1),
    (dict(ldh=32), -1), (dict(hdt=2), -2), (dict(wdt=5), -2), (dict(out=None), -1), (dict(out=A + 4), -1),
    (dict(ws=None), -4), (dict(ws_bytes=8), -4),
])
def test_output_error_rejects(lib, kw, status):
    assert _oe(lib, **kw) == status
    assert lib.qamw_last_error()


def test_metric_workspace_sizes(lib):
    # one fp32 partial per (64-row tile, column)
    assert lib.qamw_channel_rms_workspace_bytes(2048, 11008) == 32 * 11008 * 4
    assert lib.qamw_channel_rms_workspace_bytes(65, 8) == 256
    # one fp64 partial per 128 x 128 block of X dW^T (row blocks rounded up to a multiple
    # of 8), bf16 dW [N][d] and bf16 X [T][d]
    assert lib.qamw_output_error_workspace_bytes(2048, 4096, 11008) == 32 * 16 * 8 + 4096 * 11008 * 2 + 2048 * 11008 * 2
    assert lib.qamw_output_error_workspace_bytes(64, 200, 16) == 256 + 200 * 16 * 2 + 64 * 16 * 2
    assert lib.qamw_output_error_workspace_bytes(0, 4, 16) == 0


def _cal_enc(lib, **kw):
    args = dict(W=A, wdt=1, N=8, d=256, ldw=256, r=A, alpha=0.5, block=128, seed=0, cb=A, K=256, plan=None,
                plan_size=1 << 26, s=A, sigma=A, packed=A, rn=A, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_calibrate_encode(args["W"], args["wdt"], args["N"], args["d"], args["ldw"], args["r"],
                                     args["alpha"], args["block"], args["seed"], args["cb"], args["K"], args["plan"],
                                     args["plan_size"], args["s"], args["sigma"], args["packed"], args["rn"],
                                     args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(block=1), -2), (dict(K=1), -2), (dict(r=None), -1), (dict(s=MIS), -1), (dict(packed=None), -1),
    (dict(rn=None), -1), (dict(alpha=float("nan")), -1), (dict(plan=WS + 64), -1), (dict(ws=None), -4),
    (dict(plan=WS, plan_size=4096), -4),
    (dict(ws_bytes=1000), -4), (dict(ldw=100), -1), (dict(wdt=2), -2),
])
def test_calibrate_encode_rejects(lib, kw, status):
    assert _cal_enc(lib, **kw) == status
    assert lib.qamw_last_error()


def _cal_prep(lib, **kw):
    args = dict(W=A, wdt=1, N=8, d=256, ldw=256, r=A, alpha=0.5, block=128, seed=0, s=A, sigma=A, rn=A, ws=WS,
                ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_calibrate_prepare(args["W"], args["wdt"], args["N"], args["d"], args["ldw"], args["r"],
                                      args["alpha"], args["block"], args["seed"], args["s"], args["sigma"],
                                      args["rn"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(block=1), -2), (dict(block=3), -2), (dict(block=8, d=264, ldw=264), -2), (dict(r=None), -1), (dict(s=MIS), -1),
    (dict(sigma=None), -1), (dict(rn=None), -1), (dict(alpha=float("inf")), -1), (dict(ws=None), -4),
    (dict(ws_bytes=1000), -4), (dict(ws=WS + 16), -4), (dict(wdt=7), -2), (dict(ldw=100), -1),
])
def test_calibrate_prepare_rejects(lib, kw, status):
    assert _cal_prep(lib, **kw) == status
    assert lib.qamw_last_error()


def test_calibrate_encode_workspace(lib):
    # the encode workspace followed by the calibration's partial sums
    assert lib.qamw_calibrate_encode_workspace_bytes(4096, 11008) == \
        lib.qamw_encode_workspace_bytes(4096, 11008) + 256 * 5504 * 4
    assert lib.qamw_calibrate_encode_workspace_bytes(0, 16) == 0


def _lloyd(lib, **kw):
    args = dict(W=A, wdt=1, N=8, d=256, ldw=256, block=128, packed=A, cb=A, K=256, enc=WS, enc_bytes=1 << 20,
                out=A + 4096, dist=A, ws=WS + (1 << 21), ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_lloyd_update(args["W"], args["wdt"], args["N"], args["d"], args["ldw"], args["block"],
                                 args["packed"], args["cb"], args["K"], args["enc"], args["enc_bytes"], args["out"],
                                 args["dist"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(block=1), -2), (dict(K=1), -2), (dict(packed=None), -1), (dict(packed=MIS), -1), (dict(out=None), -1),
    (dict(out=A), -1), (dict(dist=None), -1), (dict(dist=A + 4), -1), (dict(enc=None), -4), (dict(enc_bytes=64), -4),
    (dict(ws=None), -4), (dict(ws_bytes=1024), -4), (dict(ldw=100), -1),
])
def test_lloyd_update_rejects(lib, kw, status):
    assert _lloyd(lib, **kw) == status
    assert lib.qamw_last_error()


def test_learn_codebook_rejects(lib):
    # one invalid argument each (a fully valid set would launch: never called here)
    args = [A, 1, 8, 256, 256, 128, WS, 1 << 20, A, 256, 3, A + 4096, A, WS + (1 << 22), 1 << 24, A,
            WS + (1 << 21), 1 << 20, None]
    bad = list(args); bad[10] = 0                           # iters
    assert lib.qamw_learn_codebook(*bad) == -1
    bad = list(args); bad[11] = A                           # codebook_out aliases codebook_init
    assert lib.qamw_learn_codebook(*bad) == -1
    bad = list(args); bad[14] = 1000                        # plan too small
    assert lib.qamw_learn_codebook(*bad) == -4


def test_lloyd_workspace(lib):
    # 3 x K int64 sums, 4096 fp64 partials, a spare K x 2 codebook; 256-byte padded each
    assert lib.qamw_lloyd_workspace_bytes(2048) == 3 * 2048 * 8 + 4096 * 8 + 2048 * 8
    assert lib.qamw_lloyd_workspace_bytes(1) == 0


def _calibrate(lib, **kw):
    args = dict(W=A, wdt=0, N=8, d=256, ldw=256, r=A, alpha=0.5, block=128, seed=0, s=A, sigma=A,
                ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return lib.qamw_calibrate(args["W"], args["wdt"], args["N"], args["d"], args["ldw"], args["r"],
                              args["alpha"], args["block"], args["seed"], args["s"], args["sigma"], args["ws"],
                              args["ws_bytes"], args["stream"])


def _decode(lib, **kw):
    args = dict(packed=A, rn=A, N=8, d=256, s=A, sigma=A, block=128, seed=0, cb=A, K=256, out=A, odt=0,
                ldo=256, stream=None)
    args.update(kw)
    return lib.qamw_decode(args["packed"], args["rn"], args["N"], args["d"], args["s"], args["sigma"],
                           args["block"], args["seed"], args["cb"], args["K"], args["out"], args["odt"],
                           args["ldo"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(block=3), -2), (dict(block=1), -2), (dict(block=8, d=264), -2), (dict(block=2048), -2), (dict(block=128, d=320), -1),
    (dict(N=0), -1), (dict(d=-16), -1), (dict(K=1), -2), (dict(K=4097), -2), (dict(ldw=128), -1),
    (dict(W=None), -1), (dict(cb=None), -1), (dict(s=None), -1), (dict(packed=None), -1),
    (dict(W=MIS), -1), (dict(packed=MIS), -1), (dict(wdt=2), -2), (dict(ldw=260), -1),
    (dict(ws=None), -4), (dict(ws_bytes=8), -4), (dict(ws=WS + 16), -4), (dict(cb=MIS), -1),
    (dict(plan=WS + 128), -1), (dict(plan=WS, plan_size=1000), -4),
])
def test_encode_rejects(lib, kw, status):
    assert _encode(lib, **kw) == status
    assert lib.qamw_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(alpha=float("nan")), -1), (dict(alpha=float("inf")), -1), (dict(r=None), -1),
    (dict(sigma=None), -1), (dict(s=MIS), -1), (dict(ws_bytes=500), -4), (dict(block=32, d=48), -1),
])
def test_calibrate_rejects(lib, kw, status):
    assert _calibrate(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(odt=3), -2), (dict(ldo=100), -1), (dict(out=MIS), -1), (dict(rn=None), -1),
    (dict(K=5000), -2), (dict(block=64, d=96), -1), (dict(odt=1, ldo=260), -1), (dict(cb=MIS), -1),
])
def test_decode_rejects(lib, kw, status):
    assert _decode(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(cb=None), -1), (dict(cb=MIS), -1), (dict(K=1), -2), (dict(K=5000), -2), (dict(plan=None), -1),
    (dict(plan=WS + 16), -1), (dict(size=1000), -4), (dict(K=4096, size=256 + (512 ** 2 + 256 ** 2) * 16), -4),
])
def test_build_plan_rejects(lib, kw, status):
    args = dict(cb=A, K=2048, plan=WS, size=1 << 23, stream=None)
    args.update(kw)
    assert lib.qamw_build_plan(args["cb"], args["K"], args["plan"], args["size"], args["stream"]) == status
    assert lib.qamw_last_error()


def test_workspace_size_is_enforced(lib):
    need = lib.qamw_calibrate_workspace_bytes(8, 256, 128)
    assert _calibrate(lib, ws_bytes=need - 1) == -4


@pytest.mark.parametrize("kw,status", [
    (dict(block=1), -2), (dict(T=0), -1), (dict(X=None), -1), (dict(X=MIS), -1), (dict(xdt=2), -2),
    (dict(out=None), -1), (dict(out=MIS), -1), (dict(ldr=260), -1), (dict(ldx=100), -1), (dict(s=MIS), -1),
])
def test_rotate_activations_rejects(lib, kw, status):
    args = dict(X=A, xdt=1, T=4, d=256, ldx=256, s=A, block=128, seed=0, out=A, ldr=256, stream=None)
    args.update(kw)
    assert lib.qamw_rotate_activations(args["X"], args["xdt"], args["T"], args["d"], args["ldx"], args["s"],
                                       args["block"], args["seed"], args["out"], args["ldr"],
                                       args["stream"]) == status
    assert lib.qamw_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), -1), (dict(N=0), -1), (dict(d=40), -1), (dict(K=1), -2), (dict(cb=MIS), -1), (dict(Xr=None), -1),
    (dict(Xr=MIS), -1), (dict(packed=MIS), -1), (dict(ydt=2), -2), (dict(ldy=2), -1), (dict(ldr=100), -1),
    (dict(ldr=260), -1), (dict(Y=None), -1),
])
def test_decode_matmul_rejects(lib, kw, status):
    args = dict(Xr=A, T=4, d=256, ldr=256, packed=A, rn=A, N=8, sigma=A, cb=A, K=256, Y=A, ydt=0, ldy=8,
                stream=None)
    args.update(kw)
    assert lib.qamw_decode_matmul(args["Xr"], args["T"], args["d"], args["ldr"], args["packed"], args["rn"],
                                  args["N"], args["sigma"], args["cb"], args["K"], args["Y"], args["ydt"],
                                  args["ldy"], args["stream"]) == status
    assert lib.qamw_last_error()


def test_encode_noalloc_rejects_before_any_device_call(lib):
    """The no-allocation encode refuses sizes beyond its 1 MiB per-GPU
    workspace, and bad arguments, on the host before looking up the device."""
    assert lib.qamw_encode_noalloc_scratch_bytes() == 1 << 20
    args = [A, 1, 8, 256, 256, A, A, 128, 0, A, 256, None, 0, A, A, None]
    big = list(args)
    big[2] = 1 << 17                      # 2^17 fp64 row norms alone fill 1 MiB
    assert lib.qamw_encode_noalloc(*big) == -2
    assert b"no-allocation" in lib.qamw_last_error()
    bad = list(args)
    bad[7] = 3                            # block
    assert lib.qamw_encode_noalloc(*bad) == -2
    bad = list(args)
    bad[13] = MIS                         # packed misaligned
    assert lib.qamw_encode_noalloc(*bad) == -1
    bad = list(args)
    bad[11], bad[12] = WS, 100            # a plan too small for K
    assert lib.qamw_encode_noalloc(*bad) == -4
