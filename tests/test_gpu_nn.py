"""GPU parity of the untransposed product (transpose = 0): the stored expert
weight [E, K, N], quantised along N, applied as x @ w_hat[e] (the backward
pass's orientation of the forward call's weight), against the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_torch, bf16_u16_to_f64, check_gate, i32_to_torch, torch_bf16_to_u16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_grouped_amd as mq
    mq.load()                       # fail loudly if the library is missing
    return torch.device("cuda:0")


def _mq():
    import quantized_moe_grouped_amd as mq
    return mq


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def nn_case(name, T, A, E, K, N, seed, **kw):
    """x [T, Ax, M, K], routing, and a stored weight [E, K, N] (bf16 bits)."""
    case = workloads.gather_case(name, T, A, E, K, N, seed=seed, **kw)
    w = np.ascontiguousarray(case.w.transpose(0, 2, 1))             # [E, K, N]
    return case, w


def gpu_nn(case, w, dev, gs, bits, ret_ws=False, sorted_hint=False):
    mq = _mq()
    wq, s, b = mq.mq_quantize(bf16_to_torch(w, dev), gs, bits)
    res = mq.mq_gather_qmm(bf16_to_torch(case.x, dev), wq, s, b, i32_to_torch(case.idx, dev),
                           False, gs, bits, sorted_hint, return_workspace=ret_ws)
    torch.cuda.synchronize()
    return res


def oracle_nn(case, w, gs, bits):
    owq, os_, ob = oracle.quantize(w, gs, bits)
    return oracle.gather_qmm(case.x, owq, os_, ob, case.idx, gs, bits, transpose=False)


NN_SHAPES = [
    # name, T, A, E, K, N, gs, bits, kwargs
    ("tiny", 64, 2, 8, 256, 128, 64, 4, {}),
    ("8bit-gs32", 48, 4, 6, 192, 96, 32, 8, {}),
    ("4bit-gs32-ragged-N", 40, 2, 4, 128, 160, 32, 4, {}),        # N % 64 = 32
    ("8bit-gs64", 30, 2, 4, 320, 64, 64, 8, {}),
    ("M2-broadcast", 24, 3, 5, 128, 64, 64, 4, dict(M=2, Ax=1)),
    ("E1", 50, 2, 1, 128, 192, 64, 4, {}),
    ("long-K", 16, 2, 3, 2048, 128, 64, 4, {}),
    ("zipf-skewed", 128, 2, 8, 256, 128, 32, 4, dict(routing="zipf", zipf_s=2.5)),
    ("many-experts-short-runs", 64, 8, 256, 128, 64, 64, 4, dict(routing="balanced")),
    ("decode", 4, 8, 64, 512, 256, 64, 4, {}),
]


@pytest.mark.parametrize("name,T,A,E,K,N,gs,bits,kw", NN_SHAPES, ids=[s[0] for s in NN_SHAPES])
def test_nn_shapes(dev, name, T, A, E, K, N, gs, bits, kw):
    case, w = nn_case(name, T, A, E, K, N, 81, **kw)
    _say(f"transpose=0 {name}")
    out = gpu_nn(case, w, dev, gs, bits)
    assert tuple(out.shape) == (T, A, case.M, N)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_nn(case, w, gs, bits), name)


@pytest.mark.parametrize("bm", ["16", "32", "64", "128"])
@pytest.mark.parametrize("gs,bits", [(64, 4), (32, 8)])
def test_nn_every_tile_height(dev, bm, gs, bits, monkeypatch):
    monkeypatch.setenv("MQ_FORCE_BM", bm)
    case, w = nn_case("nn-bm", 200, 4, 6, 256, 192, 82)
    _say(f"transpose=0 BM={bm} gs={gs} bits={bits}")
    out = gpu_nn(case, w, dev, gs, bits)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_nn(case, w, gs, bits),
               f"BM={bm} gs={gs} bits={bits}")


def test_nn_pages_shape_full_output(dev):
    """The shape of the pages' untransposed timing: E=4, K=D=512, 1024 routed
    rows (uniform routing), 4-bit groups of 64; every output."""
    case, w = nn_case("nn-E4-K512-B1024", 1024, 1, 4, 512, 512, 83)
    _say("transpose=0 E=4 K=D=512 B=1024")
    out, ws, L = gpu_nn(case, w, dev, 64, 4, ret_ws=True)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)), oracle_nn(case, w, 64, 4), "pages shape")
    _, ooff, operm = oracle.route(case.idx, case.E)
    off = ws[L.offsets:L.offsets + 4 * (case.E + 1)].view(torch.int32).cpu().numpy()
    perm = ws[L.perm:L.perm + 4 * case.idx.size].view(torch.int32).cpu().numpy()
    assert np.array_equal(off, ooff) and np.array_equal(perm, operm)


def test_nn_is_the_vjp_of_the_forward_call(dev):
    """One quantised stack serves both orientations: forward y = x w_hat^T
    (transpose=1, x with K features) and the backward product g w_hat
    (transpose=0, g with N features), each against the oracle; and
    <g, x w_hat^T> = <g w_hat, x> (the adjoint identity) holds for the GPU
    results to fp32-summation accuracy."""
    mq = _mq()
    T, A, E, K, N = 96, 2, 4, 256, 192
    case = workloads.gather_case("vjp", T, A, E, K, N, seed=84)            # w [E, N, K]
    g = workloads.gather_case("vjp-g", T, A, E, N, 8, seed=85).x          # [T, A, 1, N]
    wq, s, b = mq.mq_quantize(bf16_to_torch(case.w, dev), 64, 4)
    idx = i32_to_torch(case.idx, dev)
    y = mq.mq_gather_qmm(bf16_to_torch(case.x, dev), wq, s, b, idx, True, 64, 4, False)
    dx = mq.mq_gather_qmm(bf16_to_torch(g, dev), wq, s, b, idx, False, 64, 4, False)
    torch.cuda.synchronize()
    owq, os_, ob = oracle.quantize(case.w, 64, 4)
    y_ref = oracle.gather_qmm(case.x, owq, os_, ob, case.idx, 64, 4, transpose=True)
    dx_ref = oracle.gather_qmm(g, owq, os_, ob, case.idx, 64, 4, transpose=False)
    yo = bf16_u16_to_f64(torch_bf16_to_u16(y))
    dxo = bf16_u16_to_f64(torch_bf16_to_u16(dx))
    check_gate(yo, y_ref, "forward")
    check_gate(dxo, dx_ref, "backward (transpose=0)")
    gx = bf16_u16_to_f64(g)
    xx = bf16_u16_to_f64(case.x)
    lhs = float((gx * y_ref).sum())
    rhs = float((dx_ref * xx).sum())
    assert abs(lhs - rhs) <= 1e-9 * float(np.abs(gx * y_ref).sum())   # the oracle's identity
    # the GPU results satisfy it up to their own deviations from the oracle
    bound = float((np.abs(gx) * np.abs(yo - y_ref)).sum() + (np.abs(xx) * np.abs(dxo - dx_ref)).sum())
    assert abs(float((gx * yo).sum()) - float((dxo * xx).sum())) <= bound + 1e-9 * abs(lhs) + 1e-12


def test_nn_out_of_range_rows_zero(dev):
    case, w = nn_case("nn-oob", 20, 2, 4, 128, 64, 86)
    bad = case.idx.copy()
    bad[3, 1] = 4
    bad[7, 0] = -3
    case.idx = bad
    out, ws, L = gpu_nn(case, w, dev, 64, 4, ret_ws=True)
    o = bf16_u16_to_f64(torch_bf16_to_u16(out)).reshape(-1, 64)
    flat = bad.reshape(-1)
    ok = (flat >= 0) & (flat < 4)
    assert (o[~ok] == 0).all()
    assert ws[L.error:L.error + 4].view(torch.int32).item() == int((~ok).sum())
    good = workloads.GatherCase("ok", case.x.reshape(40, 1, 1, 128)[ok], case.w,
                                flat[ok].reshape(-1, 1).astype(np.int32), 4)
    check_gate(o[ok].reshape(-1, 1, 1, 64), oracle_nn(good, w, 64, 4), "valid rows")


def test_nn_presorted_and_deterministic(dev):
    case, w = nn_case("nn-sort", 150, 4, 8, 256, 128, 87)
    sc, order = workloads.presort(case)
    a = torch_bf16_to_u16(gpu_nn(case, w, dev, 64, 4)).reshape(-1, 128)
    b = torch_bf16_to_u16(gpu_nn(sc, w, dev, 64, 4, sorted_hint=True)).reshape(-1, 128)
    c = torch_bf16_to_u16(gpu_nn(case, w, dev, 64, 4)).reshape(-1, 128)
    assert np.array_equal(b, a[order])
    assert np.array_equal(a, c)


def test_nn_routed_call_matches(dev):
    """mq_gather_route + mq_gather_qmm_routed(transpose=0) gives the bits of
    mq_gather_qmm(transpose=0)."""
    mq = _mq()
    case, w = nn_case("nn-routed", 100, 4, 8, 256, 192, 88)
    full = torch_bf16_to_u16(gpu_nn(case, w, dev, 64, 4))
    wq, s, b = mq.mq_quantize(bf16_to_torch(w, dev), 64, 4)
    L = mq.mq_gather_qmm_workspace(case.T, case.A, 1, case.K, 192, case.E, 64, 4)
    ws = torch.empty(L.total, dtype=torch.uint8, device=dev)
    mq.mq_gather_route(i32_to_torch(case.idx, dev), case.E, 1, workspace=ws, K=case.K)
    out = mq.mq_gather_qmm_routed(bf16_to_torch(case.x, dev), wq, s, b, case.A, ws, False, 64, 4)
    torch.cuda.synchronize()
    assert np.array_equal(torch_bf16_to_u16(out), full)


@pytest.mark.parametrize("M", [1, 7, 16, 100, 300])
@pytest.mark.parametrize("gs,bits", [(64, 4), (32, 8)])
def test_nn_dense(dev, M, gs, bits):
    """mq_qmm(transpose=0): x [M, K] @ w_hat [K, N]."""
    K, N = 320, 384
    _, w_nk = workloads.small_m_dense(1, K, N, seed=M)             # [320, 384], stored as [K, N]
    x = workloads.small_m_dense(M, 8, K, seed=M + 90)[0]            # x [M, K]
    mq = _mq()
    wq, s, b = mq.mq_quantize(bf16_to_torch(w_nk, dev), gs, bits)  # stored [K=320, N=384]
    out = mq.mq_qmm(bf16_to_torch(x, dev), wq, s, b, False, gs, bits)
    torch.cuda.synchronize()
    owq, os_, ob = oracle.quantize(w_nk, gs, bits)
    check_gate(bf16_u16_to_f64(torch_bf16_to_u16(out)),
               oracle.qmm(x, owq, os_, ob, gs, bits, transpose=False), f"dense nn M={M}")
