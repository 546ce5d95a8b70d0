"""mq_gather_qmm_noalloc on the GPU: the entry point that takes no workspace
(the library's own per-GPU scratch) against mq_gather_qmm with a caller
workspace, through the C ABI, on consecutive calls of shrinking size."""
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


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


# three calls in a row, each smaller than the one before: a prefill-sized
# tiled GEMM (128-row tiles), short runs (32-row tiles), and a decode step
# (the small-M kernel, which routes the pairs itself)
CALLS = [
    ("prefill-like", 512, 8, 16, 1024, 384, 64, 4),
    ("short-runs", 40, 4, 16, 512, 200, 32, 8),
    ("decode", 4, 8, 64, 512, 128, 64, 4),
]


def test_noalloc_matches_workspace_entry_point(dev):
    import quantized_moe_grouped_amd as mq
    lib = mq.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    for name, T, A, E, K, N, gs, bits in CALLS:
        case = workloads.gather_case(name, T, A, E, K, N, seed=71, group_size=gs, bits=bits)
        _say(f"no-alloc {name} T={T} A={A} E={E} K={K} N={N} gs={gs} bits={bits}")
        x = bf16_to_torch(case.x, dev)
        idx = i32_to_torch(case.idx, dev)
        wq, s, b = mq.mq_quantize(bf16_to_torch(case.w, dev), gs, bits)
        ref_out = mq.mq_gather_qmm(x, wq, s, b, idx, True, gs, bits, False)
        out = torch.full((T, A, 1, N), float("nan"), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        st = lib.mq_gather_qmm_noalloc(x.data_ptr(), T, A, 1, K, wq.data_ptr(), s.data_ptr(),
                                       b.data_ptr(), E, N, idx.data_ptr(), A, 1, gs, bits, 0,
                                       out.data_ptr(), stream)
        assert st == mq.MQ_OK, mq.mq_status_str(st)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(dev) == before
        got = torch_bf16_to_u16(out)
        assert np.array_equal(got, torch_bf16_to_u16(ref_out)), name
        owq, os_, ob = oracle.quantize(case.w, gs, bits)
        check_gate(bf16_u16_to_f64(got), oracle.gather_qmm(case.x, owq, os_, ob, case.idx, gs, bits),
                   name)
