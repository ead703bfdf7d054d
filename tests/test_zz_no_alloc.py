"""w4a16_linear_static_ws: the linear with the library's own per-device scratch
array, for callers that cannot allocate.  Through the C ABI, its output must equal
w4a16_linear's (same kernels) bit for bit, and the oracle within the accuracy
bound, on consecutive calls that leave the array dirty for the next one (the
second smaller than the first); shapes that need more scratch than the array holds
are refused before anything is enqueued."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev_inputs

torch = pytest.importorskip("torch")
w4 = pytest.importorskip("int4_weight_only_02_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w4.lib()
    return torch.device("cuda:0")


def _case(seed, M, N, K, dev):
    d = synth.linear_inputs(seed, M, N, K)
    t = dev_inputs(d, dev)
    qw, qz = w4.w4a16_pack(t["codes"], t["zeros"])
    oqw, oqz = oracle.pack(d["codes"], d["zeros"])
    return d, t, qw, qz, oqw, oqz


def _allocations(dev):
    """Device allocations torch's allocator has made so far (a running count)."""
    return torch.cuda.memory_stats(dev).get("allocation.all.allocated", 0)


# each uses the scratch: K chunked across workgroups (partial sums and arrival
# counters), the same with fewer rows, columns and chunks, and the large-M path
# (X staged as fp16); then a call that needs none
CASES = [(16, 2560, 9728, torch.float32), (16, 264, 5760, torch.bfloat16), (130, 264, 1280, torch.float32),
         (1, 2560, 9728, torch.bfloat16)]


def test_static_ws_matches_linear_on_consecutive_calls(dev):
    for seed, (M, N, K, dt) in enumerate(CASES):
        print("static ws", M, N, K, dt, flush=True)
        d, t, qw, qz, oqw, oqz = _case(100 + seed, M, N, K, dev)
        ref = w4.w4a16_linear(t["X"], qw, t["scales"], qz, out_dtype=dt)
        Y = torch.empty((M, N), dtype=dt, device=dev)
        torch.cuda.synchronize()
        before = _allocations(dev)
        w4.w4a16_linear_static_ws(t["X"], qw, t["scales"], qz, out=Y)
        torch.cuda.synchronize()
        assert _allocations(dev) == before, "the call allocated device memory"
        assert torch.equal(Y, ref), "static-scratch call differs from w4a16_linear"
        check(Y, oracle.linear(d["X"], oqw, d["scales"], oqz), "static ws M=%d N=%d K=%d" % (M, N, K))
        # a second call into the dirty array gives the same bits
        Y2 = torch.empty_like(Y)
        w4.w4a16_linear_static_ws(t["X"], qw, t["scales"], qz, out=Y2)
        torch.cuda.synchronize()
        assert torch.equal(Y2, ref)


def test_static_ws_refuses_oversized_shapes(dev):
    M, N, K = 8192, 2560, 9728  # the large-M path needs 2 M K bytes of X alone
    assert w4.w4a16_workspace_bytes(w4.OP_LINEAR, M, N, K) > (8 << 20)
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    qw = torch.zeros((N, K // 8), dtype=torch.int32, device=dev)
    S = torch.zeros((N, K // 128), dtype=torch.float16, device=dev)
    qz = torch.zeros((N // 8, K // 128), dtype=torch.int32, device=dev)
    Y = torch.full((M, N), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_linear_static_ws(X, qw, S, qz, out=Y)
    assert e.value.status == 5  # W4A16_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all()), "a refused call must enqueue nothing"
