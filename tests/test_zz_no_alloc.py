"""awq_act_stats_noalloc (scratch in the library's static device array, no allocation) against
awq_act_stats (caller workspace) through the C ABI: two calls in a row, the second with a
smaller input, each bit-identical to the workspace call (s_X and flags), plus a bf16 and an fp32
input (exponent records in the scratch) and a row-strided view."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

F16, BF16, F32 = 1, 2, 0


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    from post_weight_quantization_channel_amd import _lib
    return _lib.load()


def _both(lib, X, xdt):
    """The same statistics through both calls on the current stream."""
    M, K = X.shape
    ldx = X.stride(0) if M > 1 else K
    stream = torch.cuda.current_stream().cuda_stream
    sx_a = torch.full((K,), -1.0, dtype=torch.float32, device="cuda")
    fl_a = torch.zeros(1, dtype=torch.int32, device="cuda")
    nbytes = lib.awq_act_stats_workspace_bytes(M, K)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert lib.awq_act_stats(X.data_ptr(), xdt, M, K, ldx, sx_a.data_ptr(), fl_a.data_ptr(),
                             ws.data_ptr(), nbytes, stream) == 0
    sx_b = torch.full((K,), -2.0, dtype=torch.float32, device="cuda")
    fl_b = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert lib.awq_act_stats_noalloc(X.data_ptr(), xdt, M, K, ldx, sx_b.data_ptr(),
                                     fl_b.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    return sx_a.cpu().numpy(), fl_a.item(), sx_b.cpu().numpy(), fl_b.item()


def test_noalloc_stats_two_calls_then_smaller(lib):
    cases = [
        ("f16 65536x4096", workloads.c2_like_layer(n=8, k=4096, m=65536, config=71).X, F16),
        ("f16 300x512 (smaller, after)", workloads.c2_like_layer(n=8, k=512, m=300,
                                                                  config=72).X, F16),
        ("bf16 4133x1024", workloads.c2_like_layer(n=8, k=1024, m=4133, config=73).X, BF16),
        ("f32 257x264", workloads.c2_like_layer(n=8, k=264, m=257, config=74).X, F32),
    ]
    for name, X, xdt in cases:
        print("   act_stats_noalloc", name, flush=True)
        t = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        t = t.to({F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}[xdt])
        sa, fa, sb, fb = _both(lib, t, xdt)
        assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32)), name
        assert fa == fb, name


def test_noalloc_stats_strided_view(lib):
    X = workloads.c2_like_layer(n=8, k=512, m=600, config=75).X
    t = torch.from_numpy(X).cuda()[:, :384]
    print("   act_stats_noalloc strided view", tuple(t.shape), flush=True)
    sa, fa, sb, fb = _both(lib, t, F16)
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32)) and fa == fb
