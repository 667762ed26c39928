"""Runtime behaviour on the GPU: one HIP runtime, streams, determinism, the tensor wrapper."""

import numpy as np
import pytest

from gpu_util import run, say, to_device
from workloads.inputs import BF16, F16, make_operands

pytestmark = pytest.mark.gpu


def test_single_hip_runtime_mapped():
    import torch

    import tiled_shared_memory_amd as tsm

    tsm.load()
    torch.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read()
    paths = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(paths) == 1, paths
    assert any("libtsm_gemm.so" in ln for ln in maps.splitlines())


def test_repeated_runs_bitwise_identical():
    M, N, K = 1000, 1500, 777
    A, B = make_operands(3, 1, M, N, K, F16, ("uniform", -1.0, 1.0))
    say("[gpu] determinism x20")
    first = run(A, B, M, N, K, F16, "f32")
    for _ in range(19):
        assert np.array_equal(run(A, B, M, N, K, F16, "f32"), first)


def test_chain_on_side_stream_matches_synchronised_chain():
    """Two dependent GEMMs and the copy back, all enqueued on a non-default stream
    without any synchronisation in between, give the same bits as the same chain
    run with a device synchronisation after every step."""
    import torch

    import tiled_shared_memory_amd as tsm

    M, N, K = 256, 384, 512
    A, B = make_operands(41, 1, M, K, K, F16, ("uniform", -1.0, 1.0))   # B is K x K
    _, B2 = make_operands(42, 1, M, N, K, F16, ("uniform", -1.0, 1.0))   # B2 is K x N
    a_buf, a = to_device(A)
    b_buf, b = to_device(B)
    b2_buf, b2 = to_device(B2)
    torch.cuda.synchronize()  # uploads were enqueued on the default stream

    def chain(stream, sync):
        c1 = torch.empty(M * K, dtype=torch.float16, device="cuda")
        c2 = torch.empty(M * N, dtype=torch.float32, device="cuda")
        h = stream.cuda_stream if stream is not None else 0
        tsm.gemm(M, K, K, a, K, b, K, c1, K, tsm.TSM_F16_F16, h)
        if sync:
            torch.cuda.synchronize()
        tsm.gemm(M, N, K, c1, K, b2, N, c2, N, tsm.TSM_F16_F32, h)
        if sync:
            torch.cuda.synchronize()
        out = torch.empty(M * N, dtype=torch.float32, pin_memory=True)
        if stream is not None:
            with torch.cuda.stream(stream):
                out.copy_(c2, non_blocking=True)
            stream.synchronize()
        else:
            out.copy_(c2)
        return out.numpy().copy()

    say("[gpu] side-stream chain")
    ref = chain(None, True)
    s = torch.cuda.Stream()
    for _ in range(3):
        assert np.array_equal(chain(s, False), ref)


def test_matmul_wrapper_reads_layouts_from_views(orc):
    import torch

    import tiled_shared_memory_amd as tsm

    M, N, K = 96, 80, 112
    A, B = make_operands(8, 1, M, N, K, BF16, ("uniform", -1.0, 1.0))
    a = torch.from_numpy(A[0].view(np.int16)).cuda().view(torch.bfloat16)
    bt = torch.from_numpy(np.ascontiguousarray(B[0].T).view(np.int16)).cuda().view(torch.bfloat16)
    say("[gpu] matmul wrapper with a transposed view")
    c = tsm.matmul(a, bt.t(), out_dtype=torch.float32)   # column-major B
    torch.cuda.synchronize()
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16)
    from gpu_util import check

    check(c.cpu().numpy().astype(np.float64)[None], Cr, S, K, "f32", "matmul wrapper")


def test_matmul_wrapper_activation_and_workspace(orc):
    """The torch-level wrapper with a fused leaky ReLU, bf16 output and a workspace that splits K."""
    import torch

    import oracle
    import tiled_shared_memory_amd as tsm

    M, N, K = 256, 256, 2048
    A, B = make_operands(9, 1, M, N, K, F16, ("uniform", -1.0, 1.0))
    a = torch.from_numpy(A[0].view(np.int16)).cuda().view(torch.float16)
    b = torch.from_numpy(B[0].view(np.int16)).cuda().view(torch.float16)
    ws = tsm.workspace_for(a, b)
    assert ws is not None
    say("[gpu] matmul wrapper with activation and workspace")
    c = tsm.matmul(a, b, out_dtype=torch.bfloat16, activation="leaky_relu", slope=0.25, workspace=ws)
    torch.cuda.synchronize()
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16)
    from gpu_util import check

    check(c.float().cpu().numpy().astype(np.float64)[None], Cr, S, K, "bf16", "matmul ws",
          act=oracle.ACT_LEAKY_RELU, slope=0.25)
    with pytest.raises(tsm.TsmError):
        tsm.matmul(a, b, activation="gelu")


def test_launch_error_is_not_raised_for_valid_calls():
    # a valid call after many invalid ones still launches (no sticky error state)
    import tiled_shared_memory_amd as tsm

    for _ in range(3):
        with pytest.raises(tsm.TsmError):
            tsm.gemm(-1, 1, 1, 0, 1, 0, 1, 0, 1, 0, 0)
    A, B = make_operands(1, 1, 8, 8, 8, F16, ("uniform", -1.0, 1.0))
    C = run(A, B, 8, 8, 8, F16, "f32")
    assert np.all(np.isfinite(C))
