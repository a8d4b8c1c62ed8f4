"""dfssm_k_gemm_noalloc (the projection on the int8 matrix cores with its
operand scratch in a static per-GPU buffer) gives exactly what dfssm_k_gemm
gives, called through the C ABI twice in a row with the second input smaller
(the buffer keeps the first call's contents), on both the decode-sized and
the tiled kernel; sizes beyond the buffer are refused before any work."""
import numpy as np
import pytest

from tests._common import assert_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _operands(rng, M, d_in, d_out):
    r = 16
    bits = rng.integers(0, 2**32, size=(d_out, d_in // 32), dtype=np.uint64).astype(np.uint32)
    sw = rng.uniform(0.01, 0.05, d_out).astype(np.float32)
    A = rng.integers(-127, 128, size=(r, d_in)).astype(np.int8)
    sA = rng.uniform(5e-4, 2e-3, r).astype(np.float32)
    Bm = rng.integers(-127, 128, size=(d_out, r)).astype(np.int8)
    sB = rng.uniform(5e-4, 2e-3, d_out).astype(np.float32)
    q = rng.integers(-127, 128, size=(M, d_in)).astype(np.int8)
    s = rng.uniform(0.01, 0.05, M).astype(np.float32)
    return [_dev(x) for x in (bits, sw, A, sA, Bm, sB, q, s)]


@pytest.mark.parametrize("sizes", [((200, 2048, 8512), (40, 2048, 1000)),   # tiled, then tiled smaller
                                   ((32, 4096, 2048), (3, 4096, 2048)),     # decode-sized twice
                                   ((100, 8192, 300), (17, 512, 96))])      # tiled, then decode-sized
def test_noalloc_gemm_equals_gemm_twice(sizes):
    from bit_quantized_mamba_amd import k_gemm, k_gemm_noalloc
    rng = np.random.default_rng(sum(sum(x) for x in sizes))
    for M, d_in, d_out in sizes:
        ops = _operands(rng, M, d_in, d_out)
        acc_ref, y_ref = k_gemm(*ops)
        acc, y = k_gemm_noalloc(*ops)
        torch.cuda.synchronize()
        assert torch.equal(acc, acc_ref), (M, d_in, d_out)
        assert torch.equal(y, y_ref), (M, d_in, d_out)
        # the integer sums against numpy on a few rows
        bits = ops[0].cpu().numpy()
        q = ops[6].cpu().numpy()
        W = np.where(np.unpackbits(bits.view(np.uint8), bitorder="little").reshape(d_out, d_in), 1, -1)
        rows = sorted({0, M // 2, M - 1})
        want = q[rows].astype(np.int64) @ W.T.astype(np.int64)
        assert np.array_equal(acc.cpu().numpy()[rows], want)
        assert_close(y.cpu().numpy(), y_ref.cpu().numpy(), what="y")


def test_noalloc_gemm_rejects_sizes_beyond_its_buffer():
    from bit_quantized_mamba_amd import DfssmError, k_gemm_noalloc
    rng = np.random.default_rng(3)
    # 1100 x 8192 bytes of bit planes alone exceed the 8 MiB buffer
    ops = _operands(rng, 1100, 8192, 64)
    with pytest.raises(DfssmError, match="scratch"):
        k_gemm_noalloc(*ops)
