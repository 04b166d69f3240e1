"""The no-allocation prefill GEMM (qgemm_prefill_noalloc): called through the C
ABI, it must return bit for bit what qgemm_prefill returns with a caller-owned
workspace (same kernels on the library's per-GPU scratch array), within the
linear tolerance of the fp64 oracle, on two calls in a row, the second with a
smaller input; it writes nothing past Y."""
import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import THREADS, announce, assert_linear, empty_f32, sync, to_dev

pytestmark = pytest.mark.gpu

# The first call splits K across workgroups (K ranges of partial sums in the
# scratch) over 40 activation rows; the second is smaller: 5 rows of a
# 1000-row weight.
CASES = [("q4_0", 5120, 17408, 40, 81), ("q8_0", 1000, 1024, 5, 82)]


def test_prefill_noalloc_matches_workspace_call_twice():
    for kind, N, K, M, seed in CASES:
        rng = np.random.default_rng(seed)
        canon = W.matrix(kind, N, K, rng)
        packed = qg.pack_weights(kind, canon, N, K)
        X = W.activation(K, rng, M=M)
        Xd = to_dev(X)
        need = qg.qg_prefill_workspace_size(kind, N, K, M)
        assert 0 < need <= qg.QG_PREFILL_NOALLOC_MAX_BYTES
        y_ws = empty_f32(M * N + 7, fill=-3.0)
        y_na = empty_f32(M * N + 7, fill=-3.0)
        announce(f"qgemm_prefill {kind} {N}x{K} M={M} (workspace {need} bytes)")
        qg.qgemm_prefill(kind, packed, Xd, y_ws[:M * N], N, K, M)
        announce(f"qgemm_prefill_noalloc {kind} {N}x{K} M={M}")
        qg.qgemm_prefill_noalloc(kind, packed, Xd, y_na[:M * N], N, K, M)
        sync()
        a_ws, a_na = y_ws.cpu().numpy(), y_na.cpu().numpy()
        assert np.all(a_na[M * N:] == -3.0), "wrote past Y"
        assert np.array_equal(a_na[:M * N].view(np.uint32), a_ws[:M * N].view(np.uint32)), \
            f"{kind} {N}x{K} M={M}: differs from qgemm_prefill"
        Y = a_na[:M * N].reshape(M, N)
        for m in range(M):
            y_ref, a_ref = O.gemv(kind, canon, np.ascontiguousarray(X[m]), N, K, threads=THREADS)
            assert_linear(Y[m], y_ref, a_ref, f"qgemm_prefill_noalloc {kind} {N}x{K} row {m}")
