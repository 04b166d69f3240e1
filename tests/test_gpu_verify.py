"""The multi-row verify GEMV: each of its rows must be memcmp-equal to the M=1
kernel's output for that activation row, and within tolerance of the oracle."""
import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import THREADS, announce, assert_linear, empty_f32, sync, to_dev

pytestmark = pytest.mark.gpu

# the verify configuration's two weights, plus ragged / split-K / large-K shapes,
# and two more shapes of the persistent form (the first weight is one too)
CASES = [("q4_0", 17408, 5120), ("q8_0", 4096, 1024), ("q8_0", 33, 2080), ("q4_0", 9, 1056),
         ("q4_0", 640, 17408), ("q8_0", 100, 3072), ("q4_0", 24, 32768), ("q4_0", 3300, 5120),
         ("q8_0", 2001, 8288),
         # the super-block types: one tile per wavefront group, K split four ways
         # (200x4096), the persistent form (2001x8448 with an 8-block last segment)
         ("q4_k", 1000, 1024), ("q4_k", 200, 4096), ("q4_k", 2001, 8448),
         ("q6_k", 1000, 1024), ("q6_k", 200, 4096), ("q6_k", 3300, 5120),
         # three segments: K split three ways (one segment per wavefront)
         ("q4_k", 1024, 3072), ("q6_k", 77, 3072), ("q8_0", 1024, 3072),
         # M K 4 bytes above the LDS from M = 3: the persistent form walks its 17 K
         # ranges in phases, staging one window of activations at a time; 17504
         # has 18 ranges, the last segment 3 blocks long (zero-filled in its window)
         ("q4_0", 5120, 17408), ("q6_k", 2001, 17408), ("q4_0", 3000, 17504),
         # super-block types on 80 row tiles of 17 segments: K split eight ways at
         # every M, activations from L2 at M = 5, 6 (kernels that spill to scratch)
         ("q4_k", 640, 17408), ("q6_k", 640, 17408),
         # eight split-K wavefronts over 8 segments: four staged rows take 128 KiB of
         # LDS; five rows (exactly 160 KiB) plus the partials do not fit, so M = 5, 6
         # read their activations from L2 (Q4_K: the four rows' block sums after
         # them, 132 KiB in all)
         ("q4_0", 1280, 8192), ("q8_0", 1280, 8192), ("q4_k", 1280, 8192),
         # Q4_K's block sums per phase window of the persistent form (M >= 3)
         ("q4_k", 2001, 17408),
         # the persistent form with one K range, whose half-tiles store their sums
         # directly: 37 segments (a prime count, activations from L2 from M = 2)
         # with a ragged row tile, and one segment (single-unit items)
         ("q4_0", 1001, 37888), ("q8_0", 20000, 1024)]


@pytest.mark.parametrize("kind,N,K", CASES)
def test_verify_rows_bit_identical_to_m1(kind, N, K):
    rng = np.random.default_rng(N + K)
    canon = W.matrix(kind, N, K, rng)
    packed = qg.pack_weights(kind, canon, N, K)
    X = W.activation(K, rng, M=6)
    Xd = to_dev(X)
    # M = 1 reference outputs of every row
    ones = []
    for m in range(6):
        y = empty_f32(N)
        announce(f"verify baseline qgemv_{kind} N={N} K={K} row={m}")
        qg.qgemv(kind, packed, Xd[m].contiguous(), y, N, K)
        ones.append(y)
    sync()
    ones = [y.cpu().numpy() for y in ones]
    for M in range(2, 7):
        Y = empty_f32(M * N + 11, fill=3.0)
        announce(f"qgemv_verify {kind} N={N} K={K} M={M} plan={qg.qg_plan_info(kind, N, K, M)}")
        qg.qgemv_verify(kind, packed, Xd[:M].contiguous(), Y, N, K, M)
        sync()
        Yh = Y.cpu().numpy()
        assert np.all(Yh[M * N:] == 3.0), "wrote past Y[M-1][N-1]"
        for m in range(M):
            assert Yh[m * N:(m + 1) * N].tobytes() == ones[m].tobytes(), f"M={M} row {m} differs from M=1"
    Y_ref, A_ref = O.verify(kind, canon, X, N, K, threads=THREADS)
    for m in range(6):
        assert_linear(ones[m], Y_ref[m], A_ref[m], f"verify {kind} {N}x{K} row {m}")


def test_verify_rows_are_independent():
    # the same activation in every row gives identical rows; rows differ when inputs do
    kind, N, K = "q4_0", 300, 5120
    rng = np.random.default_rng(17)
    canon = W.matrix(kind, N, K, rng)
    packed = qg.pack_weights(kind, canon, N, K)
    x = W.activation(K, rng)
    X = np.stack([x] * 4)
    X[2] = -X[2]
    Y = empty_f32(4 * N)
    announce("verify independence")
    qg.qgemv_verify(kind, packed, to_dev(X), Y, N, K, 4)
    sync()
    Y = Y.cpu().numpy().reshape(4, N)
    assert Y[0].tobytes() == Y[1].tobytes() == Y[3].tobytes()
    assert np.array_equal(Y[2], -Y[0])
