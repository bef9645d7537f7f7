"""The workloads' data tell the declared orders from plausible other ones (CPU only).

A parity test can only catch a wrong order if the data make orders
disagree.  On the reduce workload (OPEN-1B Appendix A.1: TreeFold) and on
rows of the weight-gradient workload (section 2.1: one ascending chain,
unfused), the oracle's result differs in many words from a sequential fold,
from a descending chain and from a fused chain.
"""
import numpy as np

import oracle
import synth


def _differing(a, b):
    return int(np.count_nonzero(np.asarray(a, np.float32).view(np.uint32) != np.asarray(b, np.float32).view(np.uint32)))


def test_reduce_workload_tree_versus_sequential():
    n = 1 << 20  # a slice of the 16,777,216-element replicas
    reps = [synth.reduce_replica(r, n) for r in range(synth.REDUCE["R"])]
    tree = oracle.tree_reduce(reps, average=False)
    seq = reps[0].copy()
    for r in reps[1:]:
        seq = (seq + r).astype(np.float32)  # ((x0 + x1) + x2) + ...
    assert _differing(tree, seq) > 1000


def test_dw_workload_rows_ascending_unfused_versus_other_orders():
    K, M, N = synth.DW["K"], synth.DW["M"], synth.DW["N"]
    x = synth.dw_x().reshape(K, M)
    dy = synth.dw_dy().reshape(K, N)
    rows = [0, 1029]
    A = np.ascontiguousarray(x[:, rows].T)          # op(A) rows of X^T
    Bt = np.ascontiguousarray(dy[:, :256].T)        # 256 output columns
    ref = oracle.gemm(A, Bt, trans_b=True)
    desc = oracle.gemm(np.ascontiguousarray(A[:, ::-1]), np.ascontiguousarray(Bt[:, ::-1]), trans_b=True)
    fused = oracle.gemm(A, Bt, trans_b=True, fused=True)
    assert _differing(ref, desc) > 100
    assert _differing(ref, fused) > 100
