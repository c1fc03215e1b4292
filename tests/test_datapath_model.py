"""CPU pin of the FP8 datapath model the GPU GEMM checks use
(gpu_util.run_truncation): on hand-built 8-K runs its outputs must equal the
hand-derived literals of datapath_cases, which the GPU GEMMs must also
reproduce (tests/test_gpu_datapath.py).  The oracle's exact fp64 sums are
checked on the same operands, so the cases show where the datapath and the
exact definition part."""
import numpy as np

import oracle
from datapath_cases import EXACT_SAMPLES, EXPECTED, expected_full, operands
from gpu_util import run_truncation


def _model(qa, qb):
    M, N = qa.shape[0], qb.shape[0]
    mi, ni = (g.reshape(-1) for g in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    ones = lambda mi_, ni_: np.ones((mi_.size, qa.shape[1] // 32))
    y, _ = run_truncation(qa, qb, ones, mi, ni)
    return y.reshape(M, N)


def test_model_matches_hand_derived_outputs():
    qa, qb = operands()
    assert np.array_equal(_model(qa, qb), expected_full())


def test_oracle_is_the_exact_sum():
    qa, qb = operands()
    sa = np.ones((qa.shape[0], 1), np.float32)
    sb = np.ones((1, 1), np.float32)
    yref, _ = oracle.gemm_blockscaled(qa, sa, qb, sb, with_abs=False)
    exact = oracle.e4m3_decode(qa) @ oracle.e4m3_decode(qb).T
    assert np.array_equal(yref, exact)
    for (m, n), v in EXACT_SAMPLES.items():
        assert yref[m, n] == v
        assert EXPECTED[m][n] != v


def test_model_rule_is_sensitive_to_each_parameter():
    """Variants of the rule (runs of 4 or 16, a unit of 2^(E-12) or
    2^(E-14), rounding to nearest, floor, normalized subnormal exponents,
    zero codes counted with exponent -6) each miss at least one literal."""
    qa, qb = operands()
    dec = oracle.e4m3_decode(np.arange(256)).copy()
    dec[np.isnan(dec)] = 0.0
    field = (np.arange(256) >> 3) & 15
    mant = np.arange(256) & 7

    def variant(run=8, shift=13, mode="trunc", subnormal_true=False, zeros_count=False):
        e = (np.maximum(field, 1) - 7).astype(np.float64)
        if subnormal_true:
            with np.errstate(divide="ignore"):
                e = np.where((field == 0) & (mant > 0), np.floor(np.log2(np.maximum(mant, 1))) - 9, e)
        p = dec[qa][:, None, :] * dec[qb][None, :, :]
        ee = e[qa][:, None, :] + e[qb][None, :, :]
        if not zeros_count:
            ee = np.where(p == 0, -1e9, ee)
        M, N, K = p.shape
        p = p.reshape(M, N, K // run, run)
        E = np.maximum(ee.reshape(M, N, K // run, run).max(axis=3), -200.0)   # all-zero runs
        u = np.exp2(E - shift)[..., None]
        f = {"trunc": np.trunc, "nearest": np.round, "floor": np.floor}[mode]
        return (f(p / u) * u).sum(axis=(2, 3))

    ref = expected_full()
    assert np.array_equal(variant(), ref)
    for kw in (dict(run=4), dict(run=16), dict(shift=12), dict(shift=14), dict(mode="nearest"),
               dict(mode="floor"), dict(subnormal_true=True), dict(zeros_count=True)):
        assert not np.array_equal(variant(**kw), ref), kw
