"""attn_backward_dense on the GPU against the oracle's gradients, element by element.

The GPU takes O and LSE from its own forward (attn_prefill_dense), as training
does; the oracle differentiates the exact definition from Q, K, V and dO alone.

Tolerance, from the arithmetic: every gradient is a sum of n products in which
one factor (P or dS) is rounded to bf16 before the MFMA and the other is exact
bf16 input, accumulated in fp32, then rounded once to bf16.  Rounding to bf16
(8 significant bits) moves a value by at most 2^-8 of itself, and n fp32
additions by at most n * 2^-24 of the sum of magnitudes, so
|gpu - exact| <= (2^-8 + n 2^-24) * A + 2^-8 * |exact|, A = the sum of the
absolute values of the terms, n = T * (q heads per kv head).  dS also
inherits the error of D_i = sum_c dO_ic O_ic taken from the forward's bf16
output O; the oracle returns a bound e on that effect (zero for dV).  The test
allows exactly that sum, plus 1e-6 absolute.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DEV

import paged_kv_cache_amd as pa

pytestmark = pytest.mark.gpu


def _gpu_grads(case):
    q, k, v, do = (x.to(DEV) for x in (case.q, case.k, case.v, case.dout))
    O, L = pa.attn_prefill_dense(q, k, v, case.scale, case.causal)
    dq, dk, dv = pa.attn_backward_dense(q, k, v, O, do, L, case.scale, case.causal)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy().astype(np.float64) for x in (dq, dk, dv)]


def _check(name, got, ref, absum, dterm, n_terms, sel=None):
    if sel is not None:
        got, ref, absum, dterm = got[sel], ref[sel], absum[sel], dterm[sel]
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    bound = (2.0 ** -8 + n_terms * 2.0 ** -24) * absum + 2.0 ** -8 * np.abs(ref) + dterm + 1e-6
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (f"{name}: |err| {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst} "
                                  f"(gpu {got[worst]}, ref {ref[worst]}, sum|terms| {absum[worst]:.3e})")


def _parity(case, pairs=None):
    dq, dk, dv = _gpu_grads(case)
    rq, rk, rv, aq, ak, av, eq, ek = oracle.attn_dense_backward(
        case.q, case.k, case.v, case.dout, case.scale, case.causal, with_abs=True, pairs=pairs)
    selq = selk = None
    if pairs is not None:
        B, T, Hq, _ = case.q.shape
        Hkv = case.k.shape[2]
        g = Hq // Hkv
        mq = np.zeros((B, T, Hq), bool)
        mk = np.zeros((B, T, Hkv), bool)
        for b, kvh in pairs:
            mq[b, :, kvh * g:(kvh + 1) * g] = True
            mk[b, :, kvh] = True
        selq, selk = mq, mk
    n = case.q.shape[1] * (case.q.shape[2] // case.k.shape[2])
    _check("dQ", dq, rq, aq, eq, n, selq)
    _check("dK", dk, rk, ak, ek, n, selk)
    _check("dV", dv, rv, av, np.zeros_like(av), n, selk)


@pytest.mark.parametrize("T", [1, 17, 64, 100, 129, 257])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_ragged_lengths(T, causal):
    _parity(W.make_dense("bwd", B=2, T=T, Hq=8, Hkv=2, d=64, causal=causal, seed=T, grad=True))


@pytest.mark.parametrize("Hq,Hkv,d", [(4, 4, 64), (8, 1, 64), (32, 4, 64), (4, 4, 128), (8, 2, 128),
                                      (16, 2, 128), (8, 8, 128), (32, 2, 64), (16, 1, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_head_shapes(Hq, Hkv, d, causal):
    _parity(W.make_dense("bwd", B=2, T=200, Hq=Hq, Hkv=Hkv, d=d, causal=causal, seed=Hq + d, grad=True))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_fa2_shape_t4096_one_head(d, causal):
    """The FA2 benchmark shape at T = 4096 (B = 4, hidden 2048) in the launch the sweep times;
    every gradient of sequence 1, head 3 against the oracle."""
    case = W.fa2_dense(4096, d, causal, grad=True)
    _parity(case, pairs=[(1, 3)])


def test_backward_deterministic():
    case = W.make_dense("det", B=2, T=300, Hq=8, Hkv=2, d=64, causal=True, seed=3, grad=True)
    a = _gpu_grads(case)
    b = _gpu_grads(case)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
