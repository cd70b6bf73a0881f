"""Pins of the oracle's attention backward (gradients of sum(O * dO)).

Routes independent of the oracle's code: torch autograd in float64 through an
explicit softmax attention (the library's own derivative), the single-key
closed form, the q = 0 closed form of dV, and the softmax shift invariance
(the key gradients of a row sum to zero).
"""

import numpy as np
import pytest
import torch

import workloads as W


def _autograd(case):
    q = case.q.double().requires_grad_()
    k = case.k.double().requires_grad_()
    v = case.v.double().requires_grad_()
    B, T, Hq, d = q.shape
    g = Hq // k.shape[2]
    kk = k.repeat_interleave(g, dim=2)             # q head h uses kv head h // g
    vv = v.repeat_interleave(g, dim=2)
    s = torch.einsum("bihc,bjhc->bhij", q, kk) * case.scale
    if case.causal:
        mask = torch.ones(T, T, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhc->bihc", p, vv)
    (o * case.dout.double()).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("Hq,Hkv,d,causal", [(4, 4, 64, True), (4, 1, 64, False), (8, 2, 128, True),
                                             (2, 2, 128, False)])
def test_backward_matches_autograd(oracle_lib, Hq, Hkv, d, causal):
    case = W.make_dense("g", B=2, T=37, Hq=Hq, Hkv=Hkv, d=d, causal=causal, seed=Hq + d, grad=True)
    dQ, dK, dV = oracle_lib.attn_dense_backward(case.q, case.k, case.v, case.dout, case.scale, causal)
    gq, gk, gv = _autograd(case)
    for name, a, b in (("dQ", dQ, gq), ("dK", dK, gk), ("dV", dV, gv)):
        assert np.allclose(a, b, rtol=0, atol=1e-10), f"{name}: max diff {np.abs(a - b).max()}"


def test_backward_single_key(oracle_lib):
    """T = 1: P = 1, so dS = 0 (dQ = dK = 0) and dV = dO summed over the group's heads."""
    case = W.make_dense("one", B=3, T=1, Hq=4, Hkv=2, d=64, causal=True, seed=2, grad=True)
    dQ, dK, dV = oracle_lib.attn_dense_backward(case.q, case.k, case.v, case.dout, case.scale, True)
    assert np.all(dQ == 0) and np.all(dK == 0)
    do = case.dout.double().numpy()
    assert np.allclose(dV, do.reshape(3, 1, 2, 2, 64).sum(3), rtol=0, atol=1e-12)


def test_backward_zero_query_dv_closed_form(oracle_lib):
    """q = 0, causal: row i weighs its i+1 keys equally, so dV_j = sum_{i >= j} dO_i / (i + 1)."""
    case = W.make_dense("z", B=1, T=20, Hq=1, Hkv=1, d=64, causal=True, seed=4, grad=True)
    case.q = torch.zeros_like(case.q)
    _, _, dV = oracle_lib.attn_dense_backward(case.q, case.k, case.v, case.dout, case.scale, True)
    do = case.dout.double().numpy()[0, :, 0]
    want = np.stack([sum(do[i] / (i + 1) for i in range(j, 20)) for j in range(20)])
    assert np.allclose(dV[0, :, 0], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_key_gradients_sum_to_zero(oracle_lib, causal):
    """Adding one vector to every key of a row moves all its scores equally, which softmax
    ignores: per (sequence, kv head), the dK rows sum to zero."""
    case = W.make_dense("s", B=2, T=30, Hq=4, Hkv=2, d=64, causal=causal, seed=9, grad=True)
    _, dK, _ = oracle_lib.attn_dense_backward(case.q, case.k, case.v, case.dout, case.scale, causal)
    assert np.abs(dK.sum(axis=1)).max() < 1e-10
    assert np.abs(dK).max() > 1e-2


def test_backward_abs_sums_bound_values(oracle_lib):
    case = W.make_dense("a", B=1, T=25, Hq=4, Hkv=1, d=64, causal=True, seed=5, grad=True)
    dQ, dK, dV, aQ, aK, aV, eQ, eK = oracle_lib.attn_dense_backward(
        case.q, case.k, case.v, case.dout, case.scale, True, with_abs=True)
    for x, a in ((dQ, aQ), (dK, aK), (dV, aV)):
        assert np.all(np.abs(x) <= a + 1e-12)
    assert np.all(eQ >= 0) and np.all(eK >= 0) and eQ.max() > 0


def test_backward_d_bound_covers_rounded_output(oracle_lib):
    """eQ, eK bound the change of dQ, dK when D is taken from O rounded to bf16: checked
    against a direct numpy evaluation with exactly that D."""
    case = W.make_dense("e", B=1, T=17, Hq=2, Hkv=1, d=64, causal=True, seed=17, grad=True)
    dQ, dK, _, _, _, _, eQ, eK = oracle_lib.attn_dense_backward(
        case.q, case.k, case.v, case.dout, case.scale, True, with_abs=True)
    q, k, v, do = (x.double().numpy()[0] for x in (case.q, case.k, case.v, case.dout))
    sc = case.scale
    gq = np.zeros_like(q)
    gk = np.zeros_like(k)
    for h in range(2):
        for i in range(17):
            s = sc * (k[:i + 1, 0] @ q[i, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            dp = v[:i + 1, 0] @ do[i, h]
            o = torch.tensor(p @ v[:i + 1, 0], dtype=torch.float32).to(torch.bfloat16).double().numpy()
            ds = p * (dp - (do[i, h] * o).sum())
            gq[i, h] = sc * ds @ k[:i + 1, 0]
            gk[:i + 1, 0] += sc * np.outer(ds, q[i, h])
    assert np.all(np.abs(gq - dQ[0]) <= eQ[0] + 1e-12)
    assert np.all(np.abs(gk - dK[0]) <= eK[0] + 1e-12)
    assert np.abs(gq - dQ[0]).max() > 1e-4          # the effect is real at this size
