"""Pins for the multi-layer distillation loss ("NLP——IndexCache" notes,
section "方法二：Training-Aware IndexCache": L_multi and Proposition 1).

Pinned to: torch autograd of the per-teacher KL sum (library KL and
log-softmax, fp64) for the gradient; Proposition 1 (the same gradient from one
KL against the mean teacher); scipy's rel_entr for the loss value; the closed
forms loss = 0 and gradient = 0 when every teacher equals softmax(I); and
causality (entries past t are never read).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import rel_entr

import oracle


def _inputs(rng, n, B, Lq, Lk, q_pos0):
    logits = rng.normal(size=(B, Lq, Lk)) * 2.0
    tl = rng.normal(size=(n, B, Lq, Lk)) * 1.5
    P = np.zeros((n, B, Lq, Lk))
    for i in range(Lq):
        t = q_pos0 + i
        e = np.exp(tl[..., i, : t + 1] - tl[..., i, : t + 1].max(axis=-1, keepdims=True))
        P[..., i, : t + 1] = e / e.sum(axis=-1, keepdims=True)
    P[0, 0, 0, 0] = 0.0                      # a zero teacher entry (0 log 0 = 0)
    P[0, 0, 0] /= P[0, 0, 0].sum()
    return logits, P


def test_gradient_is_autograd_of_the_teacher_sum_and_of_the_mean_teacher():
    rng = np.random.default_rng(4)
    n, B, Lq, Lk, q0 = 3, 2, 5, 9, 4
    logits, P = _inputs(rng, n, B, Lq, Lk, q0)
    loss, grad = oracle.distill_loss(logits, P, q0)
    for b in range(B):
        for i in range(Lq):
            t = q0 + i
            xa = torch.tensor(logits[b, i, : t + 1], dtype=torch.float64, requires_grad=True)
            xb = torch.tensor(logits[b, i, : t + 1], dtype=torch.float64, requires_grad=True)
            tp = torch.tensor(P[:, b, i, : t + 1], dtype=torch.float64)
            many = sum(F.kl_div(F.log_softmax(xa, -1), tp[j], reduction="sum")
                       for j in range(n)) / n
            many.backward()
            mean = F.kl_div(F.log_softmax(xb, -1), tp.mean(0), reduction="sum")
            mean.backward()
            assert np.allclose(grad[b, i, : t + 1], xa.grad.numpy(), atol=1e-12)
            assert np.allclose(xa.grad.numpy(), xb.grad.numpy(), atol=1e-12)   # Prop. 1
            assert loss[b, i] == pytest.approx(many.item(), rel=1e-12)
            assert np.all(grad[b, i, t + 1:] == 0.0)
            # the loss as library relative entropies
            q = torch.softmax(xa.detach(), -1).numpy()
            assert loss[b, i] == pytest.approx(
                np.mean([rel_entr(P[j, b, i, : t + 1], q).sum() for j in range(n)]), rel=1e-12)


def test_teachers_equal_to_the_student_give_zero():
    rng = np.random.default_rng(5)
    B, Lq, Lk = 1, 6, 6
    logits = rng.normal(size=(B, Lq, Lk))
    P = np.zeros((2, B, Lq, Lk))
    for i in range(Lq):
        e = np.exp(logits[0, i, : i + 1] - logits[0, i, : i + 1].max())
        P[:, 0, i, : i + 1] = e / e.sum()
    loss, grad = oracle.distill_loss(logits, P, 0)
    assert np.abs(loss).max() < 1e-12 and np.abs(grad).max() < 1e-12


def test_entries_past_t_are_not_read():
    rng = np.random.default_rng(6)
    logits, P = _inputs(rng, 2, 1, 4, 8, 2)
    l1, g1 = oracle.distill_loss(logits, P, 2)
    logits2, P2 = logits.copy(), P.copy()
    for i in range(4):
        logits2[0, i, 2 + i + 1:] = 1e9
        P2[:, 0, i, 2 + i + 1:] = 0.7
    l2, g2 = oracle.distill_loss(logits2, P2, 2)
    assert np.array_equal(l1, l2) and np.array_equal(g1, g2)
