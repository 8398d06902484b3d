"""Pins of the oracle's backward: central finite differences of the oracle's own forward
(a different computation from the hand-derived chain rule) and an independent autograd
evaluation in plain PyTorch fp64 on the CPU.

The pages state no backward; training with the layer is asserted (the news page's
contribution list, the blog's "How to Read the Reported Experiments").  The forward
being differentiated is Eq. (1)-(4) of the Griffin model-architecture page with the
conv of its "Recurrent block" section, rounding points off (fp64 mode).
"""
import numpy as np
import pytest
import torch

import oracle

NAMES = ["x", "conv_w", "conv_b", "W_a", "W_x", "b_a", "b_x", "lam", "h0"]


def _problem(seed, B, T, D, c=8.0, state=True):
    rng = np.random.default_rng(seed)
    p = {
        "x": rng.standard_normal((B, T, D)),
        "conv_w": rng.standard_normal((4, D)) * 0.5,
        "conv_b": rng.standard_normal(D) * 0.1,
        "W_a": rng.standard_normal((D, D)) / np.sqrt(D),
        "W_x": rng.standard_normal((D, D)) / np.sqrt(D),
        "b_a": rng.standard_normal(D) * 0.3,
        "b_x": rng.standard_normal(D) * 0.3,
        "lam": rng.uniform(2.0, 6.0, D),
        "h0": rng.standard_normal((B, D)),
    }
    st = rng.standard_normal((B, 3, D)) if state else None
    dy = rng.standard_normal((B, T, D))
    dhT = rng.standard_normal((B, D))
    return p, st, dy, dhT, c


def _loss(p, st, dy, dhT, c):
    o = oracle.forward(p["x"], p["conv_w"], p["conv_b"], st, p["W_a"], p["W_x"], p["b_a"],
                       p["b_x"], p["lam"], p["h0"], c, "f64")
    return float((dy * o["y"]).sum() + (dhT * o["h_T"]).sum())


def _grads(p, st, dy, dhT, c):
    g = oracle.backward(p["x"], p["conv_w"], p["conv_b"], st, p["W_a"], p["W_x"], p["b_a"],
                        p["b_x"], p["lam"], p["h0"], c, "f64", dy, dhT)
    return {"x": g["dx"], "conv_w": g["dconv_w"], "conv_b": g["dconv_b"], "W_a": g["dW_a"],
            "W_x": g["dW_x"], "b_a": g["db_a"], "b_x": g["db_x"], "lam": g["dlambda"],
            "h0": g["dh0"]}


@pytest.mark.parametrize("c,state", [(8.0, True), (8.0, False), (0.0, True), (2.5, True)])
def test_backward_matches_central_differences(c, state):
    p, st, dy, dhT, c = _problem(20, 1, 16, 8, c, state)
    g = _grads(p, st, dy, dhT, c)
    eps = 1e-6
    for name in NAMES:
        v = p[name]
        fd = np.empty_like(v)
        for idx in np.ndindex(v.shape):
            old = v[idx]
            v[idx] = old + eps
            lp = _loss(p, st, dy, dhT, c)
            v[idx] = old - eps
            lm = _loss(p, st, dy, dhT, c)
            v[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(g[name] - fd) / np.maximum(1.0, np.abs(fd)))
        assert err < 1e-6, (name, err)
        assert np.all(np.isfinite(g[name]))


def _torch_forward(t, st, c):
    """Eq. (1)-(4) with the conv, written with plain torch ops for autograd."""
    x = t["x"]
    B, T, D = x.shape
    X = torch.cat([torch.as_tensor(st), x], dim=1)
    u = t["conv_b"] + sum(t["conv_w"][k] * X[:, 3 - k:3 - k + T] for k in range(4))
    r = torch.sigmoid(u @ t["W_a"].T + t["b_a"])
    i = torch.sigmoid(u @ t["W_x"].T + t["b_x"])
    a = torch.sigmoid(t["lam"]) ** (c * r)
    m = torch.sqrt(1 - a * a)
    h = t["h0"]
    ys = []
    for s in range(T):
        h = a[:, s] * h + m[:, s] * i[:, s] * u[:, s]
        ys.append(h)
    return torch.stack(ys, 1), h


def test_backward_matches_torch_autograd():
    p, st, dy, dhT, c = _problem(21, 2, 40, 16)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    y, hT = _torch_forward(t, st, c)
    loss = (torch.as_tensor(dy) * y).sum() + (torch.as_tensor(dhT) * hT).sum()
    loss.backward()
    g = _grads(p, st, dy, dhT, c)
    for name in NAMES:
        np.testing.assert_allclose(g[name], t[name].grad.numpy(), rtol=1e-9, atol=1e-10,
                                   err_msg=name)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5])
def test_backward_of_sequences_shorter_than_the_conv(T):
    """Sequences of fewer steps than the conv's width: the transposed conv then drops the
    taps that reach past the end (no index wraps round)."""
    p, st, dy, dhT, c = _problem(22 + T, 2, T, 8)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    y, hT = _torch_forward(t, st, c)
    loss = (torch.as_tensor(dy) * y).sum() + (torch.as_tensor(dhT) * hT).sum()
    loss.backward()
    g = _grads(p, st, dy, dhT, c)
    for name in NAMES:
        np.testing.assert_allclose(g[name], t[name].grad.numpy(), rtol=1e-9, atol=1e-10,
                                   err_msg=name)
