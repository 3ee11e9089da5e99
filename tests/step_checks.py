"""Checks on a whole training step shared by the full-size GPU tests."""


def check_first_order_step(M, di, dt, loss):
    """One AdamW step at t = 1 moves every parameter by -lr g / (|g| + eps)
    (bias-corrected moments m = g, v = g^2; no weight decay), so for a small
    lr the loss must drop by lr * sum g^2 / (|g| + eps) to first order.  lr is
    chosen so that this predicted drop is 0.1 (second-order terms then stay a
    few percent); the measured drop must match it: a check of the gradients'
    size and direction over all parameters at once."""
    eps = 1e-8
    gd = M.grads.double()
    pred_per_lr = float((gd * gd / (gd.abs() + eps)).sum())
    del gd
    lr = 0.1 / pred_per_lr
    M.update(lr=lr, beta1=0.9, beta2=0.999, eps=eps, weight_decay=0.0, t=1)
    loss2 = M.forward(di, dt)
    ratio = (loss - loss2) / (lr * pred_per_lr)
    print(f"lr {lr:.3g}: loss {loss:.6f} -> {loss2:.6f}, drop / first-order prediction {ratio:.4f}", flush=True)
    assert 0.8 <= ratio <= 1.02, ratio
