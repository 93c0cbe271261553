"""Oracle for the AdamW elementwise step (test infrastructure only).

The pages route embedding, prediction head, RMSNorm weights, biases and gate
factors to AdamW (the deep-dive page, "为什么嵌入层、输出头、bias、RMSNorm 还在用
AdamW"; DeepSeek-V4 book ch. 6, §7).  The form used is the one the deep-dive
page describes in "AdamW 到底哪里不协调" (bias-corrected first and second
moments) with the decoupled multiplicative decay it describes in
"V4 的完整更新公式" (step 5):

    p  <- (1 - lr*wd) * p
    m  <- beta1 * m + (1 - beta1) * g
    v  <- beta2 * v + (1 - beta2) * g^2
    p  <- p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)

Arithmetic: numpy float32, one IEEE round-to-nearest per operation, in
exactly this order; square root and division are correctly rounded.  The
scalars 1 - lr*wd, 1 - beta1, 1 - beta2, 1 - beta1^t and 1 - beta2^t are
formed in float64 and rounded once to float32.
"""

import numpy as np


def adamw_scalars_f32(lr, beta1, beta2, eps, weight_decay, step):
    """The float32 scalars of one AdamW step (see module docstring)."""
    if step < 1:
        raise ValueError("AdamW step count starts at 1")
    f = np.float32
    return {
        "decay": f(1.0 - lr * weight_decay),
        "beta1": f(beta1),
        "beta2": f(beta2),
        "one_minus_beta1": f(1.0 - beta1),
        "one_minus_beta2": f(1.0 - beta2),
        "bias_corr1": f(1.0 - beta1 ** step),
        "bias_corr2": f(1.0 - beta2 ** step),
        "lr": f(lr),
        "eps": f(eps),
    }


def adamw_step_f32(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """One AdamW step; returns (p_new, m_new, v_new) as float32 arrays."""
    k = adamw_scalars_f32(lr, beta1, beta2, eps, weight_decay, step)
    p = np.asarray(p, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    p_decayed = k["decay"] * p
    m_new = (k["beta1"] * m) + (k["one_minus_beta1"] * g)
    v_new = (k["beta2"] * v) + ((k["one_minus_beta2"] * g) * g)
    m_hat = m_new / k["bias_corr1"]
    v_hat = v_new / k["bias_corr2"]
    denom = np.sqrt(v_hat) + k["eps"]
    p_new = p_decayed - (k["lr"] * (m_hat / denom))
    return (p_new.astype(np.float32), m_new.astype(np.float32),
            v_new.astype(np.float32))
