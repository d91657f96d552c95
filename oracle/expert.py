"""SwiGLU expert FFN and the weighted top-k combine, float64.

[PE] "Why is it fast when experts keep crossing PCIe?": an expert of this model
is 3 x 2048 x 768 weights, i.e. the gate, up and down matrices of a SwiGLU FFN.
[PE] "What does Paged Experts actually do?": once the routed experts are
resident, the usual fused MoE computation runs over them; its output for a
token is the router-weighted sum of its top_k experts' outputs.

Reading: standard SwiGLU without biases, h = SiLU(W_gate x) * (W_up x),
y = W_down h, SiLU(a) = a * sigmoid(a); no shared expert.
"""
import numpy as np


def silu(a, dtype=np.float64):
    a = np.asarray(a, dtype=dtype)
    return a / (a.dtype.type(1.0) + np.exp(-a))


def swiglu_expert(w_gate, w_up, w_down, x, dtype=np.float64):
    """x [H] or [n, H] -> y [H] or [n, H], computed in `dtype` (float64 for
    parity; float32 is the variant timed as the CPU baseline)."""
    x = np.asarray(x, dtype=dtype)
    g = x @ w_gate.T
    u = x @ w_up.T
    h = silu(g, dtype) * u
    return h @ w_down.T
