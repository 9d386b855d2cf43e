"""The steps on either side of the KDA recurrence in a layer, in fp64 numpy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Plain definitions, one
array operation per step, no fusion:

  prologue (per token t, head h, channel c):
    conv   y_t = sum_{j=0..3} w[j] x_{t-3+j}: causal depthwise convolution of
           width 4 per channel, with the previous call's last three inputs
           (the conv cache) standing for x_{-3..-1} (zeros without a cache).
           Source: "Kimi K3 核心算子拆解" (devpress.csdn.net) section 2.6
           (weight index 0 applies to t-3, index 3 to t) and "Kimi K3 四个核心
           模块的公式与真实张量流" (gentlecold.top) section 1.2 (q, k and v each
           take the width-4 causal depthwise convolution, then Swish; q and k
           are L2-normalised; the last 3 inputs per channel persist).
    q = l2norm(silu(conv(q_raw))), k = l2norm(silu(conv(k_raw))),
    v = silu(conv(v_raw)),  silu(z) = z sigmoid(z),
    l2norm(x) = x / sqrt(sum_c x_c^2 + eps) over the head's 128 channels.
    log_alpha = -5 sigmoid(a): the lower-bounded log decay g_min sigmoid(.)
           with g_min = -5, "Kimi K3 技术报告解读" (marsggbo.github.io)
           section 3.3 (class KDA) and section 3.5.
    beta = sigmoid(b): the write strength, same class KDA.
  epilogue:
    out = o / sqrt(mean_c o_c^2 + eps) * w * sigmoid(g): RMSNorm over the
           head's channels with a per-channel weight, then the sigmoid output
           gate ("把注意力换成一块「会遗忘的内存」" (jokeuncle.github.io),
           section "层的实现" (the gated RMSNorm with sigmoid activation);
           gentlecold.top section 1.4 (a full-rank gate per head and channel)).

Shapes: x_raw, a, g, o [T, H, d]; b [T, H]; conv weights [H, d, 4];
conv cache [3, H, d] (inputs at t-3, t-2, t-1); w [d].
"""
from __future__ import annotations

import numpy as np

G_MIN = -5.0
L2_EPS = 1e-6
RMS_EPS = 1e-6


def sigmoid(x):
    x = np.asarray(x, np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = np.asarray(x, np.float64)
    return x * sigmoid(x)


def short_conv(x_raw, w, cache=None):
    """Causal depthwise width-4 convolution of one sequence.
    x_raw [T, H, d], w [H, d, 4], cache [3, H, d] or None.
    Returns (y [T, H, d], new cache [3, H, d] = the last three inputs)."""
    x = np.asarray(x_raw, np.float64)
    T = x.shape[0]
    prev = np.zeros((3,) + x.shape[1:]) if cache is None else np.asarray(cache, np.float64)
    ext = np.concatenate([prev, x], axis=0)          # ext[t + 3] = x_t
    w = np.asarray(w, np.float64)
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(4):
            y[t] += w[..., j] * ext[t + j]               # ext[t + j] = x_{t - 3 + j}
    return y, ext[T:T + 3].copy()


def l2norm(x, eps=L2_EPS):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def prologue(q_raw, k_raw, v_raw, conv_w, a, b, cache=None):
    """One sequence.  conv_w [3, H, d, 4] for (q, k, v); cache [3, 3, H, d]
    (tensor, tap) or None.  Returns q, k, v, log_alpha [T, H, d], beta [T, H]
    and the new cache [3, 3, H, d]."""
    outs, caches = [], []
    for i, x in enumerate((q_raw, k_raw, v_raw)):
        y, c = short_conv(x, conv_w[i], None if cache is None else cache[i])
        outs.append(silu(y))
        caches.append(c)
    q, k, v = l2norm(outs[0]), l2norm(outs[1]), outs[2]
    log_alpha = G_MIN * sigmoid(a)
    beta = sigmoid(b)
    return q, k, v, log_alpha, beta, np.stack(caches)


def epilogue(o, g, w, eps=RMS_EPS):
    o = np.asarray(o, np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * np.asarray(w, np.float64) * sigmoid(g)
