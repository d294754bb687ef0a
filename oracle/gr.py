"""Plain fp64 CPU oracle of the gated residual read and write around a
sublayer (the MoE layer here).

TEST INFRASTRUCTURE ONLY.  Only the tests may import or run this module; the
library path never calls it and shares no code with it.

Source: the Qwen3.8-Flash-Next study, section "Gated residual: four streams,
one sublayer input" (its four equations); the RMSNorm epsilon is the model
config's rms_norm_eps (model-atlas page "Qwen3.8 2.4T A95B", raw config).

  Rhat_i = GroupRMSNorm(R_i)                    each stream i = 0..3 alone
  G      = sigmoid(W_up SiLU(W_down vec(Rhat) / 4))
  x      = mean_i (G_i * Rhat_i),   s = 2 sigmoid(W_write vec(Rhat) / 4)
  R'_i   = R_i + s_i F(x)

Readings where the section leaves a step open (listed in the design notes):
  * GroupRMSNorm of stream i: R_i / sqrt(mean_c R_i[c]^2 + eps) times a
    learned per-channel gain g_i (the section says each stream is normalised
    independently; the gain is the usual RMSNorm weight);
  * the "/ 4" divides the flattened normalised streams (equivalently the
    projection, which is linear);
  * W_down [r, 4H] and the four write-gate rows W_write [4, 4H] read the same
    input and are passed as one matrix w_read = [W_down; W_write];
  * vec(Rhat) flattens the streams in order, stream i at columns iH .. iH+H-1,
    and G_i is rows iH .. iH+H-1 of G.
Everything is computed in fp64 from the stored values; nothing is rounded.
"""
from __future__ import annotations

import numpy as np


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def group_rmsnorm(resid: np.ndarray, norm_w: np.ndarray, eps: float) -> np.ndarray:
    """resid [T, 4, H] -> each stream divided by its root mean square (plus
    eps under the root), times the stream's gain norm_w [4, H]."""
    r = np.asarray(resid, np.float64)
    rms = np.sqrt(np.mean(r * r, axis=2, keepdims=True) + eps)
    return r / rms * np.asarray(norm_w, np.float64)[None]


def gr_read(resid, norm_w, w_read, w_up, eps: float = 1e-6):
    """Returns (x [T, H], s [T, 4], rhat [T, 4, H], G [T, 4, H])."""
    T, S, H = resid.shape
    rank = w_read.shape[0] - S
    rhat = group_rmsnorm(resid, norm_w, eps)
    v = rhat.reshape(T, S * H) / 4.0
    proj = v @ np.asarray(w_read, np.float64).T          # [T, rank + 4]
    z = silu(proj[:, :rank])
    s = 2.0 * sigmoid(proj[:, rank:])
    G = sigmoid(z @ np.asarray(w_up, np.float64).T).reshape(T, S, H)
    x = np.mean(G * rhat, axis=1)
    return x, s, rhat, G


def gr_write(resid, s, f):
    """R'_i = R_i + s_i F: resid [T, 4, H], s [T, 4], f [T, H]."""
    return np.asarray(resid, np.float64) + np.asarray(s, np.float64)[:, :, None] * np.asarray(f, np.float64)[:, None, :]
