"""QK-Norm and RoPE on the new tokens' q and k, then the store (oracle; test infrastructure only).

The attention sub-layer runs, between splitting the merged projection and calling attention [P2 §2, the
seven steps; §4 "QK-Norm 与 RoPE"]:

* step 4, QK-Norm: every head's q vector and k vector is RMS-normalised over its head_dim elements, each
  head on its own, then scaled elementwise by a learned weight of head_dim entries (one weight for q, one
  for k) [P2 §4]; the RMSNorm itself divides by the root of the mean square plus eps [P1, layernorm.py
  walkthrough];
* step 5, RoPE: q and k (not v) are rotated according to each token's absolute position [P2 §4];
* step 6, first half: k and v are written to the paged cache at slot_mapping [P2 §5.1] -- the store of
  ``store.store_ref``; the page's integration check compares the cache's k rows with the normalised and
  rotated k [P2 §7].

Readings where the page leaves a step open:

* RoPE's formula is left to another lesson; the plain reading is the rotary embedding of RoFormer in the
  "rotate half" layout: element i of a head is paired with element i + head_dim/2 and the pair is rotated
  by the angle position * theta^(-2i/head_dim), i < head_dim/2.  The base theta is an argument.
* Precision: float64 throughout with no intermediate rounding (P1's RMSNorm rounds to the input type
  before the weight multiply; the kernel keeps float32 through RoPE and rounds once at the end).
"""

import numpy as np


def rms_norm_ref(x, weight, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * weight, in float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * w


def rope_angles_ref(positions, head_dim, theta):
    """[N, head_dim/2] rotation angles: position * theta^(-2i/head_dim)."""
    pos = np.asarray(positions, dtype=np.float64)
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / head_dim)
    return pos[:, None] * inv_freq[None, :]


def rope_ref(x, positions, theta):
    """Rotate ``x`` [N, heads, head_dim] by each token's position (pairs i, i + head_dim/2)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    ang = rope_angles_ref(positions, hd, theta)[:, None, :]  # broadcast over heads
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def qk_norm_rope_ref(q, k, positions, q_weight, k_weight, eps, theta):
    """Steps 4 and 5 for the new tokens: returns (q', k') in float64."""
    qn = rms_norm_ref(q, q_weight, eps)
    kn = rms_norm_ref(k, k_weight, eps)
    return rope_ref(qn, positions, theta), rope_ref(kn, positions, theta)
