"""The attention sub-layer around the hot path, with given weights (oracle; test infrastructure only).

The seven steps of the Qwen3 attention sub-layer [P2 §2; P1 attention.py walkthrough]:

1. ``qkv = x W_qkv^T`` -- one merged projection of the hidden states;
2. split into q ``[N, Hq, hd]``, k and v ``[N, Hkv, hd]`` (the ``[Hq*hd, Hkv*hd, Hkv*hd]`` split and views);
3. (views only);
4. QK-Norm of q and k, each head over its hd elements with its own weight;
5. RoPE of q and k by each token's absolute position in its sequence;
6. store k and v in the paged cache, then attention: causal varlen over each sequence's keys (prefill) or
   one query against the whole context (decode);
7. ``y = o W_o^T`` after flattening o ``[N, Hq, hd]`` to ``[N, Hq*hd]`` [P2 §6].

Here the sequences are kept as plain per-sequence arrays of their (normalised, rotated) keys and values -- the
logical K/V the paged cache holds -- so this oracle checks the sub-layer's arithmetic, not the cache layout
(the cache layout has its own pins).  float64 throughout, no intermediate rounding.
"""

import numpy as np

from .attention import attention_ref
from .qknorm_rope import qk_norm_rope_ref


def project_split_ref(x, w_qkv, num_q_heads, num_kv_heads, head_dim):
    """Steps 1-3: returns q ``[N, Hq, hd]``, k, v ``[N, Hkv, hd]`` in float64."""
    x = np.asarray(x, dtype=np.float64)
    qkv = x @ np.asarray(w_qkv, dtype=np.float64).T
    nq, nk = num_q_heads * head_dim, num_kv_heads * head_dim
    n = x.shape[0]
    q = qkv[:, :nq].reshape(n, num_q_heads, head_dim)
    k = qkv[:, nq:nq + nk].reshape(n, num_kv_heads, head_dim)
    v = qkv[:, nq + nk:nq + 2 * nk].reshape(n, num_kv_heads, head_dim)
    return q, k, v


def sublayer_step_ref(x, positions, hist_k, hist_v, w_qkv, q_norm_w, k_norm_w, w_o, num_q_heads, num_kv_heads,
                      head_dim, eps, theta, scale):
    """One sequence's step: ``x [n, hidden]`` are its new tokens at ``positions`` (the last n positions),
    ``hist_k``/``hist_v`` ``[p, Hkv, hd]`` its cached (already normalised and rotated) keys and values.
    Returns ``(y [n, hidden], k_all, v_all)``: the output and the sequence's keys and values after the step."""
    q, k, v = project_split_ref(x, w_qkv, num_q_heads, num_kv_heads, head_dim)
    qn, kn = qk_norm_rope_ref(q, k, positions, q_norm_w, k_norm_w, eps, theta)
    k_all = np.concatenate([np.asarray(hist_k, dtype=np.float64).reshape(-1, num_kv_heads, head_dim), kn])
    v_all = np.concatenate([np.asarray(hist_v, dtype=np.float64).reshape(-1, num_kv_heads, head_dim), v])
    n, lk = x.shape[0], k_all.shape[0]
    o = attention_ref(qn, k_all, v_all, [0, n], [0, lk], scale, causal=True)
    y = o.reshape(n, num_q_heads * head_dim) @ np.asarray(w_o, dtype=np.float64).T
    return y, k_all, v_all
