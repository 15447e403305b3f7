"""Plain statement of the projections around the absorbed decode step.

TEST INFRASTRUCTURE: used by tests, the smoke check and the benchmark's CPU
baseline only.  The GPU library never imports it and shares no code with it.

Sources (cited by page title and section):

* [MLRA]  "超越MLA！新架构MLRA百万token，解码最高2.8倍速 | ICLR'26" (aitntnews): the MLA
  paragraph (W_UK is folded into the query, so attention runs in latent space
  and the latent output is mapped back by W_UV) and "求和顺序外移 (Moving the Sum
  Outside)" (the branch outputs are summed after each is projected).
* The "MLA vs MQA" page (developer.baidu.com), its list of engineering needs:
  a custom kernel for the latent projection.

Every projection here is, per head h, C[m, h, :] = W[h] A[m, h, :] with W[h]
stored [N, K] (row n holds the K weights of output n):

* query absorption: A = q^C [B, H, d_nope], W[h] = W_UK[h]^T [d_latent, d_nope]
  (so C = q_lat = W_UK^T q^C, the ``absorb_query`` of attention.py);
* output up-projection: A = o_lat [B, H, d_latent], W[h] = W_UV[h] [d_v, d_latent];
* MLRA: A = the branch outputs of a head side by side [B, H, G*d_latent],
  W[h] = [W_UV^0[h] | ... | W_UV^{G-1}[h]] [d_v, G*d_latent], which is the sum
  over branches of W_UV^beta[h] o_beta.
"""
from __future__ import annotations

import numpy as np

__all__ = ["head_projection", "stack_branch_weights"]


def head_projection(A, W):
    """C[m, h, n] = sum_k W[h, n, k] A[m, h, k] in fp64.  A [M, H, K], W [H, N, K] -> [M, H, N]."""
    A = np.asarray(A, np.float64)
    W = np.asarray(W, np.float64)
    M, H, K = A.shape
    out = np.empty((M, H, W.shape[1]))
    for h in range(H):
        out[:, h, :] = A[:, h, :] @ W[h].T
    return out


def stack_branch_weights(W_branches):
    """[G, H, d_v, d_latent] per-branch up-projections -> [H, d_v, G*d_latent] side by side."""
    W = np.asarray(W_branches)
    G, H, dv, dc = W.shape
    return np.transpose(W, (1, 2, 0, 3)).reshape(H, dv, G * dc)
