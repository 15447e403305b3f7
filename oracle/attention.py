"""Plain, slow, fp64 statement of what decode attention over a shrunk cache computes.

TEST INFRASTRUCTURE: used by tests, the smoke check and the benchmark's CPU
baseline only.  Nothing here is blocked, fused or reordered beyond what the
definitions below say; matrix products and sums are numpy's.

Sources (cited by page title and section):

* [MLA-RoPE]  the MLA explainer on mlqm.cn (news 371735): section 2.1 (latent
  compression), 2.2 (the semantic branch and the separate RoPE branch,
  q = [q^C, q^R], k = [k^C, k^R]), 2.3 (o_{t,i} = sum_j softmax_j(q^T k / sqrt(d))
  v^C_{j,i}; only the semantic value enters the output; the scale uses the
  full concatenated dimension).
* [MLRA]  "超越MLA！新架构MLRA百万token，解码最高2.8倍速 | ICLR'26" (aitntnews):
  the MLA paragraph (W_UK absorbed into the query so per-head K/V are never
  materialised; absorbed MLA decode is one 576-dim MQA), "块分解视角 (The Block
  Decomposition)" and "求和顺序外移 (Moving the Sum Outside)" (four sub-blocks,
  attention per branch, branch outputs summed).
* [GTA-GLA]  "Mamba核心作者新作：取代DeepSeek在用的注意力机制，专为推理打造"
  (jsbsmhs.com): "分组绑定注意力机制 GTA" (heads in a group share tied K and V)
  and "分组潜在注意力机制 GLA" (head groups, each attending its own latent).
* GQA / MQA sharing: the [MLRA] page's list of cache-reduction methods.

Readings where the pages are silent:
the cache row holds the latent followed by the already rotated RoPE key; the
query sits at position L-1 and attends tokens [0, L) with no mask; an empty
sequence gives out = 0 and lse = -inf; lse is the natural log of the sum of
exp(scaled score); GLA heads are split into contiguous groups; MLRA shares one
RoPE key per token and has a RoPE query per branch, with one softmax per
branch; fp8 is OCP E4M3 with a per-token fp32 scale; with several query
tokens per sequence (multi-token decode) token i of Q sits at position
L-Q+i and attends rows [0, L-Q+i] (causal), nothing when that is empty.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "attend", "attend_heads", "attend_split", "combine_partials",
    "rope", "e4m3_value", "e4m3_decode",
    "logical_rows", "absorb_query",
    "mla_materialised", "gla_materialised", "mlra_materialised", "shared_kv_attention",
    "decode_paged", "decode_paged_tokens",
]


# ----------------------------------------------------------------------------------------------
# softmax attention of one query ([MLA-RoPE] section 2.3)
# ----------------------------------------------------------------------------------------------
def attend(q, K, V, scale: float):
    """One query row against L key/value rows.

    s_j = scale * (q . k_j);  o = sum_j softmax_j(s) v_j;  lse = log sum_j exp(s_j).
    L = 0 gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], np.float64), -np.inf
    s = scale * (K @ q)
    m = np.max(s)
    w = np.exp(s - m)
    l = np.sum(w)
    o = (w / l) @ V
    return o, m + np.log(l)


def attend_heads(Q, K, V, scale: float):
    """Every row of Q (one per head) attends the same K/V rows; rows are independent.

    Returns o [H, dv] and lse [H].  Same definition as ``attend`` per row.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    H = Q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1]), np.float64), np.full(H, -np.inf)
    S = scale * (Q @ K.T)                      # [H, L]
    m = np.max(S, axis=1, keepdims=True)
    W = np.exp(S - m)
    l = np.sum(W, axis=1, keepdims=True)
    O = (W / l) @ V
    return O, (m + np.log(l))[:, 0]


def attend_split(q, K, V, scale: float, bounds):
    """Attention of one query restricted to each token range [a, b) of ``bounds``.

    Each range yields its own normalised output and its own lse (a partial result).
    """
    return [attend(q, K[a:b], V[a:b], scale) for a, b in bounds]


def combine_partials(outs, lses):
    """Merge partial results of disjoint token ranges into the full-range result.

    With lse = log sum_s exp(lse_s):  o = sum_s exp(lse_s - lse) o_s.
    Empty parts (lse_s = -inf) carry zero weight; if every part is empty the
    result is o = 0, lse = -inf.
    """
    lses = np.asarray(lses, np.float64)
    if lses.size == 0:                    # no parts: the empty sum
        return np.zeros(np.shape(outs)[1:], np.float64), -np.inf
    outs = np.asarray(outs, np.float64)
    M = np.max(lses)
    if M == -np.inf:
        return np.zeros(outs.shape[1:], np.float64), -np.inf
    total = M + np.log(np.sum(np.exp(lses - M)))
    w = np.exp(lses - total)
    return np.tensordot(w, outs, axes=(0, 0)), total


# ----------------------------------------------------------------------------------------------
# decoupled RoPE ([MLA-RoPE] section 2.2): used to build inputs upstream of the decode step only
# ----------------------------------------------------------------------------------------------
def rope(x, pos, base: float = 10000.0):
    """Rotate consecutive pairs (x_{2i}, x_{2i+1}) by pos * base^(-2i/d).

    The pages say only that RoPE is a trigonometric rotation; the pair layout
    and the base are a reading.  The decode step consumes already rotated
    vectors, so its result does not depend on this choice.
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[..., None] * base ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return y


# ----------------------------------------------------------------------------------------------
# OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
# S.1111.111 is NaN.  The pages say only that the 236B model was served in FP8 ([GTA-GLA]).
# ----------------------------------------------------------------------------------------------
def e4m3_value(code: int) -> float:
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], np.float64)


def e4m3_decode(codes):
    """Element-wise E4M3 code -> value (a 256-entry table of ``e4m3_value``)."""
    return _E4M3_TABLE[np.asarray(codes, np.uint8)]


# ----------------------------------------------------------------------------------------------
# the paged cache: logical token j of a sequence lives in slot j % page of page table[j // page]
# ----------------------------------------------------------------------------------------------
def logical_rows(pool, table_row, L: int, page_size: int):
    j = np.arange(int(L))
    return np.asarray(pool)[np.asarray(table_row)[j // page_size], j % page_size]


# ----------------------------------------------------------------------------------------------
# the materialised (non-absorbed) forms
# ----------------------------------------------------------------------------------------------
def absorb_query(q_nope, W_UK):
    """Fold the key up-projection into the query ([MLRA], MLA paragraph): q_lat = W_UK^T q^C.

    q_nope [..., dn], W_UK [..., dn, dc] -> [..., dc].
    """
    return np.einsum("...n,...nc->...c", np.asarray(q_nope, np.float64), np.asarray(W_UK, np.float64))


def mla_materialised(q_nope, q_rope, W_UK, W_UV, C, KR, scale: float):
    """Per-head MLA attention with K and V materialised ([MLA-RoPE] 2.2-2.3).

    Head h: k_j = [W_UK[h] c_j ; kr_j], v_j = W_UV[h] c_j, q = [q_nope[h] ; q_rope[h]].
    q_nope [H, dn], q_rope [H, dr], W_UK [H, dn, dc], W_UV [H, dv, dc], C [L, dc], KR [L, dr].
    Returns o [H, dv], lse [H].
    """
    C = np.asarray(C, np.float64)
    KR = np.asarray(KR, np.float64)
    H = q_nope.shape[0]
    outs, lses = [], []
    for h in range(H):
        K = np.concatenate([C @ np.asarray(W_UK[h], np.float64).T, KR], axis=1)
        V = C @ np.asarray(W_UV[h], np.float64).T
        q = np.concatenate([np.asarray(q_nope[h], np.float64), np.asarray(q_rope[h], np.float64)])
        o, lse = attend(q, K, V, scale)
        outs.append(o)
        lses.append(lse)
    return np.array(outs), np.array(lses)


def gla_materialised(q_nope, q_rope, W_UK, W_UV, C_groups, KR, scale: float):
    """GLA ([GTA-GLA], GLA section): head h of H attends group g = h // (H / G).

    C_groups [G, L, dg] are the per-group latents; the RoPE key is shared.
    """
    G = len(C_groups)
    H = q_nope.shape[0]
    per = H // G
    outs, lses = [], []
    for h in range(H):
        g = h // per
        o, lse = mla_materialised(q_nope[h:h + 1], q_rope[h:h + 1], W_UK[h:h + 1], W_UV[h:h + 1],
                                  C_groups[g], KR, scale)
        outs.append(o[0])
        lses.append(lse[0])
    return np.array(outs), np.array(lses)


def mlra_materialised(q_nope, q_rope, W_UK, W_UV, C_branches, KR, scale: float):
    """MLRA ([MLRA], "Moving the Sum Outside"): each branch attends separately, outputs are summed.

    q_nope [H, G, dn], q_rope [H, G, dr], W_UK [H, G, dn, dg], W_UV [H, G, dv, dg],
    C_branches [G, L, dg], KR [L, dr].  Returns o [H, dv] (branch sum) and the
    per-branch lse [H, G].
    """
    H, G = q_nope.shape[0], q_nope.shape[1]
    outs = []
    lses = np.empty((H, G))
    for h in range(H):
        acc = None
        for b in range(G):
            o, lse = mla_materialised(q_nope[h:h + 1, b], q_rope[h:h + 1, b], W_UK[h:h + 1, b],
                                      W_UV[h:h + 1, b], C_branches[b], KR, scale)
            acc = o[0] if acc is None else acc + o[0]
            lses[h, b] = lse[0]
        outs.append(acc)
    return np.array(outs), lses


def shared_kv_attention(Q, K, V, scale: float):
    """GQA / MQA / GTA for one sequence.

    Q [H, d]; K, V [L, n_kv, d].  Head h uses kv head h // (H / n_kv).  MQA is
    n_kv = 1; GTA passes the same array as K and V (tied state).
    """
    Q = np.asarray(Q, np.float64)
    H, nkv = Q.shape[0], K.shape[1]
    per = H // nkv
    outs, lses = [], []
    for h in range(H):
        g = h // per
        o, lse = attend(Q[h], K[:, g], V[:, g], scale)
        outs.append(o)
        lses.append(lse)
    return np.array(outs), np.array(lses)


# ----------------------------------------------------------------------------------------------
# the decode step over the paged cache in the layouts the GPU library consumes
# ----------------------------------------------------------------------------------------------
def decode_paged(variant: str, q_lat, q_rope, k_pool, block_table, seq_lens, *, groups: int, scale: float,
                 page_size: int, v_pool=None, rope_pool=None, scale_pool=None, d_rope: int = 0,
                 batches=None, heads=None):
    """Reference result of one decode step.

    Latent variants (absorbed form, [MLRA] MLA paragraph: every head scores
    against the shared row, the value is the latent part of that row):

    * mla:  row = [c (dc) | kr (dr)]; head h: q = [q_lat[h] | q_rope[h]], K = row, V = c.
    * gla:  row = [c_0 | ... | c_{G-1} | kr]; head h uses c_{h // (H/G)}.
    * mlra: row = [c_0 | ... | c_{G-1} | kr]; (h, branch) uses c_branch with q_lat[h, branch].

    With an fp8 cache, ``k_pool`` holds E4M3 codes of the latent part, the
    latent value is code_value * scale_pool[token], and the RoPE key comes from
    ``rope_pool``.

    Shared variants: gqa / mqa / gta (``v_pool`` None means V is K).

    Returns out [B, H, dv] (mlra: [B, H, G, dv]) and lse [B, H] (mlra: [B, H, G]).
    ``batches`` / ``heads`` restrict the computation to the listed sequences
    and heads (others stay NaN).
    """
    q_lat = np.asarray(q_lat, np.float64)
    B, H = q_lat.shape[0], q_lat.shape[1]
    dv = q_lat.shape[-1]
    out_shape = (B, H, groups, dv) if variant == "mlra" else (B, H, dv)
    out = np.full(out_shape, np.nan)
    lse = np.full(out_shape[:-1], np.nan)
    bs = range(B) if batches is None else batches
    hs = list(range(H)) if heads is None else list(heads)
    fp8 = scale_pool is not None
    for b in bs:
        L = int(seq_lens[b])
        if variant in ("gqa", "mqa", "gta"):
            K = logical_rows(k_pool, block_table[b], L, page_size).astype(np.float64)
            V = K if v_pool is None else logical_rows(v_pool, block_table[b], L, page_size).astype(np.float64)
            o, s = shared_kv_attention(q_lat[b], K, V, scale)
            out[b][hs] = o[hs]
            lse[b][hs] = s[hs]
            continue
        if fp8:
            codes = logical_rows(k_pool, block_table[b], L, page_size)
            sc = logical_rows(scale_pool, block_table[b], L, page_size).astype(np.float64)
            lat = e4m3_decode(codes) * sc[:, None]
            kr = logical_rows(rope_pool, block_table[b], L, page_size).astype(np.float64)
        else:
            rows = logical_rows(k_pool, block_table[b], L, page_size).astype(np.float64)
            lat = rows[:, : rows.shape[1] - d_rope]
            kr = rows[:, rows.shape[1] - d_rope:]
        qr = np.asarray(q_rope, np.float64)
        if variant == "mla":
            Q = np.concatenate([q_lat[b][hs], qr[b][hs]], axis=1)
            o, s = attend_heads(Q, np.concatenate([lat, kr], axis=1), lat, scale)
            out[b][hs] = o
            lse[b][hs] = s
        elif variant == "gla":
            per = H // groups
            dg = dv
            for g in range(groups):
                gh = [h for h in hs if h // per == g]
                if not gh:
                    continue
                c = lat[:, g * dg:(g + 1) * dg]
                Q = np.concatenate([q_lat[b][gh], qr[b][gh]], axis=1)
                o, s = attend_heads(Q, np.concatenate([c, kr], axis=1), c, scale)
                out[b][gh] = o
                lse[b][gh] = s
        elif variant == "mlra":
            dg = dv
            for br in range(groups):
                c = lat[:, br * dg:(br + 1) * dg]
                Q = np.concatenate([q_lat[b][hs, br], qr[b][hs, br]], axis=1)
                o, s = attend_heads(Q, np.concatenate([c, kr], axis=1), c, scale)
                out[b][hs, br] = o
                lse[b][hs, br] = s
        else:
            raise ValueError(f"unknown variant {variant!r}")
    return out, lse


def decode_paged_tokens(variant: str, q_lat, q_rope, k_pool, block_table, seq_lens, *, q_len: int, groups: int,
                        scale: float, page_size: int, v_pool=None, rope_pool=None, scale_pool=None, d_rope: int = 0,
                        batches=None, heads=None):
    """Several query tokens per sequence (mla, mqa): the last ``q_len`` positions of every sequence
    query the cache at once, token i (position L - q_len + i) attending rows 0 .. L - q_len + i.

    Causal attention restricted to the last q_len positions: token i's result is the one-token
    decode (decode_paged) over the cache prefix of length max(0, L - q_len + 1 + i), which is that
    definition written out.  ``q_lat`` / ``q_rope`` hold q_len*H rows per sequence (row i*H + h);
    out and lse come back in the same row order.
    """
    q_lat = np.asarray(q_lat)
    H = q_lat.shape[1] // q_len
    lens = np.asarray(seq_lens, np.int64)
    outs, lses = [], []
    for i in range(q_len):
        rows = slice(i * H, (i + 1) * H)
        qr = None if q_rope is None else np.asarray(q_rope)[:, rows]
        o, s = decode_paged(variant, q_lat[:, rows], qr, k_pool, block_table, np.maximum(lens - q_len + 1 + i, 0),
                            groups=groups, scale=scale, page_size=page_size, v_pool=v_pool, rope_pool=rope_pool,
                            scale_pool=scale_pool, d_rope=d_rope, batches=batches, heads=heads)
        outs.append(o)
        lses.append(s)
    return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1)
