"""Plain fp64 CPU oracle for GQLA decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library under decode_attention_02_amd/ may
import, call or execute this module; only the tests, the smoke check and the CPU
baseline leg of the benchmark use it. It shares no code with the HIP path: it takes
the already-rounded inputs (as fp64) and writes out the definitions one step at a
time, with library matmuls as the only helpers and no blocking, fusion or reordering.

Sources, cited by page title and section:
  [GQLA-A]  "GQLA: Attention latente par requêtes groupées pour le décodage de grands
            modèles de langage adaptatif au matériel" (chatpaper.ai), English abstract.
  [GQLA-B]  "GQLA: Group-Query Latent Attention for Hardware-Adaptive Decoding"
            (scholarbro.com), Abstract.
  [GQA]     "Grouped Query Attention (GQA)" (Ultralytics glossary), sections
            "Fonctionnement de la GQA" and "Pourquoi la GQA réduit le cache KV".
  [MODULE]  gqla_attn.py module source (frankenstein-transformer docs), GQLAAttention
            class docstring and forward().

What the method computes. GQLA keeps MLA's joint low-rank latent c_KV per token and
gives each group of gs = H/G query heads one shared key up-projection W_UK^g and one
value up-projection W_UV^g ([GQLA-B]). The same weights decode two algebraically
equivalent ways ([GQLA-A]): MQA-absorb (W_UK^g folded into each query; every head
attends over the cached latent; W_UV^g applied to the latent output) and GQA (the
latent expanded into G key/value heads that the group's query heads share). Both equal
the head-expanded MLA form ([GQLA-B]), which is `mla_expanded_attention` below.

Readings where the pages are silent (each also listed in the design notes):
  * softmax scale 1/sqrt(d_n + d_R) on every path (the module scales by head_dim**-0.5,
    [MODULE] forward; the non-absorbed query/key width is d_n + d_R);
  * the decoupled RoPE key (d_R values per token) is cached after rotation and shared by
    all heads; it joins the key as [k_nope | k_rope] (the pages never mention RoPE);
  * head h belongs to group h // gs ([GQA] repeat_interleave of key/value heads, and the
    module's view(bsz, G, gs, ...) in forward());
  * with s_q new rows per sequence and a context of L tokens that includes them, row i
    sees tokens 0 .. L - s_q + i (bottom-right causal; the module masks with
    triu(diagonal=1) in decoder mode, which is this rule when the queries are the last
    s_q positions);
  * RoPE rotates half-split pairs (component k with k + d_R/2) at angle
    position * theta^(-2k/d_R), theta = 10000 (`rope_at`; the pages never describe RoPE);
  * the output projection concatenates the heads' outputs head-major before W_O (the
    module's transpose-then-view in forward(); `hidden_projection`);
  * W_UV^g may be folded into W_O on the absorb path (`fold_out_weight`): both are linear
    maps applied one after the other, so this is their product formed once; the pages
    name the absorbed form but not this step.
"""
import math
from typing import List, Sequence, Tuple

import numpy as np

BLOCK = 64


# ---------------------------------------------------------------- basic definitions

def qk_scale(d_nope: int, d_rope: int) -> float:
    """Softmax scale 1/sqrt(d_n + d_R), the width of a non-absorbed query/key head."""
    return 1.0 / math.sqrt(d_nope + d_rope)


def head_group(h: int, num_heads: int, num_groups: int) -> int:
    """Group of query head h: contiguous runs of H/G heads share one key/value head ([GQA])."""
    if num_heads % num_groups:
        raise ValueError("num_groups must divide num_heads")
    return h // (num_heads // num_groups)


def visible_tokens(ctx_len: int, s_q: int, i: int) -> int:
    """Number of tokens row i (0 <= i < s_q) attends to: L - s_q + 1 + i (causal)."""
    return ctx_len - s_q + 1 + i


def softmax_average(scores: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, float]:
    """Softmax-weighted average of value rows, plus log-sum-exp of the scores.

    out = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m),  lse = m + ln sum_t exp(s_t - m),
    m = max_t s_t (scaled dot-product attention, [GQA] "Fonctionnement de la GQA").
    """
    m = float(np.max(scores))
    w = np.exp(scores - m)
    total = float(np.sum(w))
    return (w @ values) / total, m + math.log(total)


# ------------------------------------------------- definition: head-expanded MLA form

def mla_expanded_attention(c, kr, w_uk, w_uv, q_nope, q_rope, s_q, scale):
    """Non-absorbed (head-expanded) attention of one sequence: the definition ([GQLA-B]).

    c [L][d_c] latent, kr [L][d_R] rotated RoPE keys, w_uk [G][d_n][d_c],
    w_uv [G][d_v][d_c], q_nope [s_q][H][d_n], q_rope [s_q][H][d_R].
    Head h in group g sees keys K = [c W_UK^g^T | kr] and values V = c W_UV^g^T.
    Returns out [s_q][H][d_v] and lse [s_q][H].
    """
    L = c.shape[0]
    H = q_nope.shape[1]
    G = w_uk.shape[0]
    d_v = w_uv.shape[1]
    out = np.zeros((s_q, H, d_v))
    lse = np.zeros((s_q, H))
    kv = {}   # K and V of a group, formed the first time one of its heads needs them
    for h in range(H):
        g = head_group(h, H, G)
        if g not in kv:
            kv[g] = (np.concatenate([c @ w_uk[g].T, kr], axis=1), c @ w_uv[g].T)
        k, v = kv[g]
        for i in range(s_q):
            n = visible_tokens(L, s_q, i)
            q = np.concatenate([q_nope[i, h], q_rope[i, h]])
            out[i, h], lse[i, h] = softmax_average(scale * (k[:n] @ q), v[:n])
    return out, lse


def brute_mla_attention(c, kr, w_uk, w_uv, q_nope, q_rope, s_q, scale):
    """The same definition in pure Python loops (math.exp, math.fsum), for tiny shapes."""
    c, kr, w_uk, w_uv = (np.asarray(a).tolist() for a in (c, kr, w_uk, w_uv))
    q_nope, q_rope = np.asarray(q_nope).tolist(), np.asarray(q_rope).tolist()
    L, d_c = len(c), len(c[0])
    H, G = len(q_nope[0]), len(w_uk)
    d_n, d_v = len(w_uk[0]), len(w_uv[0])
    out = [[[0.0] * d_v for _ in range(H)] for _ in range(s_q)]
    lse = [[0.0] * H for _ in range(s_q)]
    for i in range(s_q):
        n = L - s_q + 1 + i
        for h in range(H):
            g = h // (H // G)
            scores = []
            for t in range(n):
                key = [math.fsum(c[t][j] * w_uk[g][e][j] for j in range(d_c)) for e in range(d_n)]
                key += kr[t]
                q = q_nope[i][h] + q_rope[i][h]
                scores.append(scale * math.fsum(a * b for a, b in zip(q, key)))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            tot = math.fsum(w)
            for e in range(d_v):
                acc = math.fsum(
                    w[t] * math.fsum(c[t][j] * w_uv[g][e][j] for j in range(d_c)) for t in range(n))
                out[i][h][e] = acc / tot
            lse[i][h] = m + math.log(tot)
    return np.array(out), np.array(lse)


# --------------------------------------------------------------- path (a): MQA-absorb

def absorb_query(q_nope, q_rope, w_uk):
    """Fold W_UK^g into each query ([GQLA-A]; [MODULE] docstring, MQA-absorb path).

    q_nope [..][H][d_n], q_rope [..][H][d_R] -> q_abs [..][H][d_c + d_R] with
    q_abs[.., h] = [W_UK^g^T q_nope[.., h] ; q_rope[.., h]], g the group of h.
    """
    H = q_nope.shape[-2]
    G, _, d_c = w_uk.shape
    lead = q_nope.shape[:-2]
    q_abs = np.zeros(lead + (H, d_c + q_rope.shape[-1]))
    for h in range(H):
        g = head_group(h, H, G)
        q_abs[..., h, :d_c] = q_nope[..., h, :] @ w_uk[g]
        q_abs[..., h, d_c:] = q_rope[..., h, :]
    return q_abs


def absorb_attention(q_abs, c, kr, s_q, scale):
    """Every head attends over the one shared latent "key head" [c | kr] with the latent c
    as its value ([MODULE] docstring: a single MQA-style head per layer).

    q_abs [s_q][H][d_c + d_R] -> o_lat [s_q][H][d_c], lse [s_q][H].
    """
    L = c.shape[0]
    H = q_abs.shape[1]
    key = np.concatenate([c, kr], axis=1)
    o_lat = np.zeros((s_q, H, c.shape[1]))
    lse = np.zeros((s_q, H))
    for i in range(s_q):
        n = visible_tokens(L, s_q, i)
        for h in range(H):
            o_lat[i, h], lse[i, h] = softmax_average(scale * (key[:n] @ q_abs[i, h]), c[:n])
    return o_lat, lse


def out_projection(o_lat, w_uv):
    """Apply W_UV^g to each head's latent output: out[.., h] = W_UV^g o_lat[.., h]."""
    H = o_lat.shape[-2]
    G, d_v, _ = w_uv.shape
    out = np.zeros(o_lat.shape[:-1] + (d_v,))
    for h in range(H):
        out[..., h, :] = o_lat[..., h, :] @ w_uv[head_group(h, H, G)].T
    return out


# ------------------------------------------------------ output side: W_O and its fold

def hidden_projection(out, w_o):
    """The module's output projection ([MODULE] forward(), its last step): the heads'
    outputs laid side by side head-major (feature h*d_v + v of the concatenation is value
    v of head h) and multiplied by W_O^T, W_O being [hidden][H*d_v]:
    y[.., n] = sum_h sum_v W_O[n, h*d_v + v] out[.., h, v]."""
    flat = out.reshape(out.shape[:-2] + (out.shape[-2] * out.shape[-1],))
    return flat @ w_o.T


def fold_out_weight(w_o, w_uv, num_heads):
    """W_O with every head's value up-projection folded in. On the absorb path (MLA's
    absorbed form, [GQLA-A]) W_UV^g acts on each head's latent output and W_O right after
    it; both are linear, so their product can be formed once (reading: the pages name the
    absorbed form but not this step; it is associativity of the two products):
    W_fold[n, h*d_c + c] = sum_v W_O[n, h*d_v + v] W_UV^g[v, c]."""
    G, d_v, d_c = w_uv.shape
    hidden = w_o.shape[0]
    w_fold = np.zeros((hidden, num_heads * d_c))
    for h in range(num_heads):
        w_fold[:, h * d_c:(h + 1) * d_c] = w_o[:, h * d_v:(h + 1) * d_v] @ w_uv[head_group(h, num_heads, G)]
    return w_fold


def folded_hidden_projection(o_lat, w_fold):
    """The absorb path's output side with the folded weight: the heads' latent outputs
    laid side by side head-major and multiplied by W_fold^T."""
    flat = o_lat.reshape(o_lat.shape[:-2] + (o_lat.shape[-2] * o_lat.shape[-1],))
    return flat @ w_fold.T


# ------------------------------------------------------------------- path (b): GQA

def expand_latent(c, kr, w_uk, w_uv):
    """Expand the latent into G full key/value heads ([MODULE] docstring, GQA path).

    c [L][d_c], kr [L][d_R] -> K [G][L][d_n + d_R] = [c W_UK^g^T | kr],
                               V [G][L][d_v]       = c W_UV^g^T.
    """
    G = w_uk.shape[0]
    K = np.stack([np.concatenate([c @ w_uk[g].T, kr], axis=1) for g in range(G)])
    V = np.stack([c @ w_uv[g].T for g in range(G)])
    return K, V


def gqa_attention(q, K, V, s_q, scale):
    """Standard grouped-query attention: head h uses key/value head g = h // gs ([GQA]).

    q [s_q][H][d_qk], K [G][L][d_qk], V [G][L][d_v] -> out [s_q][H][d_v], lse [s_q][H].
    """
    H = q.shape[1]
    G, L, _ = K.shape
    out = np.zeros((s_q, H, V.shape[2]))
    lse = np.zeros((s_q, H))
    for i in range(s_q):
        n = visible_tokens(L, s_q, i)
        for h in range(H):
            g = head_group(h, H, G)
            out[i, h], lse[i, h] = softmax_average(scale * (K[g, :n] @ q[i, h]), V[g, :n])
    return out, lse


# ------------------------------------------------------------------- paged caches

def gather_tokens(cache, block_table_row, n_tokens):
    """Logical rows 0..n-1 of one sequence from a paged cache: token t lives in slot
    t % 64 of physical block block_table_row[t // 64] (fixed-size KV blocks, [GQA]
    "GQA et techniques connexes", PagedAttention)."""
    rows = []
    for t in range(n_tokens):
        rows.append(cache[block_table_row[t // BLOCK], t % BLOCK])
    return np.array(rows)


def expand_blocks(latent_cache, block_ids, w_uk, w_uv, d_c):
    """Expansion of whole physical latent blocks into per-group K and V.

    latent_cache [NB][64][d_c + d_R]; returns K [n][G][64][d_qk], V [n][G][64][d_v]
    for the listed blocks, in logical (token-major) order.
    """
    Ks, Vs = [], []
    for p in block_ids:
        rows = latent_cache[p]
        K, V = expand_latent(rows[:, :d_c], rows[:, d_c:], w_uk, w_uv)
        Ks.append(K)
        Vs.append(V)
    return np.array(Ks), np.array(Vs)


# ------------------------------------------------------------------- append path

def rope_at(x, position, theta=10000.0):
    """Rotary position embedding of one d_R-vector at an integer position.

    The pages never describe RoPE; reading: half-split pairs, i.e. component k is paired
    with component k + d_R/2 and the pair is rotated by the angle
    position * theta**(-2k/d_R) (x_k cos - x_{k+d/2} sin, x_k sin + x_{k+d/2} cos).
    """
    d = len(x)
    half = d // 2
    out = np.zeros(d)
    for k in range(half):
        angle = position * theta ** (-2.0 * k / d)
        c, s = math.cos(angle), math.sin(angle)
        out[k] = x[k] * c - x[k + half] * s
        out[k + half] = x[k] * s + x[k + half] * c
    return out


def append_rows(c_new, kr_new, ctx_lens, s_q, theta=10000.0):
    """Cache rows that appending each sequence's s_q new tokens writes: row i of sequence
    b sits at position t = L_b - s_q + i (the context counts the new tokens) and is stored
    as [c ; RoPE_t(k_rope)] (the latent from the down-projection plus the rotated
    decoupled key, cached once per token for all heads).

    c_new [B][s_q][d_c], kr_new [B][s_q][d_R] -> {(b, t): row [d_c + d_R]}.
    """
    rows = {}
    for b in range(len(ctx_lens)):
        L = int(ctx_lens[b])
        if L < s_q:
            continue
        for i in range(s_q):
            t = L - s_q + i
            rows[(b, t)] = np.concatenate([c_new[b, i], rope_at(kr_new[b, i], t, theta)])
    return rows


# ----------------------------------------------------------- split-KV partial merge

def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[float]):
    """Combine softmax averages over disjoint token ranges into the average over their
    union: weight each part by exp(lse_s - M), M = max lse_s; lse = M + ln sum weights.
    Parts with lse = -inf (no visible token) carry zero weight."""
    lses = np.asarray(lses, dtype=np.float64)
    m = float(np.max(lses))
    w = np.exp(lses - m)
    total = float(np.sum(w))
    acc = sum(wi * np.asarray(o) for wi, o in zip(w, outs))
    return acc / total, m + math.log(total)


def attention_over_ranges(scores, values, bounds: List[int]):
    """Softmax average computed separately on [bounds[j], bounds[j+1]) and merged."""
    outs, lses = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b > a:
            o, l = softmax_average(scores[a:b], values[a:b])
        else:
            o, l = np.zeros(values.shape[1]), -math.inf
        outs.append(o)
        lses.append(l)
    return merge_partials(outs, lses)


# ------------------------------------------------------------ cache sizes per token

def latent_values_per_token(d_c: int, d_rope: int) -> int:
    """Values cached per token per layer on the MQA-absorb path: the joint latent plus
    the shared RoPE key ([GQLA-A])."""
    return d_c + d_rope


def kv_values_per_token(kv_heads: int, head_dim: int) -> int:
    """Values cached per token per layer by a GQA/MHA layer: one key and one value vector
    per key/value head ([GQA] "Pourquoi la GQA réduit le cache KV")."""
    return 2 * kv_heads * head_dim


def expanded_values_per_token(groups: int, d_qk: int, d_v: int) -> int:
    """Values cached per token per layer by the GQA path's expanded cache."""
    return groups * (d_qk + d_v)


# ------------------------------------------------------------- batch-level drivers

def batch_naive(c_seq, kr_seq, w_uk, w_uv, q_nope, q_rope, s_q, scale, seqs=None):
    """mla_expanded_attention for each listed sequence; returns lists of (out, lse)."""
    seqs = range(len(c_seq)) if seqs is None else seqs
    return [mla_expanded_attention(c_seq[b], kr_seq[b], w_uk, w_uv, q_nope[b], q_rope[b],
                                   s_q, scale) for b in seqs]


def batch_absorb(c_seq, kr_seq, w_uk, w_uv, q_nope, q_rope, s_q, scale, seqs=None):
    """Full MQA-absorb path per listed sequence: (q_abs, o_lat, lse, out)."""
    seqs = range(len(c_seq)) if seqs is None else seqs
    res = []
    for b in seqs:
        q_abs = absorb_query(q_nope[b], q_rope[b], w_uk)
        o_lat, lse = absorb_attention(q_abs, c_seq[b], kr_seq[b], s_q, scale)
        res.append((q_abs, o_lat, lse, out_projection(o_lat, w_uv)))
    return res


def batch_gqa(c_seq, kr_seq, w_uk, w_uv, q, s_q, scale, seqs=None):
    """Full GQA path per listed sequence: (out, lse)."""
    seqs = range(len(c_seq)) if seqs is None else seqs
    res = []
    for b in seqs:
        K, V = expand_latent(c_seq[b], kr_seq[b], w_uk, w_uv)
        res.append(gqa_attention(q[b], K, V, s_q, scale))
    return res
