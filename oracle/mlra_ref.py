"""Float64 oracle: MLA and MLRA-n decode attention, written from the pages.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the CPU-baseline leg of the benchmark use it. Plain numpy, float64,
loops over sequences, heads and branches; no blocking, fusion or reordering
beyond what the definitions state.

Notation follows the pages: C_KV (latent cache rows, width d_c), K_RoPE (the
shared decoupled RoPE key, width d_r), W_UK / W_UV (per-head up-projections),
n branches of latent width d_c' = d_c / n, variance scales alpha_q and
alpha_kv, softmax scale tau.

Array conventions (all float64 after conversion):

* ``ckv``    [B, L_max, d_c]  latent rows c_t as stored
* ``krope``  [B, L_max, d_r]  K_RoPE rows, stored already rotated at their
                              own position t
* ``lens``   [B]              valid cache length L_b of each sequence
* ``q_nope`` [B, H, d_n]      NoPE query part
* ``q_rope`` [B, H, d_r]      RoPE query part, not yet rotated
* ``w_uk``   [H, d_c, d_n]    K^N_h = C_KV @ w_uk[h]
* ``w_uv``   [H, d_c, d_v]    V_h   = C_KV @ w_uv[h]

Readings where the pages leave a step open (each is listed with its reason
in the design notes of the repository):

* the query of sequence b sits at position p = L_b - 1 (it attends to all L_b
  cached tokens, its own row included); ``q_pos`` overrides this;
* L_b = 0 gives an all-zero output;
* RoPE pairs consecutive elements (2i, 2i+1) with frequency theta^(-2i/d_r)
  (RoFormer);
* branch j owns the contiguous latent slice [j d_c', (j+1) d_c');
* alpha_q multiplies the NoPE score term of every branch, alpha_kv the summed
  output; tau = (d_n + d_r)^-1/2 unless given.
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rope(x, pos, theta=10000.0):
    """Rotate x[..., d_r] to position ``pos`` (RoFormer rotary embedding).

    Pages: "Multi-Head Low-Rank Attention", 前置知识 / RoPE (scores depend only
    on relative position; MLA applies RoPE to one part of the key only);
    "从MHA到MLA", 3.2 (the RoPE part is rotated by position). The pairing and
    frequencies are RoFormer's: pair i = (x[2i], x[2i+1]) is turned by the
    angle pos * theta^(-2i/d_r).

    ``pos`` is a scalar or an array broadcastable to x.shape[:-1].
    Pinned by closed-form rotations of unit vectors, norm preservation,
    composition and the relative-position property.
    """
    x = _f64(x)
    d_r = x.shape[-1]
    if d_r % 2:
        raise ValueError("RoPE width must be even")
    i = np.arange(d_r // 2, dtype=np.float64)
    omega = theta ** (-2.0 * i / d_r)
    ang = _f64(pos)[..., None] * omega
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d_r,)))
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


def branch_slices(d_c, n):
    """Latent slices of the n branches: branch j owns [j d_c', (j+1) d_c').

    Page: "Multi-Head Low-Rank Attention", 研究动机 (K_NoPE as a sum over
    blocks C_KV^(b) W_UK^(b)) and 方法步骤详情 (each branch takes a quarter of
    C_KV). Pinned by the block-sum identity test.
    """
    if n < 1 or d_c % n:
        raise ValueError("d_c must be a positive multiple of n")
    w = d_c // n
    return [slice(j * w, (j + 1) * w) for j in range(n)]


def _query_pos(lens, q_pos, b):
    return int(lens[b]) - 1 if q_pos is None else int(q_pos[b])


def mlra_decode_ref(q_nope, q_rope, w_uk, w_uv, ckv, krope, lens, n,
                    tau=None, alpha_q=1.0, alpha_kv=1.0, theta=10000.0,
                    q_pos=None):
    """Unabsorbed MLRA-n decode: o = alpha_kv * sum_j softmax(s_j) V_j.

    For each sequence b with L = L_b >= 1, head h and branch j with slice S_j:

    * K^N_j = C[:, S_j] @ W_UK[h][S_j, :] and V_j = C[:, S_j] @ W_UV[h][S_j, :]
      (explicit up-projection of the latent: "MLA多头潜在注意力机制" 3.1, 3.2;
      per-block keys: "Multi-Head Low-Rank Attention", 研究动机);
    * s_j = tau * (alpha_q * K^N_j q^N + K_RoPE RoPE(q^R, p)), the RoPE key
      shared by all branches and heads ("Multi-Head Low-Rank Attention",
      技术新颖性; "ML Revisit: Attention", Multi-Head Latent Attention);
    * o_j = softmax(s_j) V_j; the branch outputs are summed and scaled by
      alpha_kv ("Multi-Head Low-Rank Attention", 核心方法 formula
      O = sum_b Softmax(Q K_b^T) V_b, and 方法步骤详情 for the scales).

    With n = 1 this is MLA. Returns o [B, H, d_v] float64.
    Pinned by: the absorption identity, the separately written MLA, torch's
    float64 scaled-dot-product attention, scalar brute force, RoPE shift
    invariance, branch permutation and the variance statements.
    """
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    B, H, d_n = q_nope.shape
    d_c, d_v = w_uv.shape[1], w_uv.shape[2]
    d_r = q_rope.shape[-1]
    if tau is None:
        tau = 1.0 / math.sqrt(d_n + d_r)
    slices = branch_slices(d_c, n)
    out = np.zeros((B, H, d_v))
    for b in range(B):
        L = int(lens[b])
        if L <= 0:
            continue
        C = _f64(ckv[b, :L])
        KR = _f64(krope[b, :L])
        p = _query_pos(lens, q_pos, b)
        for h in range(H):
            rho = rope(q_rope[b, h], p, theta)
            acc = np.zeros(d_v)
            for S in slices:
                KN = C[:, S] @ w_uk[h][S, :]
                V = C[:, S] @ w_uv[h][S, :]
                s = tau * (alpha_q * (KN @ q_nope[b, h]) + KR @ rho)
                e = np.exp(s - s.max())
                acc += (e / e.sum()) @ V
            out[b, h] = alpha_kv * acc
    return out


def mla_decode_ref(q_nope, q_rope, w_uk, w_uv, ckv, krope, lens,
                   tau=None, alpha_q=1.0, alpha_kv=1.0, theta=10000.0,
                   q_pos=None):
    """Unabsorbed MLA decode written as textbook attention on full keys.

    Builds, per head, the full key K = [alpha_q * C W_UK[h] || K_RoPE] and the
    query [q^N || RoPE(q^R, p)], then softmax(tau K q) (C W_UV[h])
    ("MLA多头潜在注意力机制" 3.2 steps 2-3; "ML Revisit: Attention",
    Multi-Head Latent Attention: the key is the concatenation of the content
    part and the shared RoPE part). Written independently of
    ``mlra_decode_ref`` so that MLRA with one branch can be checked against it.
    """
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    B, H, d_n = q_nope.shape
    d_r = q_rope.shape[-1]
    if tau is None:
        tau = 1.0 / math.sqrt(d_n + d_r)
    out = np.zeros((B, H, w_uv.shape[2]))
    for b in range(B):
        L = int(lens[b])
        if L <= 0:
            continue
        C = _f64(ckv[b, :L])
        KR = _f64(krope[b, :L])
        p = _query_pos(lens, q_pos, b)
        for h in range(H):
            K = np.concatenate([alpha_q * (C @ w_uk[h]), KR], axis=1)
            q = np.concatenate([q_nope[b, h], rope(q_rope[b, h], p, theta)])
            logits = tau * (K @ q)
            w = np.exp(logits - logits.max())
            w /= w.sum()
            out[b, h] = alpha_kv * (w @ (C @ w_uv[h]))
    return out


def absorb_q_ref(q_nope, q_rope, w_uk, q_pos, tau, alpha_q, theta=10000.0):
    """Absorbed query q_abs[b, h] = [alpha_q tau W_UK[h] q^N || tau RoPE(q^R, p)].

    Query-side weight absorption: q^T (c W) = (W q)^T c
    ("Multi-Head Low-Rank Attention", 方法步骤详情 step 1; "ML Revisit:
    Attention", Multi-Head Latent Attention; "vllbc02MLA", 核心思想 and 苏神思路).
    The scales are folded in so that a score is q_abs . [c || k^R].
    ``q_pos`` [B] holds each sequence's query position.
    Returns [B, H, d_c + d_r]. Pinned by the absorption identity.
    """
    q_nope, q_rope, w_uk = _f64(q_nope), _f64(q_rope), _f64(w_uk)
    B, H, _ = q_nope.shape
    d_c = w_uk.shape[1]
    d_r = q_rope.shape[-1]
    out = np.zeros((B, H, d_c + d_r))
    for b in range(B):
        for h in range(H):
            out[b, h, :d_c] = alpha_q * tau * (w_uk[h] @ q_nope[b, h])
            out[b, h, d_c:] = tau * rope(q_rope[b, h], q_pos[b], theta)
    return out


def latent_attn_ref(q_abs, ckv, krope, lens, n):
    """MQA-style decode in latent space, one softmax per branch.

    For branch j: scores s_t = q_abs[S_j] . c_t[S_j] + q_abs[rope] . k^R_t over
    the L_b cached tokens, p = softmax(s), and the branch output
    o~_j = sum_t p_t c_t[S_j] ("Multi-Head Low-Rank Attention", 方法步骤详情
    step 2: C_KV and K_RoPE concatenated into one key shared by all heads, C_KV
    as the value; "vllbc02MLA", 苏神思路: decoding works like MQA).
    Returns latent_out [B, H, d_c] = concat_j o~_j (zeros where L_b = 0).
    Pinned by the absorption identity (through ``out_proj_ref``).
    """
    q_abs = _f64(q_abs)
    B, H, _ = q_abs.shape
    d_c = ckv.shape[-1]
    out = np.zeros((B, H, d_c))
    for b in range(B):
        L = int(lens[b])
        if L <= 0:
            continue
        C = _f64(ckv[b, :L])
        KR = _f64(krope[b, :L])
        rope_scores = q_abs[b, :, d_c:] @ KR.T           # [H, L], shared
        for S in branch_slices(d_c, n):
            s = q_abs[b, :, S] @ C[:, S].T + rope_scores
            e = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, :, S] = (e / e.sum(axis=1, keepdims=True)) @ C[:, S]
    return out


def out_proj_ref(latent_out, w_uv, alpha_kv):
    """o[b, h] = alpha_kv * W_UV[h]^T latent_out[b, h].

    Output up-projection ("Multi-Head Low-Rank Attention", 方法步骤详情 step 3).
    Because latent_out concatenates the branch outputs o~_j over disjoint
    slices, this one contraction is also the branch sum sum_j W_UV[h][S_j]^T o~_j
    (核心方法 formula). Pinned by the absorption identity.
    """
    lo, w_uv = _f64(latent_out), _f64(w_uv)
    B, H, _ = lo.shape
    out = np.zeros((B, H, w_uv.shape[2]))
    for b in range(B):
        for h in range(H):
            out[b, h] = alpha_kv * (w_uv[h].T @ lo[b, h])
    return out


def mlra_prefill_ref(q_nope, q_rope, w_uk, w_uv, ckv, krope, lens, n,
                     tau=None, alpha_q=1.0, alpha_kv=1.0, theta=10000.0):
    """Causal MLRA-n prefill in the unabsorbed (MHA) form.

    The prompt's positions attend causally: position t of sequence b sees the
    cached tokens u <= t ("MLA多头潜在注意力机制" 3.3: a key whose position
    lies after the query's is masked out), and the prefill takes the form with
    explicit up-projected keys and values ("vllbc02MLA", 苏神思路: prefill with
    the MHA form, generation with the MQA form). Per branch j with slice S_j
    ("Multi-Head Low-Rank Attention", 核心方法):

    * K^N_j = C[:, S_j] W_UK[h][S_j], V_j = C[:, S_j] W_UV[h][S_j];
    * S_j[t, u] = tau (alpha_q q^N_t . K^N_j[u] + RoPE(q^R_t, t) . k^R_u), and
      -inf for u > t;
    * o[t] = alpha_kv sum_j softmax_u(S_j[t]) V_j.

    Inputs: q_nope [B, T, H, d_n], q_rope [B, T, H, d_r] (unrotated; row t is
    position t), cache arrays as for the decode with T = L_max. Returns
    [B, T, H, d_v] float64, zero for t >= L_b.
    Pinned by: every row against ``mlra_decode_ref`` on the cache cut after
    that row with the query at its position; torch's float64 causal
    scaled-dot-product attention per branch; the first row's closed form
    (one key: alpha_kv c_0 W_UV[h]); causality (later rows and later queries
    change nothing).
    """
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    B, T, H, d_n = q_nope.shape
    d_c, d_v = w_uv.shape[1], w_uv.shape[2]
    d_r = q_rope.shape[-1]
    if tau is None:
        tau = 1.0 / math.sqrt(d_n + d_r)
    out = np.zeros((B, T, H, d_v))
    for b in range(B):
        L = min(max(int(lens[b]), 0), T)
        if L == 0:
            continue
        C = _f64(ckv[b, :L])
        KR = _f64(krope[b, :L])
        later = np.arange(L)[None, :] > np.arange(L)[:, None]   # [t, u]: u > t
        for h in range(H):
            QN = q_nope[b, :L, h]                               # [L, d_n]
            rho = rope(q_rope[b, :L, h], np.arange(L), theta)   # [L, d_r]
            rope_part = rho @ KR.T
            for S in branch_slices(d_c, n):
                KN = C[:, S] @ w_uk[h][S, :]
                V = C[:, S] @ w_uv[h][S, :]
                s = tau * (alpha_q * (QN @ KN.T) + rope_part)
                s[later] = -np.inf
                e = np.exp(s - s.max(axis=1, keepdims=True))
                out[b, :L, h] += alpha_kv * ((e / e.sum(axis=1, keepdims=True)) @ V)
    return out


def partial_state(scores, values):
    """Softmax state of one token range: (m, l, acc) with m = max s,
    l = sum exp(s - m), acc = sum exp(s - m) v. An empty range gives
    (-inf, 0, 0). Pinned by the split-merge law."""
    scores, values = _f64(scores), _f64(values)
    if scores.size == 0:
        return -np.inf, 0.0, np.zeros(values.shape[-1])
    m = scores.max()
    e = np.exp(scores - m)
    return m, e.sum(), e @ values


def merge_partials(states):
    """Merge token-range softmax states into the full softmax-weighted sum.

    M = max_s m_s; l = sum_s exp(m_s - M) l_s; o = sum_s exp(m_s - M) acc_s / l.
    This is the textbook online-softmax law (not on the pages); it models the
    split combine. All-empty input gives zeros. Pinned by the split-merge test
    (any partition equals the full softmax)."""
    ms = np.array([s[0] for s in states], dtype=np.float64)
    M = ms.max()
    if not np.isfinite(M):
        return np.zeros_like(_f64(states[0][2]))
    l = 0.0
    acc = np.zeros_like(_f64(states[0][2]))
    for m, ls, a in states:
        if np.isfinite(m):
            w = math.exp(m - M)
            l += w * ls
            acc += w * _f64(a)
    return acc / l


def kv_elems_per_token_per_device(d_c, d_r, n, tp):
    """Cache elements one device streams per token under tp-way tensor
    parallelism when the latent is split into n independent groups.

    Each device holds d_c / min(n, tp) latent columns (a single latent cannot
    be split further than its group count) plus the full shared RoPE key.
    Pages: "Multi-Head Low-Rank Attention", 前置知识 (MLA caches 4.5 d_h),
    研究动机 (MLA stays at 4.5 d_h under 4-way TP, GLA-2 reaches 2.5 d_h and no
    lower, MLRA-4 1.5 d_h) and the results table (1.5 d_h vs 4.5 d_h).
    Pinned by those printed numbers (tests/golden/kv_load_per_device.txt).
    """
    if n < 1 or tp < 1 or d_c % n:
        raise ValueError("bad group count")
    return d_c // min(n, tp) + d_r


def variance_scales(d, d_c, n):
    """(alpha_q, alpha_kv) = (sqrt(d / d_c'), sqrt(d / d_c)), d_c' = d_c / n.

    Page: "Multi-Head Low-Rank Attention", 方法步骤详情 (both formulas) and
    技术新颖性 (the correction also applies to MLA). d is the model width.
    Pinned statistically by what the page says they are for: the NoPE score
    term matching the RoPE term's variance, and the summed branch output
    keeping unit variance.
    """
    if d_c % n:
        raise ValueError("d_c must be a multiple of n")
    return math.sqrt(d / (d_c // n)), math.sqrt(d / d_c)


def rms_norm(x, gain=None, eps=1e-6):
    """RMS normalisation of each row: x / sqrt(mean(x^2) + eps), times ``gain``.

    Page: "vllbc02MLA", 猛猿大佬思路 (code walk-through): the compressed KV
    latent passes through an RMSNorm (``kv_a_layernorm`` over kv_lora_rank)
    before it is cached. Pinned by unit RMS of the output, invariance under
    a positive rescaling of the input, and an elementwise gain.
    """
    x = _f64(x)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x / r
    return y if gain is None else y * _f64(gain)


def cache_append_ref(ckv, krope, lens, new_c, new_kr, max_len, gain=None, eps=1e-6,
                     theta=10000.0, round_to=None):
    """Append one token per sequence to the latent cache.

    Pages: "vllbc02MLA", 猛猿大佬思路 (the projected row is split into the
    latent and the RoPE key; the latent is RMS-normalised; the RoPE key is
    rotated by the token's position and comes from the input, not from the
    latent); "从MHA到MLA" 3.2 (the cache is updated by writing the new latent
    at the token's position); "MLA多头潜在注意力机制" 3 (only the latent and
    the decoupled RoPE key are cached).

    Sequence b's new token sits at position p = L_b (0-based), so row p gets
    [RMSNorm(new_c[b]) * gain || RoPE(new_kr[b], p)] and L_b becomes L_b + 1.
    A sequence with L_b >= max_len is left unchanged (no room). ``round_to``
    (a function) rounds the written values to the cache's storage type.
    Returns new (ckv, krope, lens) arrays; the inputs are not modified.
    Pinned by the RMS and rotation properties of the written row, untouched
    rows and full sequences, and decode after append against the decode of
    a cache built with the row in place.
    """
    ckv = _f64(ckv).copy()
    krope = _f64(krope).copy()
    lens = np.asarray(lens, dtype=np.int64).copy()
    new_c, new_kr = _f64(new_c), _f64(new_kr)
    for b in range(len(lens)):
        p = int(lens[b])
        if p >= max_len:
            continue
        c = rms_norm(new_c[b], gain, eps)
        k = rope(new_kr[b], p, theta)
        if round_to is not None:
            c, k = _f64(round_to(c)), _f64(round_to(k))
        ckv[b, p] = c
        krope[b, p] = k
        lens[b] = p + 1
    return ckv, krope, lens.astype(np.int32)



# ---------------------------------------------------------------- fp8 cache --
#
# Quantised latent cache. The pages name INT8 for inference deployment
# ("MLA多头潜在注意力机制", 9.2 部署注意事项) and fix no format or scale. The
# reading taken here: 8-bit floating point E4M3 in the OCP 8-bit floating
# point layout (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
# subnormals, no infinities, exponent and mantissa all ones = NaN; largest
# finite value 448), one float32 scale per cache tensor: a stored latent value
# is c = ckv_scale * e4m3(code), a stored RoPE key value k = krope_scale *
# e4m3(code). Writing a value x stores the code nearest to x / scale, ties to
# the code with an even mantissa, saturating at +-448.


def e4m3_decode(codes):
    """Float64 value of each E4M3 code (uint8 array).

    Normal codes (exponent field e in 1..15): (-1)^s 2^(e - 7) (1 + m / 8);
    subnormals (e = 0): (-1)^s 2^-6 (m / 8); e = 15, m = 7: NaN.
    Pinned by closed-form values, torch's float8_e4m3fn conversion of all 256
    codes and the count of finite codes.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """E4M3 code nearest to each value of x (ties to the even mantissa),
    saturating at +-448; NaN gives 0x7F, the sign of zero is kept.

    Written from the format: in the subnormal range (|x| < 2^-6) the code is
    |x| / 2^-9 rounded; above it x = f 2^k with f in [1, 2), the mantissa is
    (f - 1) 8 rounded, and a mantissa that rounds up to 8 moves to the next
    exponent. Pinned by brute-force search for the nearest of the 254 finite
    values, round trips of every code, torch's conversion inside the finite
    range and the saturation values.
    """
    x = _f64(x)
    # infinities and magnitudes past the range saturate like any |x| > 448
    a = np.abs(np.where(np.isnan(x), 0.0, x))
    a = np.minimum(a, 1024.0)
    out = np.zeros(x.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: integer multiples of 2^-9 (a result of 8 is the
    # smallest normal, code 0x08, which the same formula gives)
    out = np.where(sub, np.rint(a / 2.0 ** -9).astype(np.int64), out)
    f, k = np.frexp(np.where(sub, 1.0, a))  # a = f 2^k, f in [0.5, 1)
    f, k = 2.0 * f, k - 1                  # f in [1, 2)
    m = np.rint((f - 1.0) * 8.0).astype(np.int64)
    k = np.where(m == 8, k + 1, k)
    m = np.where(m == 8, 0, m)
    e = k + 7
    normal = ((e << 3) | m).astype(np.int64)
    normal = np.where((e > 15) | (normal > 0x7E), 0x7E, normal)  # saturate
    out = np.where(sub, out, normal)
    out = np.where(np.signbit(x), out | 0x80, out)
    out = np.where(np.isnan(x), 0x7F, out)
    return out.astype(np.uint8)


def fp8_dequantize(codes, scale):
    """Stored value of an fp8 cache entry: scale * e4m3(code), float64."""
    return float(scale) * e4m3_decode(codes)


def fp8_quantize(x, scale):
    """Codes that an fp8 cache with this scale stores for the values x."""
    return e4m3_encode(_f64(x) / float(scale))
