"""The oracle's pins catch plausible slips.

Each case plants one mistake in a copy of the oracle's source (a wrong sign,
frequency, index, slice, scale, axis or mask), loads that copy as a separate
module and runs it against references that do not use the oracle: the scalar
brute force of the pins, a direct softmax for the split-merge law, that brute
force row by row for the prefill, and the appended row written out element by
element. Every planted mistake must move at least one of them far outside
rounding, while the unchanged source agrees with all of them to 1e-12. Only
CPU work; nothing here touches the real oracle module.
"""

import math
import os
import types

import numpy as np
import pytest

from tests.test_oracle_fp8 import _samples, brute_encode, torch_values
from tests.test_oracle_pins import _brute, rel, tiny

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "mlra_ref.py")

TAU, AQ, AKV = 0.4, 1.3, 0.7

# (name, text in the oracle's source, planted replacement)
MUTATIONS = [
    ("rope rotates the wrong way",
     "    out[..., 0::2] = x0 * cos - x1 * sin\n", "    out[..., 0::2] = x0 * cos + x1 * sin\n"),
    ("rope frequency exponent halved",
     "    omega = theta ** (-2.0 * i / d_r)\n", "    omega = theta ** (-1.0 * i / d_r)\n"),
    ("query one position late",
     "    return int(lens[b]) - 1 if q_pos is None else int(q_pos[b])",
     "    return int(lens[b]) if q_pos is None else int(q_pos[b])"),
    ("branches take strided columns",
     "    return [slice(j * w, (j + 1) * w) for j in range(n)]",
     "    return [slice(j, d_c, n) for j in range(n)]"),
    ("alpha_q also scales the RoPE term",
     "                s = tau * (alpha_q * (KN @ q_nope[b, h]) + KR @ rho)",
     "                s = tau * alpha_q * (KN @ q_nope[b, h] + KR @ rho)"),
    ("alpha_kv dropped in the decode",
     "            out[b, h] = alpha_kv * acc", "            out[b, h] = acc"),
    ("branches averaged instead of summed",
     "                acc += (e / e.sum()) @ V\n", "                acc += (e / e.sum()) @ V / len(slices)\n"),
    ("keys of the neighbouring head",
     "                KN = C[:, S] @ w_uk[h][S, :]\n                V = C[:, S] @ w_uv[h][S, :]\n"
     "                s = tau * (alpha_q * (KN @ q_nope[b, h])",
     "                KN = C[:, S] @ w_uk[(h + 1) % H][S, :]\n                V = C[:, S] @ w_uv[h][S, :]\n"
     "                s = tau * (alpha_q * (KN @ q_nope[b, h])"),
    ("absorbed query without alpha_q",
     "            out[b, h, :d_c] = alpha_q * tau * (w_uk[h] @ q_nope[b, h])",
     "            out[b, h, :d_c] = tau * (w_uk[h] @ q_nope[b, h])"),
    ("absorbed RoPE part without tau",
     "            out[b, h, d_c:] = tau * rope(", "            out[b, h, d_c:] = rope("),
    ("latent softmax normalised over heads",
     "            out[b, :, S] = (e / e.sum(axis=1, keepdims=True)) @ C[:, S]",
     "            out[b, :, S] = (e / e.sum(axis=0, keepdims=True)) @ C[:, S]"),
    ("latent scores miss the shared RoPE term",
     "            s = q_abs[b, :, S] @ C[:, S].T + rope_scores",
     "            s = q_abs[b, :, S] @ C[:, S].T"),
    ("output projection without alpha_kv",
     "            out[b, h] = alpha_kv * (w_uv[h].T @ lo[b, h])",
     "            out[b, h] = (w_uv[h].T @ lo[b, h])"),
    ("merge weights with the exponent reversed",
     "            w = math.exp(m - M)", "            w = math.exp(M - m)"),
    ("causal mask hides the query's own token",
     "        later = np.arange(L)[None, :] > np.arange(L)[:, None]",
     "        later = np.arange(L)[None, :] >= np.arange(L)[:, None]"),
    ("prefill query rotated one position late",
     "            rho = rope(q_rope[b, :L, h], np.arange(L), theta)",
     "            rho = rope(q_rope[b, :L, h], np.arange(L) + 1, theta)"),
    ("RMS over the sum instead of the mean",
     "    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
     "    r = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)"),
    ("appended key rotated at the previous position",
     "        k = rope(new_kr[b], p, theta)", "        k = rope(new_kr[b], p - 1, theta)"),
    ("appended row written one row early",
     "        ckv[b, p] = c\n        krope[b, p] = k", "        ckv[b, p - 1] = c\n        krope[b, p - 1] = k"),
    ("prefill without alpha_kv",
     "                out[b, :L, h] += alpha_kv * ((e / e.sum(axis=1, keepdims=True)) @ V)",
     "                out[b, :L, h] += ((e / e.sum(axis=1, keepdims=True)) @ V)"),
    ("e4m3 exponent bias 8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("e4m3 subnormals one binade low",
     "mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6,", "mag = np.where(e == 0, (m / 8.0) * 2.0 ** -7,"),
    ("e4m3 encoder rounds ties away from zero",
     "    m = np.rint((f - 1.0) * 8.0).astype(np.int64)",
     "    m = np.floor((f - 1.0) * 8.0 + 0.5).astype(np.int64)"),
    ("e4m3 encoder overflows to NaN instead of saturating",
     "    normal = np.where((e > 15) | (normal > 0x7E), 0x7E, normal)  # saturate",
     "    normal = np.where((e > 15) | (normal > 0x7E), 0x7F, normal)"),
    ("e4m3 subnormal step 2^-10", "np.rint(a / 2.0 ** -9)", "np.rint(a / 2.0 ** -10)"),
    ("e4m3 mantissa carry kept in the exponent",
     "    k = np.where(m == 8, k + 1, k)\n", "    k = k\n"),
]

# fp8 codec inputs: sampled values, every midpoint, saturating values
FP8_X = _samples(7, 300)
FP8_WANT = brute_encode(FP8_X)


def load(source):
    mod = types.ModuleType("oracle_copy")
    exec(compile(source, "oracle_copy", "exec"), mod.__dict__)
    return mod


def check_errors(m):
    """Relative error of each oracle path of module m against a reference
    that does not use the oracle (nan counts as a failure)."""
    errs = {}
    t = tiny(seed=5, B=2, H=3, d_c=8, d_r=4, d_n=3, d_v=2, L=(6, 1))
    for n in (1, 2):
        ref = _brute(t, n, TAU, AQ, AKV)
        errs[f"decode n={n}"] = rel(m.mlra_decode_ref(**t, n=n, tau=TAU, alpha_q=AQ, alpha_kv=AKV), ref)
        q = m.absorb_q_ref(t["q_nope"], t["q_rope"], t["w_uk"], t["lens"] - 1, TAU, AQ)
        lo = m.latent_attn_ref(q, t["ckv"], t["krope"], t["lens"], n)
        errs[f"absorbed n={n}"] = rel(m.out_proj_ref(lo, t["w_uv"], AKV), ref)
    # split-merge law against one direct softmax
    rng = np.random.default_rng(3)
    s, v = rng.standard_normal(11) * 3.0, rng.standard_normal((11, 4))
    e = np.exp(s - s.max())
    direct = (e / e.sum()) @ v
    parts = [m.partial_state(s[a:b], v[a:b]) for a, b in ((0, 4), (4, 4), (4, 11))]
    errs["merge"] = rel(m.merge_partials(parts), direct)
    # prefill rows against the brute-force decode of the cut cache
    T = 5
    rng = np.random.default_rng(9)
    H, d_c, d_r, d_n, d_v = 2, 8, 4, 3, 2
    P = dict(q_nope=rng.standard_normal((1, T, H, d_n)), q_rope=rng.standard_normal((1, T, H, d_r)),
             w_uk=rng.standard_normal((H, d_c, d_n)) / math.sqrt(d_c),
             w_uv=rng.standard_normal((H, d_c, d_v)) / math.sqrt(d_c),
             ckv=rng.standard_normal((1, T, d_c)), krope=rng.standard_normal((1, T, d_r)))
    got = m.mlra_prefill_ref(**P, lens=np.array([T], np.int32), n=2, tau=TAU, alpha_q=AQ, alpha_kv=AKV)
    worst = 0.0
    for tq in range(T):
        row = dict(q_nope=P["q_nope"][:, tq], q_rope=P["q_rope"][:, tq], w_uk=P["w_uk"], w_uv=P["w_uv"],
                   ckv=P["ckv"], krope=P["krope"], lens=np.array([tq + 1], np.int32))
        worst = max(worst, rel(got[0, tq], _brute(row, 2, TAU, AQ, AKV)[0]))
    errs["prefill"] = worst
    # cache append against the row written out directly: RMS-normalised latent
    # times the gain, key turned pair by pair by p theta^(-2i/d_r), p = L_b
    rng = np.random.default_rng(13)
    B, Lmax, d_c, d_r, eps = 3, 4, 6, 4, 1e-6
    ckv, krope = rng.standard_normal((B, Lmax, d_c)), rng.standard_normal((B, Lmax, d_r))
    lens = np.array([0, 2, Lmax], np.int32)
    nc, nk, gain = rng.standard_normal((B, d_c)), rng.standard_normal((B, d_r)), rng.standard_normal(d_c)
    c2, k2, l2 = m.cache_append_ref(ckv, krope, lens, nc, nk, Lmax, gain=gain, eps=eps)
    want_c, want_k = ckv.copy(), krope.copy()
    for b in range(B):
        p = int(lens[b])
        if p >= Lmax:
            continue
        want_c[b, p] = nc[b] / math.sqrt(sum(x * x for x in nc[b]) / d_c + eps) * gain
        for i in range(d_r // 2):
            a = p * 10000.0 ** (-2.0 * i / d_r)
            x0, x1 = nk[b, 2 * i], nk[b, 2 * i + 1]
            want_k[b, p, 2 * i] = x0 * math.cos(a) - x1 * math.sin(a)
            want_k[b, p, 2 * i + 1] = x0 * math.sin(a) + x1 * math.cos(a)
    errs["append"] = max(rel(c2, want_c), rel(k2, want_k),
                         0.0 if l2.tolist() == [1, 3, Lmax] else np.inf)
    # fp8 codec: every code's value against torch's float8_e4m3fn, the
    # encoder against the brute-force nearest-value search
    want = torch_values()
    got = m.e4m3_decode(np.arange(256, dtype=np.uint8))
    ok = ~np.isnan(want)
    errs["e4m3 decode"] = (rel(got[ok], want[ok])
                           if np.array_equal(np.isnan(got), np.isnan(want)) else np.inf)
    errs["e4m3 encode"] = float(np.count_nonzero(m.e4m3_encode(FP8_X) != FP8_WANT))
    return {k: (v if np.isfinite(v) else np.inf) for k, v in errs.items()}


def test_unchanged_oracle_agrees_with_every_reference():
    errs = check_errors(load(open(SRC).read()))
    assert max(errs.values()) < 1e-12, errs


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: the text to mutate must occur exactly once"
    with np.errstate(all="ignore"):
        errs = check_errors(load(src.replace(old, new)))
    caught = {k: v for k, v in errs.items() if v > 1e-6}
    assert caught, f"{name}: no reference noticed ({errs})"
