"""Pins of the float64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: closed-form
rotations, the absorption identity, the block decomposition, a separately
written MLA, scalar brute force, torch's float64 attention routine, the
relative-position property, branch independence, linearity, the online-softmax
merge law, the pages' printed per-device cache loads and the variance
statements of the scales. A plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand) fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (absorb_q_ref, branch_slices, cache_append_ref, kv_elems_per_token_per_device,
                    latent_attn_ref, merge_partials, mla_decode_ref, mlra_decode_ref,
                    mlra_prefill_ref, out_proj_ref, partial_state, rms_norm, rope, variance_scales)
from synth import WORKLOADS, make_inputs, round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(seed=0, B=3, H=4, d_c=64, d_r=16, d_n=32, d_v=24, L=(7, 1, 0), Lmax=None):
    rng = np.random.default_rng(seed)
    Lmax = Lmax or max(max(L), 1)
    return dict(
        q_nope=rng.standard_normal((B, H, d_n)),
        q_rope=rng.standard_normal((B, H, d_r)),
        w_uk=rng.standard_normal((H, d_c, d_n)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_c, d_v)) / math.sqrt(d_c),
        ckv=rng.standard_normal((B, Lmax, d_c)),
        krope=rng.standard_normal((B, Lmax, d_r)),
        lens=np.array(L, dtype=np.int32),
    )


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- RoPE ----

def test_rope_closed_form_unit_vectors():
    # A 2-d rotation by angle a maps e0 -> (cos a, sin a), e1 -> (-sin a, cos a).
    for p in (0.0, 1.0, 2.5, 1234.0):
        np.testing.assert_allclose(rope([1.0, 0.0], p), [math.cos(p), math.sin(p)], atol=1e-15)
        np.testing.assert_allclose(rope([0.0, 1.0], p), [-math.sin(p), math.cos(p)], atol=1e-15)
    # frequency of pair i is theta^(-2i/d): d=4, theta=1e4 -> pair 1 turns at 0.01 rad/pos,
    # and the pairs are consecutive elements (2, 3)
    np.testing.assert_allclose(rope([0, 0, 1.0, 0], 100.0), [0, 0, math.cos(1.0), math.sin(1.0)], atol=1e-15)
    np.testing.assert_allclose(rope([1.0, 0, 0, 0], 100.0), [math.cos(100.0), math.sin(100.0), 0, 0], atol=1e-13)
    # d=8, theta=16: pair 3 turns at 16^(-6/8) = 1/8 rad/pos
    x = np.zeros(8)
    x[7] = 1.0
    np.testing.assert_allclose(rope(x, 8.0, theta=16.0)[6:], [-math.sin(1.0), math.cos(1.0)], atol=1e-15)


def test_rope_properties():
    rng = np.random.default_rng(1)
    x, y = rng.standard_normal(64), rng.standard_normal(64)
    np.testing.assert_allclose(rope(x, 0), x, atol=0)
    for a, b in ((3, 5), (1000, 131071), (100000, 7)):
        np.testing.assert_allclose(np.linalg.norm(rope(x, a)), np.linalg.norm(x), rtol=1e-14)
        np.testing.assert_allclose(rope(rope(x, a), b), rope(x, a + b), atol=1e-9)
        # relative position: <R(a) x, R(b) y> = <R(a - b) x, y>
        np.testing.assert_allclose(rope(x, a) @ rope(y, b), rope(x, a - b) @ y, atol=1e-9)
    # vectorised positions agree with scalar calls
    X = rng.standard_normal((5, 16))
    P = np.array([0, 1, 7, 4095, 131071])
    np.testing.assert_allclose(rope(X, P), np.stack([rope(X[i], P[i]) for i in range(5)]), atol=0)


# --------------------------------------------------- absorption identity ----

@pytest.mark.parametrize("n", [1, 2, 4])
def test_absorbed_equals_unabsorbed(n):
    t = tiny(seed=10 + n, L=(9, 1, 0, 5), B=4)
    tau, aq, akv = 0.21, 1.7, 0.6
    ref = mlra_decode_ref(**t, n=n, tau=tau, alpha_q=aq, alpha_kv=akv)
    pos = np.maximum(t["lens"] - 1, 0)
    qa = absorb_q_ref(t["q_nope"], t["q_rope"], t["w_uk"], pos, tau, aq)
    lo = latent_attn_ref(qa, t["ckv"], t["krope"], t["lens"], n)
    got = out_proj_ref(lo, t["w_uv"], akv)
    assert rel(got, ref) < 1e-12
    assert np.all(got[2] == 0) and np.all(ref[2] == 0)   # L_b = 0 -> zeros


def test_block_decomposition():
    # K^N = C W_UK = sum_b C^(b) W_UK^(b) over contiguous latent blocks
    rng = np.random.default_rng(2)
    C, W = rng.standard_normal((11, 512)), rng.standard_normal((512, 128))
    for n in (1, 2, 4, 8):
        parts = sum(C[:, S] @ W[S, :] for S in branch_slices(512, n))
        assert rel(parts, C @ W) < 1e-12
    assert [(s.start, s.stop) for s in branch_slices(8, 4)] == [(0, 2), (2, 4), (4, 6), (6, 8)]
    with pytest.raises(ValueError):
        branch_slices(10, 4)


@pytest.mark.parametrize("alphas", [(1.0, 1.0), (math.sqrt(14.0), math.sqrt(14.0))])
def test_mlra_one_branch_is_mla(alphas):
    t = tiny(seed=3, L=(6, 3, 1))
    a = mlra_decode_ref(**t, n=1, alpha_q=alphas[0], alpha_kv=alphas[1])
    b = mla_decode_ref(**t, alpha_q=alphas[0], alpha_kv=alphas[1])
    assert rel(a, b) < 1e-12


def test_softmax_trivial_special_cases():
    # (i) W_UK = 0: every branch sees the same RoPE-only scores, so one shared
    # softmax; sum_j P V_j = P sum_j V_j = MLA.  (ii) L_b = 1: P = 1 everywhere.
    t = tiny(seed=4, L=(5, 2, 8))
    t0 = dict(t, w_uk=np.zeros_like(t["w_uk"]))
    for n in (2, 4):
        assert rel(mlra_decode_ref(**t0, n=n), mla_decode_ref(**t0)) < 1e-12
    t1 = dict(t, lens=np.array([1, 1, 1], np.int32))
    for n in (2, 4):
        assert rel(mlra_decode_ref(**t1, n=n, alpha_q=2.0), mla_decode_ref(**t1, alpha_q=2.0)) < 1e-12
    # and for L > 1 with real keys MLRA differs from MLA (softmax is nonlinear)
    assert rel(mlra_decode_ref(**t, n=4), mla_decode_ref(**t)) > 1e-3


# ----------------------------------------------------------- brute force ----

def _brute(t, n, tau, aq, akv, theta=10000.0):
    q_nope, q_rope, w_uk, w_uv = t["q_nope"], t["q_rope"], t["w_uk"], t["w_uv"]
    ckv, krope, lens = t["ckv"], t["krope"], t["lens"]
    B, H, d_n = q_nope.shape
    d_c, d_v, d_r = w_uv.shape[1], w_uv.shape[2], q_rope.shape[2]
    w = d_c // n
    out = np.zeros((B, H, d_v))
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        p = L - 1
        for h in range(H):
            rho = [0.0] * d_r
            for i in range(d_r // 2):
                a = p * theta ** (-2.0 * i / d_r)
                x0, x1 = q_rope[b, h, 2 * i], q_rope[b, h, 2 * i + 1]
                rho[2 * i] = x0 * math.cos(a) - x1 * math.sin(a)
                rho[2 * i + 1] = x0 * math.sin(a) + x1 * math.cos(a)
            o = [0.0] * d_v
            for j in range(n):
                cols = range(j * w, (j + 1) * w)
                s = []
                for tt in range(L):
                    kn = [math.fsum(ckv[b, tt, c] * w_uk[h, c, e] for c in cols) for e in range(d_n)]
                    nope = math.fsum(kn[e] * q_nope[b, h, e] for e in range(d_n))
                    rp = math.fsum(krope[b, tt, r] * rho[r] for r in range(d_r))
                    s.append(tau * (aq * nope + rp))
                m = max(s)
                e_ = [math.exp(x - m) for x in s]
                Z = math.fsum(e_)
                for k in range(d_v):
                    v = [math.fsum(ckv[b, tt, c] * w_uv[h, c, k] for c in cols) for tt in range(L)]
                    o[k] += math.fsum(e_[tt] / Z * v[tt] for tt in range(L))
            out[b, h] = [akv * x for x in o]
    return out


@pytest.mark.parametrize("n", [1, 2])
def test_brute_force_scalar_loops(n):
    t = tiny(seed=5, B=2, H=2, d_c=8, d_r=4, d_n=3, d_v=2, L=(6, 1))
    tau, aq, akv = 0.4, 1.3, 0.7
    assert rel(mlra_decode_ref(**t, n=n, tau=tau, alpha_q=aq, alpha_kv=akv),
               _brute(t, n, tau, aq, akv)) < 1e-13


@pytest.mark.parametrize("n", [1, 4])
def test_against_torch_sdpa(n):
    # Unabsorbed attention is textbook scaled-dot-product attention on the
    # explicit per-branch keys [alpha_q C_j W_UK_j || K_R] and values C_j W_UV_j.
    t = tiny(seed=6, B=2, H=3, L=(13, 4))
    tau, aq, akv = 0.17, 2.0, 0.8
    ref = mlra_decode_ref(**t, n=n, tau=tau, alpha_q=aq, alpha_kv=akv)
    d_c = t["w_uk"].shape[1]
    for b in range(2):
        L = int(t["lens"][b])
        C, KR = torch.from_numpy(t["ckv"][b, :L]), torch.from_numpy(t["krope"][b, :L])
        for h in range(3):
            q_r = torch.from_numpy(rope(t["q_rope"][b, h], L - 1))
            o = torch.zeros(t["w_uv"].shape[2], dtype=torch.float64)
            for S in branch_slices(d_c, n):
                K = torch.cat([aq * C[:, S] @ torch.from_numpy(t["w_uk"][h][S]), KR], 1)
                V = C[:, S] @ torch.from_numpy(t["w_uv"][h][S])
                q = torch.cat([torch.from_numpy(t["q_nope"][b, h]), q_r])
                o += torch.nn.functional.scaled_dot_product_attention(
                    q[None, None, None], K[None, None], V[None, None], scale=tau)[0, 0, 0]
            assert rel(ref[b, h], akv * o.numpy()) < 1e-12


# ------------------------------------------------------------ invariants ----

@pytest.mark.parametrize("delta", [1, 1000, 100000])
def test_rope_shift_invariance(delta):
    # Shift every cached key and the query by the same delta: scores depend
    # only on relative position, so the output is unchanged.
    t = tiny(seed=7, L=(12, 5, 1))
    B, Lmax = t["ckv"].shape[:2]
    for n in (1, 4):
        base = mlra_decode_ref(**t, n=n, alpha_q=1.5)
        kr = rope(t["krope"], np.full((B, Lmax), float(delta)))
        shifted = mlra_decode_ref(**dict(t, krope=kr), n=n, alpha_q=1.5,
                                  q_pos=t["lens"] - 1 + delta)
        assert rel(shifted, base) < 1e-9


def test_branch_permutation_invariance():
    t = tiny(seed=8, d_c=64, L=(10, 3, 7))
    perm = [2, 0, 3, 1]
    w = 16
    idx = np.concatenate([np.arange(j * w, (j + 1) * w) for j in perm])
    tp = dict(t, ckv=t["ckv"][..., idx], w_uk=t["w_uk"][:, idx], w_uv=t["w_uv"][:, idx])
    assert rel(mlra_decode_ref(**tp, n=4, alpha_q=1.2), mlra_decode_ref(**t, n=4, alpha_q=1.2)) < 1e-12


def test_linearity_and_rope_only():
    t = tiny(seed=9, L=(8, 2, 5))
    for n in (1, 4):
        one = mlra_decode_ref(**t, n=n, alpha_kv=1.0)
        assert rel(mlra_decode_ref(**t, n=n, alpha_kv=3.5), 3.5 * one) < 1e-14
        # alpha_q = 0 leaves attention on the shared RoPE key only: one softmax
        # over tau K_R rho for every branch, applied to sum_j V_j = C W_UV.
        got = mlra_decode_ref(**t, n=n, alpha_q=0.0, tau=0.3)
        for b in range(3):
            L = int(t["lens"][b])
            KR = torch.from_numpy(t["krope"][b, :L])
            for h in range(4):
                q = torch.from_numpy(rope(t["q_rope"][b, h], L - 1))
                V = torch.from_numpy(t["ckv"][b, :L] @ t["w_uv"][h])
                o = torch.nn.functional.scaled_dot_product_attention(
                    q[None, None, None], KR[None, None], V[None, None], scale=0.3)[0, 0, 0]
                assert rel(got[b, h], o.numpy()) < 1e-12


def test_split_merge_law():
    rng = np.random.default_rng(11)
    s = rng.standard_normal(200) * 4
    v = rng.standard_normal((200, 7))
    e = np.exp(s - s.max())
    full = (e / e.sum()) @ v
    for cuts in ([0, 200], [0, 1, 200], [0, 50, 50, 120, 199, 200], list(range(0, 201, 20))):
        states = [partial_state(s[a:b], v[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
        assert rel(merge_partials(states), full) < 1e-13
    # all ranges empty -> zeros
    assert np.all(merge_partials([partial_state(s[:0], v[:0])] * 3) == 0)


def test_empty_and_single_token():
    t = tiny(seed=12, L=(0, 1, 0))
    o = mlra_decode_ref(**t, n=2)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    # one token: softmax weight 1, output = alpha_kv * W_UV^T c_0 (summed over branches)
    np.testing.assert_allclose(o[1], np.einsum("hcv,c->hv", t["w_uv"], t["ckv"][1, 0]), rtol=1e-12)


# -------------------------------------------------- the pages' own numbers ----

def test_kv_load_per_device_golden():
    d_h = 128
    rows = []
    with open(os.path.join(GOLDEN, "kv_load_per_device.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, groups, tp, load = line.split()
                rows.append((name, int(groups), int(tp), float(load)))
    assert len(rows) == 5
    for name, groups, tp, load in rows:
        assert kv_elems_per_token_per_device(4 * d_h, d_h // 2, groups, tp) == load * d_h, name
    # the table's "-67%" reduction
    assert abs(1 - 1.5 / 4.5 - 0.67) < 0.005


def test_variance_scales_do_what_the_page_says():
    # Under the page's assumption (weights i.i.d., independent of the inputs,
    # here N(0, 1/d) with unit-variance latents), alpha_q brings the NoPE key
    # of one branch to the unit variance of the RoPE key, and alpha_kv brings
    # the summed branch output back to unit variance.
    d, d_c, n = 1024, 256, 4
    aq, akv = variance_scales(d, d_c, n)
    assert (aq, akv) == (math.sqrt(d / 64), math.sqrt(d / 256))
    rng = np.random.default_rng(13)
    C = rng.standard_normal((4000, d_c))
    W = rng.standard_normal((d_c, 64)) / math.sqrt(d)
    kn = aq * (C[:, branch_slices(d_c, n)[1]] @ W[branch_slices(d_c, n)[1]])
    assert abs(kn.var() - 1.0) < 0.08
    # summed output with one cached token (softmax weight 1): var ~ 1
    B, H = 400, 8
    t = dict(q_nope=rng.standard_normal((B, H, 16)), q_rope=rng.standard_normal((B, H, 8)),
             w_uk=rng.standard_normal((H, d_c, 16)) / math.sqrt(d),
             w_uv=rng.standard_normal((H, d_c, 16)) / math.sqrt(d),
             ckv=rng.standard_normal((B, 1, d_c)), krope=rng.standard_normal((B, 1, 8)),
             lens=np.ones(B, np.int32))
    o = mlra_decode_ref(**t, n=n, alpha_q=aq, alpha_kv=akv)
    assert abs(o.var() - 1.0) < 0.08
    # the MLRA-4 values at the DeepSeek-V3 width d = 7168, d_c = 512
    aq4, akv4 = variance_scales(7168, 512, 4)
    assert abs(aq4 - math.sqrt(56)) < 1e-12 and abs(akv4 - math.sqrt(14)) < 1e-12


# ------------------------------------------------------- cache append ----

def test_rms_norm_closed_form_and_torch():
    # worked example: [3, 4] has mean square 12.5
    y = rms_norm(np.array([3.0, 4.0]), eps=0.0)
    assert np.allclose(y, np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=0, atol=1e-15)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 512)) * 3.0
    g = rng.standard_normal(512)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), torch.from_numpy(g), 1e-6)
    assert np.allclose(rms_norm(x, g, 1e-6), ref.numpy(), rtol=1e-12, atol=1e-12)
    # unit RMS without gain, and no change under a positive rescaling (eps = 0)
    y = rms_norm(x, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-12)
    assert np.allclose(rms_norm(7.5 * x, eps=0.0), y, atol=1e-12)


def test_cache_append_writes_one_row_and_counts():
    rng = np.random.default_rng(4)
    B, Lmax, d_c, d_r = 4, 6, 32, 8
    ckv = rng.standard_normal((B, Lmax, d_c))
    kr = rng.standard_normal((B, Lmax, d_r))
    lens = np.array([0, 3, 6, 5], np.int32)  # sequence 2 is full
    new_c = rng.standard_normal((B, d_c)) * 5.0
    new_k = rng.standard_normal((B, d_r))
    c2, k2, l2 = cache_append_ref(ckv, kr, lens, new_c, new_k, Lmax)
    assert l2.tolist() == [1, 4, 6, 6]
    for b in range(B):
        p = int(lens[b])
        for t in range(Lmax):
            if t == p and p < Lmax:
                continue
            assert np.array_equal(c2[b, t], ckv[b, t]) and np.array_equal(k2[b, t], kr[b, t])
    # inputs are not modified
    assert lens.tolist() == [0, 3, 6, 5]
    for b, p in ((0, 0), (1, 3), (3, 5)):
        # the latent row has unit RMS (eps is negligible here)
        assert abs(math.sqrt(np.mean(c2[b, p] ** 2)) - 1.0) < 1e-6
        assert np.allclose(c2[b, p] * np.sqrt(np.mean(new_c[b] ** 2)), new_c[b], rtol=1e-6)
        # the key is turned by exactly p: a query rotated to p sees the
        # unrotated dot product, and each pair keeps its length
        q = rng.standard_normal(d_r)
        assert math.isclose(float(rope(q, p) @ k2[b, p]), float(q @ new_k[b]), rel_tol=1e-12,
                            abs_tol=1e-12)
        pair = lambda v: np.hypot(v[0::2], v[1::2])  # noqa: E731
        assert np.allclose(pair(k2[b, p]), pair(new_k[b]))
    # position 0 is the identity rotation
    assert np.allclose(k2[0, 0], new_k[0])


def test_append_then_decode_sees_the_new_token():
    # the next decode step's query sits at the new token (p = L_b after the
    # append): its output changes only through that row, and equals the
    # decode of the cache with the row in place
    rng = np.random.default_rng(6)
    B, H, d_c, d_r, d_n, d_v, Lmax = 2, 3, 32, 8, 16, 16, 9
    ckv = rng.standard_normal((B, Lmax, d_c))
    kr = rng.standard_normal((B, Lmax, d_r))
    lens = np.array([4, 8], np.int32)
    qn, qr = rng.standard_normal((B, H, d_n)), rng.standard_normal((B, H, d_r))
    wk, wv = rng.standard_normal((H, d_c, d_n)) / 6, rng.standard_normal((H, d_c, d_v)) / 6
    c2, k2, l2 = cache_append_ref(ckv, kr, lens, rng.standard_normal((B, d_c)),
                                  rng.standard_normal((B, d_r)), Lmax)
    got = mlra_decode_ref(qn, qr, wk, wv, c2, k2, l2, 1)
    # the same tokens placed by hand (rows past the old lengths are ignored)
    ckv_h, kr_h = ckv.copy(), kr.copy()
    for b in range(B):
        ckv_h[b, lens[b]] = c2[b, lens[b]]
        kr_h[b, lens[b]] = k2[b, lens[b]]
    assert np.allclose(got, mlra_decode_ref(qn, qr, wk, wv, ckv_h, kr_h, lens + 1, 1))
    assert not np.allclose(got, mlra_decode_ref(qn, qr, wk, wv, ckv, kr, lens + 1, 1))


# ------------------------------------------------------------- prefill ----

def prefill_tiny(seed, B=2, H=3, d_c=64, d_r=16, d_n=32, d_v=24, L=(9, 5), T=11):
    rng = np.random.default_rng(seed)
    return dict(
        q_nope=rng.standard_normal((B, T, H, d_n)),
        q_rope=rng.standard_normal((B, T, H, d_r)),
        w_uk=rng.standard_normal((H, d_c, d_n)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_c, d_v)) / math.sqrt(d_c),
        ckv=rng.standard_normal((B, T, d_c)),
        krope=rng.standard_normal((B, T, d_r)),
        lens=np.array(L, dtype=np.int32),
    )


@pytest.mark.parametrize("n", [1, 2, 4])
def test_prefill_rows_are_decode_steps(n):
    # row t of the prefill is the decode of a cache holding tokens 0..t with
    # the query of position t (a separately written loop over one query)
    t = prefill_tiny(20 + n)
    kw = dict(n=n, tau=0.21, alpha_q=1.7, alpha_kv=0.6, theta=500.0)
    got = mlra_prefill_ref(**t, **kw)
    B, T = t["q_nope"].shape[:2]
    for b in range(B):
        for r in range(T):
            if r >= t["lens"][b]:
                assert not np.any(got[b, r])
                continue
            want = mlra_decode_ref(t["q_nope"][b:b + 1, r], t["q_rope"][b:b + 1, r], t["w_uk"],
                                   t["w_uv"], t["ckv"][b:b + 1], t["krope"][b:b + 1],
                                   np.array([r + 1]), q_pos=np.array([r]), **kw)
            assert rel(got[b, r], want[0]) < 1e-12, (b, r)


@pytest.mark.parametrize("n", [1, 4])
def test_prefill_against_torch_causal_sdpa(n):
    # per branch, torch's float64 causal attention on the explicit keys
    # [alpha_q C_j W_UK_j || K_R], queries [q^N || RoPE(q^R, t)], values C_j W_UV_j
    t = prefill_tiny(30, L=(11, 6))
    tau, aq, akv = 0.19, 1.3, 0.9
    ref = mlra_prefill_ref(**t, n=n, tau=tau, alpha_q=aq, alpha_kv=akv)
    d_c = t["w_uk"].shape[1]
    for b in range(2):
        L = int(t["lens"][b])
        C, KR = torch.from_numpy(t["ckv"][b, :L]), torch.from_numpy(t["krope"][b, :L])
        for h in range(3):
            q_r = torch.from_numpy(np.stack([rope(t["q_rope"][b, r, h], r) for r in range(L)]))
            q = torch.cat([torch.from_numpy(t["q_nope"][b, :L, h]), q_r], 1)
            o = torch.zeros(L, t["w_uv"].shape[2], dtype=torch.float64)
            for S in branch_slices(d_c, n):
                K = torch.cat([aq * C[:, S] @ torch.from_numpy(t["w_uk"][h][S]), KR], 1)
                V = C[:, S] @ torch.from_numpy(t["w_uv"][h][S])
                o += torch.nn.functional.scaled_dot_product_attention(
                    q[None], K[None], V[None], is_causal=True, scale=tau)[0]
            assert rel(ref[b, :L, h], akv * o.numpy()) < 1e-12


def test_prefill_first_row_and_causality():
    t = prefill_tiny(40, L=(10, 10), T=10)
    kw = dict(n=4, tau=0.3, alpha_q=1.1, alpha_kv=0.7)
    ref = mlra_prefill_ref(**t, **kw)
    # position 0 sees one key: weight 1 in every branch, so the branch sum is
    # alpha_kv c_0 W_UV[h] whatever the query
    for b in range(2):
        for h in range(3):
            assert rel(ref[b, 0, h], 0.7 * t["ckv"][b, 0] @ t["w_uv"][h]) < 1e-13
    # later cache rows and later queries leave rows 0..4 unchanged; row 5 moves
    u = {k: v.copy() for k, v in t.items()}
    rng = np.random.default_rng(41)
    for k in ("ckv", "krope", "q_nope", "q_rope"):
        u[k][:, 5:] = rng.standard_normal(u[k][:, 5:].shape)
    ref2 = mlra_prefill_ref(**u, **kw)
    np.testing.assert_array_equal(ref2[:, :5], ref[:, :5])
    assert rel(ref2[:, 5], ref[:, 5]) > 1e-3
    # shorter lengths cut the output, not the rows before the cut
    u = dict(t, lens=np.array([4, 0], np.int32))
    ref3 = mlra_prefill_ref(**u, **kw)
    assert rel(ref3[0, :4], ref[0, :4]) < 1e-13   # equal up to the matmul's summation order
    assert not np.any(ref3[0, 4:]) and not np.any(ref3[1])


# -------------------------------------------------------- input recipe ----

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)


def test_workload_recipe_shapes():
    w = WORKLOADS["tiny_mla_fp32"]
    a = make_inputs(w)
    b = make_inputs(w)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert a["ckv"].shape == (1, 256, 64) and a["w_uk"].shape == (4, 64, 32)
    s = WORKLOADS["shard_b64_ragged"]
    lens = make_inputs(s, parts=())["lens"]
    assert lens.shape == (64,) and lens.min() >= 1024 and lens.max() <= 65536
    m = make_inputs(WORKLOADS["mla_b16_l4k"].replace(batch=2, cache_len=64))
    rms = np.sqrt(np.mean(np.square(m["ckv"].astype(np.float64)), -1))
    assert np.all(np.abs(rms - 1) < 0.01)
    assert np.array_equal(round_bf16(m["ckv"]), m["ckv"])
