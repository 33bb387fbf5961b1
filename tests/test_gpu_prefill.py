"""GPU parity of the causal prefill (mlra_prefill) against the float64 oracle.

Small ragged prompts are compared on every row against the unabsorbed causal
oracle; the full 4 x 4096 prompt is compared on sampled rows, each against
the oracle's decode of the cache cut after that row (the prefill's row t is
that decode, as the oracle pins show). Rows at or past a sequence's length
must be exactly zero. Tolerance: the decode path's bf16 bound, 1e-2 in
row-relative L2 (the absorbed queries and the softmax weights are rounded to
bf16 before their products).
"""

import numpy as np
import pytest
import torch

import branch_rank_amd as br
import oracle
from synth import WORKLOADS, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def run_prefill(w, inp, d=None, out_dtype=torch.float32):
    d = Dev(w, inp) if d is None else d
    cfg = config_for(w)
    B, T = d.B, d.Lmax
    out = torch.empty(B, T, w.heads, w.d_v, dtype=out_dtype, device="cuda")
    br.mlra_prefill(cfg, w.n, d.q_nope, d.q_rope, d.w_uk, d.w_uv, d.cache(cfg), out)
    torch.cuda.synchronize()
    return out, d


def oracle_prefill(w, inp):
    return oracle.mlra_prefill_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"],
                                   inp["ckv"], inp["krope"], inp["lens"], w.n, tau=w.tau,
                                   alpha_q=w.alpha_q, alpha_kv=w.alpha_kv, theta=w.theta)


def check_rows(got, ref, lens):
    worst = 0.0
    for b, L in enumerate(lens):
        L = int(min(max(L, 0), got.shape[1]))
        assert not np.any(got[b, L:]), f"sequence {b}: rows past {L} not zero"
        if L:
            worst = max(worst, row_rel_err(got[b, :L], ref[b, :L]))
    return worst


@pytest.mark.parametrize("lens,T", [([300, 1, 129, 0], 300), ([128, 127, 33], 160)])
def test_prefill_all_rows_small(lens, T):
    # several 64-position blocks, ragged last blocks and tiles, a one-token
    # prompt and an empty one
    w = WORKLOADS["mlra4_prefill_b4_t4k"].replace(batch=len(lens), heads=8)
    inp = make_inputs(w, lens=np.array(lens, np.int32), max_len=T, q_rows=T)
    say(f"prefill lens {lens} T={T}")
    got, _ = run_prefill(w, inp)
    err = check_rows(host(got), oracle_prefill(w, inp), lens)
    say(f"  worst row rel err {err:.2e}")
    assert err <= TOL


def test_prefill_bf16_output_and_clamped_lengths():
    w = WORKLOADS["mlra4_prefill_b4_t4k"].replace(batch=3, heads=4)
    T = 96
    inp = make_inputs(w, lens=np.array([96, 40, 0], np.int32), max_len=T, q_rows=T)
    want, d = run_prefill(w, inp)
    got16, _ = run_prefill(w, inp, d=d, out_dtype=torch.bfloat16)
    assert torch.equal(got16, want.to(torch.bfloat16))
    # lengths outside [0, T] act as their clamped values, bit for bit
    d.lens.copy_(torch.tensor([96 + 7, 40, -5], dtype=torch.int32))
    got, _ = run_prefill(w, inp, d=d)
    assert torch.equal(got, want)
    assert check_rows(host(want), oracle_prefill(w, inp), [96, 40, 0]) <= TOL


@pytest.mark.slow
def test_prefill_full_size_sampled_rows():
    # 4 prompts of 4096 tokens, 128 heads: rows sampled at block and tile
    # edges and at random, each against the oracle's decode of the cut cache
    w = WORKLOADS["mlra4_prefill_b4_t4k"]
    T = w.cache_len
    lens = np.array([T, T - 1, 2049, 1], np.int32)
    inp = make_inputs(w, lens=lens, q_rows=T)
    say(f"prefill B={w.batch} T={T} H={w.heads}")
    got, _ = run_prefill(w, inp)
    got = host(got)
    rng = np.random.default_rng(5)
    picks = [(0, 0), (0, 31), (0, 127), (0, 128), (0, T - 1), (1, T - 2), (2, 2048), (2, 1000),
             (3, 0)] + [(int(b), int(rng.integers(0, lens[b]))) for b in rng.integers(0, 3, 6)]
    for b, t in picks:
        cut = np.array([t + 1], np.int32)
        qa = oracle.absorb_q_ref(inp["q_nope"][b:b + 1, t], inp["q_rope"][b:b + 1, t],
                                 inp["w_uk"], np.array([t]), w.tau, w.alpha_q, w.theta)
        lo = oracle.latent_attn_ref(qa, inp["ckv"][b:b + 1], inp["krope"][b:b + 1], cut, w.n)
        ref = oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv)[0]
        err = row_rel_err(got[b, t], ref)
        say(f"  row ({b}, {t}): rel err {err:.2e}")
        assert err <= TOL
    for b, L in enumerate(lens):
        assert not np.any(got[b, L:])


# ---- MLA (one branch) in the unabsorbed, multi-head form: mla_prefill ----

def run_mla_prefill(w, inp, d=None, out_dtype=torch.float32):
    d = Dev(w, inp) if d is None else d
    cfg = config_for(w)
    out = torch.empty(d.B, d.Lmax, w.heads, w.d_v, dtype=out_dtype, device="cuda")
    br.mla_prefill(cfg, d.q_nope, d.q_rope, d.w_uk, d.w_uv, d.cache(cfg), out)
    torch.cuda.synchronize()
    return out, d


@pytest.mark.parametrize("lens,T", [([300, 1, 129, 0], 300), ([128, 127, 33], 160),
                                    ([64, 65, 255], 256)])
def test_mla_prefill_all_rows_small(lens, T):
    # several 128-position blocks and 64-position projection blocks, ragged
    # ends, a one-token prompt and an empty one; MLA at the pages' scales
    # (alpha_q = alpha_kv = sqrt(7168 / 512)) against the unabsorbed oracle
    w = WORKLOADS["mla_prefill_b4_t4k"].replace(batch=len(lens), heads=8)
    inp = make_inputs(w, lens=np.array(lens, np.int32), max_len=T, q_rows=T)
    say(f"mla_prefill lens {lens} T={T}")
    got, _ = run_mla_prefill(w, inp)
    err = check_rows(host(got), oracle_prefill(w, inp), lens)
    say(f"  worst row rel err {err:.2e}")
    assert err <= TOL


def test_mla_prefill_bf16_output_and_clamped_lengths():
    w = WORKLOADS["mla_prefill_b4_t4k"].replace(batch=3, heads=4)
    T = 96
    inp = make_inputs(w, lens=np.array([96, 40, 0], np.int32), max_len=T, q_rows=T)
    want, d = run_mla_prefill(w, inp)
    got16, _ = run_mla_prefill(w, inp, d=d, out_dtype=torch.bfloat16)
    assert torch.equal(got16, want.to(torch.bfloat16))
    d.lens.copy_(torch.tensor([96 + 7, 40, -5], dtype=torch.int32))
    got, _ = run_mla_prefill(w, inp, d=d)
    assert torch.equal(got, want)
    assert check_rows(host(want), oracle_prefill(w, inp), [96, 40, 0]) <= TOL


def test_mla_prefill_row_equals_decode_of_cut_cache():
    # row t of the prefill is the decode (num_branches = 1) of the cache cut
    # after row t: both through the library, on the same inputs
    w = WORKLOADS["mla_prefill_b4_t4k"].replace(batch=2, heads=128)
    T = 200
    lens = np.array([200, 77], np.int32)
    inp = make_inputs(w, lens=lens, max_len=T, q_rows=T)
    got, d = run_mla_prefill(w, inp)
    got = host(got)
    cfg = config_for(w, q_residue=True)
    for b, t in [(0, 0), (0, 31), (0, 127), (0, 128), (0, 199), (1, 76)]:
        dec = Dev(w.replace(batch=1), dict(ckv=inp["ckv"][b:b + 1], krope=inp["krope"][b:b + 1],
                                           q_nope=inp["q_nope"][b:b + 1, t],
                                           q_rope=inp["q_rope"][b:b + 1, t], w_uk=inp["w_uk"],
                                           w_uv=inp["w_uv"], lens=np.array([t + 1], np.int32)))
        row = host(dec.decode(cfg))[0]
        err = row_rel_err(got[b, t], row)
        say(f"  row ({b}, {t}) vs decode: rel err {err:.2e}")
        assert err <= 2 * TOL


@pytest.mark.slow
def test_mla_prefill_full_size_sampled_rows():
    w = WORKLOADS["mla_prefill_b4_t4k"]
    T = w.cache_len
    lens = np.array([T, T - 1, 2049, 1], np.int32)
    inp = make_inputs(w, lens=lens, q_rows=T)
    say(f"mla_prefill B={w.batch} T={T} H={w.heads}")
    got, _ = run_mla_prefill(w, inp)
    got = host(got)
    rng = np.random.default_rng(6)
    picks = [(0, 0), (0, 31), (0, 127), (0, 128), (0, T - 1), (1, T - 2), (2, 2048), (2, 1000),
             (3, 0)] + [(int(b), int(rng.integers(0, lens[b]))) for b in rng.integers(0, 3, 6)]
    for b, t in picks:
        # the unabsorbed decode of the cache cut after row t, one query
        ref = oracle.mlra_decode_ref(inp["q_nope"][b:b + 1, t], inp["q_rope"][b:b + 1, t],
                                     inp["w_uk"], inp["w_uv"], inp["ckv"][b:b + 1, :t + 1],
                                     inp["krope"][b:b + 1, :t + 1], np.array([t + 1], np.int32), 1,
                                     tau=w.tau, alpha_q=w.alpha_q, alpha_kv=w.alpha_kv,
                                     theta=w.theta)[0]
        err = row_rel_err(got[b, t], ref)
        say(f"  row ({b}, {t}): rel err {err:.2e}")
        assert err <= TOL
    for b, L in enumerate(lens):
        assert not np.any(got[b, L:])
