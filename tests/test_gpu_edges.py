"""GPU edge cases of the decode path through the C ABI, against the float64
oracle: the largest sizes the library accepts, out-of-range cache lengths
(clamped to [0, max_len]), degenerate branch and head counts, and one long
sequence split over every work item of the branch decode kernel."""

import numpy as np
import pytest
import torch

import branch_rank_amd as br
import oracle
from synth import WORKLOADS, Workload, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2}


def full_oracle(w, inp, n=None):
    n = w.n if n is None else n
    return oracle.mlra_decode_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"],
                                  inp["ckv"], inp["krope"], inp["lens"], n, tau=w.tau,
                                  alpha_q=w.alpha_q, alpha_kv=w.alpha_kv, theta=w.theta)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_largest_accepted_sizes(dtype):
    # d_latent 1024, d_rope 256, d_nope 512, 8 branches (the library's limits);
    # none of the MFMA specialisations covers them, so the generic kernels run
    w = Workload("max_sizes", 2, 4, 1024, 256, 512, 256, 8, 40, dtype=dtype, init="fan_in",
                 seed=2001)
    lens = np.array([37, 5], np.int32)
    inp = make_inputs(w, lens=lens, max_len=40)
    cfg = config_for(w)
    assert br.select_decode_kernel(cfg, Dev(w, inp).cache(cfg)) == "portable"
    got = host(Dev(w, inp).decode(cfg))
    err = row_rel_err(got, full_oracle(w, inp))
    say(f"max sizes {dtype}: rel err {err:.2e}")
    assert err <= TOL[dtype]


def test_one_wide_branches_and_single_head():
    # as many branches as latent columns (each softmax sees one latent
    # column plus the RoPE key; 8 is the library's most), one head
    w = Workload("degenerate", 3, 1, 8, 16, 32, 32, 8, 64, dtype="fp32", init="fan_in",
                 seed=2002)
    lens = np.array([64, 1, 9], np.int32)
    inp = make_inputs(w, lens=lens, max_len=64)
    got = host(Dev(w, inp).decode(config_for(w)))
    err = row_rel_err(got, full_oracle(w, inp))
    say(f"8 one-wide branches, H=1: rel err {err:.2e}")
    assert err <= TOL["fp32"]


@pytest.mark.parametrize("name,kernel", [("mlra4_b16_l32k", "branch"),
                                         ("mlra4_b16_l32k", "head_group"),
                                         ("mlra4_b16_l32k", "portable"),
                                         ("mla_b16_l4k", "wide")])
def test_out_of_range_lengths_are_clamped(name, kernel):
    # lengths below 0 act as 0 and above max_len as max_len: the same output,
    # bit for bit, as the clamped lengths
    w = WORKLOADS[name].replace(batch=4)
    Lmax = 96
    inp = make_inputs(w, lens=np.array([0, 96, 0, 7], np.int32), max_len=Lmax)
    cfg = config_for(w, kernel=kernel)
    d = Dev(w, inp)
    want = host(d.decode(cfg))
    d.lens.copy_(torch.tensor([-3, 96 + 5, -2147483647, 7], dtype=torch.int32))
    got = host(d.decode(cfg))
    assert np.array_equal(got, want)
    assert not np.any(got[0]) and not np.any(got[2])
    ref = oracle.out_proj_ref(
        oracle.latent_attn_ref(
            oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"],
                                np.maximum(inp["lens"] - 1, 0), w.tau, w.alpha_q),
            inp["ckv"], inp["krope"], inp["lens"], w.n),
        inp["w_uv"], w.alpha_kv)
    assert row_rel_err(got[[1, 3]], ref[[1, 3]]) <= TOL["bf16"]


@pytest.mark.slow
def test_single_long_sequence_over_all_items():
    # B = 1: every work item of the branch kernel cuts the same sequence, so
    # the merge combines ~128 partial states of one (branch, head)
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=1, cache_len=65536)
    inp = make_inputs(w)
    cfg = config_for(w)
    d = Dev(w, inp)
    assert br.select_decode_kernel(cfg, d.cache(cfg)) == "branch"
    got = host(d.decode(cfg))
    say("  oracle")
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["lens"] - 1, w.tau,
                             w.alpha_q)
    lo = oracle.latent_attn_ref(qa, inp["ckv"], inp["krope"], inp["lens"], w.n)
    err = row_rel_err(got, oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv))
    say(f"B=1, L=65536: rel err {err:.2e}")
    assert err <= TOL["bf16"]


@pytest.mark.slow
@pytest.mark.parametrize("kernel", ["wide", "head_group"])
def test_single_long_mla_sequence_over_all_items(kernel):
    # MLA, B = 1, L = 65536: every work item cuts the same sequence
    w = WORKLOADS["mla_b16_l32k"].replace(batch=1, cache_len=65536)
    inp = make_inputs(w)
    cfg = config_for(w, kernel=kernel)
    d = Dev(w, inp)
    got = host(d.decode(cfg))
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["lens"] - 1, w.tau,
                             w.alpha_q)
    lo = oracle.latent_attn_ref(qa, inp["ckv"], inp["krope"], inp["lens"], w.n)
    err = row_rel_err(got, oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv))
    say(f"MLA B=1, L=65536 ({kernel}): worst row rel err {err:.2e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("kernel", ["wide", "head_group"])
def test_many_short_contexts_mla(kernel):
    # 64 sequences of 2..200 tokens at MLA's scales on the pages (8192 rows)
    w = WORKLOADS["mla_b16_l4k"].replace(batch=64)
    rng = np.random.default_rng(2004)
    lens = rng.integers(2, 201, size=w.batch).astype(np.int32)
    inp = make_inputs(w, lens=lens, max_len=int(lens.max()))
    got = host(Dev(w, inp).decode(config_for(w, kernel=kernel)))
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], lens - 1, w.tau, w.alpha_q,
                             w.theta)
    ref = oracle.out_proj_ref(oracle.latent_attn_ref(qa, inp["ckv"], inp["krope"], lens, w.n),
                              inp["w_uv"], w.alpha_kv)
    err = row_rel_err(got, ref)
    say(f"64 short MLA contexts ({kernel}): worst row rel err {err:.2e}")
    assert err <= TOL["bf16"]


def test_many_short_contexts_mlra4():
    # 64 sequences of 2..200 tokens at MLRA-4's alpha_q: sharp softmax over
    # few keys is where rounding q~ to bf16 shows most (8192 rows checked)
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=64)
    rng = np.random.default_rng(2003)
    lens = rng.integers(2, 201, size=w.batch).astype(np.int32)
    inp = make_inputs(w, lens=lens, max_len=int(lens.max()))
    got = host(Dev(w, inp).decode(config_for(w)))
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], lens - 1, w.tau, w.alpha_q,
                             w.theta)
    ref = oracle.out_proj_ref(oracle.latent_attn_ref(qa, inp["ckv"], inp["krope"], lens, w.n),
                              inp["w_uv"], w.alpha_kv)
    err = row_rel_err(got, ref)
    say(f"64 short MLRA-4 contexts: worst row rel err {err:.2e}")
    assert err <= TOL["bf16"]
