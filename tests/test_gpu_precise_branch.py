"""The four-branch branch kernel in fp16 (cfg->q_residue = 1, and every fp8
cache).

MLRA-4's bf16 path rounds q~ to one bf16 and P to bf16 (2^-9), which leaves
its worst rows near 7.4e-3 (short contexts up to 9.8e-3) against the 1e-2 bar
at the pages' scales ("Multi-Head Low-Rank Attention", 方法步骤详情: alpha_q =
sqrt(7168 / 128)). With q_residue = 1 the kernel takes q~ from both bf16 parts
as fp16, converts each tile to fp16 in LDS and keeps P in fp16 (2^-11). These
cases hold that mode to 3e-3 (the bar stays 1e-2 for every path; 3e-3 pins what
the mode is for), against the float64 oracle on every row.
"""

import numpy as np
import pytest

import branch_rank_amd as br
import oracle
from synth import WORKLOADS, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu

PRECISE = 3e-3


def reference(w, inp):
    lens = inp["lens"]
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], np.maximum(lens - 1, 0),
                             w.tau, w.alpha_q)
    lo = oracle.latent_attn_ref(qa, inp["ckv"], inp["krope"], lens, w.n)
    return oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv), lo


def test_short_contexts_precise_mode():
    # 64 sequences of 2..200 tokens: a sharp softmax over few keys, where the
    # query's rounding shows most (8192 rows)
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=64)
    rng = np.random.default_rng(2003)
    lens = rng.integers(2, 201, size=w.batch).astype(np.int32)
    inp = make_inputs(w, lens=lens, max_len=int(lens.max()))
    d = Dev(w, inp)
    ref, lo_ref = reference(w, inp)
    cfg = config_for(w, q_residue=True)
    assert br.select_decode_kernel(cfg, d.cache(cfg)) == "branch"
    err = row_rel_err(host(d.decode(cfg)), ref)
    fast = row_rel_err(host(d.decode(config_for(w))), ref)
    say(f"64 short MLRA-4 contexts: precise mode {err:.2e}, bf16 mode {fast:.2e}")
    assert err <= PRECISE and fast <= 1e-2
    # the step calls: mla_absorb_q with the residue, then mla_decode_attn
    err = row_rel_err(host(d.latent(cfg, d.absorb(cfg))), lo_ref)
    say(f"  mla_decode_attn latent (precise): {err:.2e}")
    assert err <= PRECISE


@pytest.mark.parametrize("chunk", [0, 96])
def test_ragged_precise_mode(chunk):
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=5)
    lens = np.array([333, 1, 0, 97, 1000], np.int32)
    inp = make_inputs(w, lens=lens, max_len=1024)
    d = Dev(w, inp)
    err = row_rel_err(host(d.decode(config_for(w, kv_chunk=chunk, q_residue=True))),
                      reference(w, inp)[0])
    say(f"MLRA-4 ragged, chunk={chunk}, precise mode: {err:.2e}")
    assert err <= PRECISE


@pytest.mark.slow
def test_full_size_precise_mode_every_row():
    w = WORKLOADS["mlra4_b16_l32k"]
    inp = make_inputs(w)
    d = Dev(w, inp)
    cfg = config_for(w, q_residue=True)
    got = host(d.decode(cfg))
    assert np.array_equal(got, host(d.decode(cfg))), "not run-to-run deterministic"
    err = row_rel_err(got, reference(w, inp)[0])
    say(f"MLRA-4 16 x 32K precise mode, every row: {err:.2e}")
    assert err <= PRECISE
