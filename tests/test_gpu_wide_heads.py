"""GPU parity of the wide MLA decode at 32 and 64 heads.

One device's share of MLA under 4- or 2-way tensor parallelism keeps every
latent column and a quarter or half of the heads ("Multi-Head Low-Rank
Attention", 研究动机: MLA's cache cannot be split over devices, so each device
reads the whole 576-wide row for its heads). The wide kernel then runs H/16
score waves; all eight waves still load, convert and accumulate their share of
every tile. Each case compares every row with the float64 oracle (the
absorbed chain) at the bf16 bar (max row relative L2 error 1e-2), on ragged
lengths that span several 32-token tiles and a ragged tail, with and without
a forced split, on bf16 and fp8 caches.
"""

import numpy as np
import pytest

import branch_rank_amd as br
import oracle
import synth
from synth import WORKLOADS, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def oracle_out(w, inp, fp8):
    if fp8:
        ckv = oracle.fp8_dequantize(inp["ckv8"], inp["sc"])
        kr = oracle.fp8_dequantize(inp["krope8"], inp["sr"])
    else:
        ckv, kr = inp["ckv"], inp["krope"]
    lens = inp["lens"]
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], np.maximum(lens - 1, 0),
                             w.tau, w.alpha_q)
    lo = oracle.latent_attn_ref(qa, ckv, kr, lens, w.n)
    return oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv), lo


@pytest.mark.parametrize("heads", [32, 64])
@pytest.mark.parametrize("chunk", [0, 96])
@pytest.mark.parametrize("fp8", [False, True])
def test_wide_kernel_with_fewer_heads(heads, chunk, fp8):
    w = WORKLOADS["mla_tp4_b16_l32k"].replace(batch=5, heads=heads)
    lens = np.array([333, 1, 0, 97, 1000], np.int32)
    inp = make_inputs(w, lens=lens, max_len=1024)
    if fp8:
        inp = synth.fp8_inputs(inp)
    d = Dev(w, inp, fp8=fp8)
    cfg = config_for(w, kv_chunk=chunk)
    assert br.select_decode_kernel(cfg, d.cache(cfg)) == "wide"
    ref, lo_ref = oracle_out(w, inp, fp8)
    err = row_rel_err(host(d.decode(cfg)), ref)
    say(f"MLA H={heads} wide chunk={chunk} fp8={fp8}: mlra_decode worst row rel err {err:.2e}")
    assert err <= TOL
    # the step calls: absorb, the latent of the cache (query with its residue)
    cfg = config_for(w, kv_chunk=chunk, q_residue=True)
    err = row_rel_err(host(d.latent(cfg, d.absorb(cfg))), lo_ref)
    say(f"  mla_decode_attn latent worst row rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.slow
def test_tp4_share_full_size_every_row():
    # the 4-way share at its full size (16 x 32K, 32 heads), every row, and
    # bitwise the same on a second run
    w = WORKLOADS["mla_tp4_b16_l32k"]
    inp = make_inputs(w)
    d = Dev(w, inp)
    cfg = config_for(w)
    assert br.select_decode_kernel(cfg, d.cache(cfg)) == "wide"
    got = host(d.decode(cfg))
    assert np.array_equal(got, host(d.decode(cfg))), "not run-to-run deterministic"
    err = row_rel_err(got, oracle_out(w, inp, False)[0])
    say(f"MLA 4-way share, 16 x 32K, every row: worst row rel err {err:.2e}")
    assert err <= TOL
