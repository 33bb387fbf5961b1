"""GPU parity of the quantised (FP8 E4M3) latent cache.

The reading ("MLA多头潜在注意力机制", 9.2: an 8-bit cache for inference; the
format and scale convention are the library's): the cache holds E4M3 codes,
one fp32 scale per cache tensor, value = scale * e4m3(code). The reference is
the float64 oracle on the cache the codes stand for (oracle.fp8_dequantize),
so the bar is the bf16 one (max row relative L2 error <= 1e-2): the kernels'
arithmetic, not the format's rounding, is what is measured. The codes come
from torch's float8_e4m3fn cast of the synthetic cache (synth.fp8_inputs),
never from the library.

Cases: every kernel that reads fp8 (the branch kernel for MLRA-4, the wide
kernel for MLA, the portable kernel for any shape) on ragged lengths that span
several tiles and a ragged tail, split and unsplit, through mlra_decode and
through the step calls (mla_decode_attn rescales the caller's query); the
full-size workloads on every sequence; the append's codes against the
oracle's quantiser; NaN codes past every sequence's end.
"""

import numpy as np
import pytest
import torch

import branch_rank_amd as br
import oracle
import synth
from synth import WORKLOADS, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def deq(inp):
    """The cache the codes stand for, float64."""
    return (oracle.fp8_dequantize(inp["ckv8"], inp["sc"]),
            oracle.fp8_dequantize(inp["krope8"], inp["sr"]))


def oracle_out(w, inp, n=None, seqs=None):
    n = w.n if n is None else n
    seqs = np.arange(w.batch) if seqs is None else np.asarray(seqs)
    ckv, kr = deq(inp)
    lens = inp["lens"][seqs]
    qa = oracle.absorb_q_ref(inp["q_nope"][seqs], inp["q_rope"][seqs], inp["w_uk"], lens - 1,
                             w.tau, w.alpha_q)
    lo = oracle.latent_attn_ref(qa, ckv[seqs], kr[seqs], lens, n)
    return oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv), lo


CASES = [("mlra4_b16_l32k", "auto", "branch"), ("mlra4_b16_l32k", "portable", "portable"),
         ("mla_b16_l4k", "auto", "wide"), ("mla_b16_l4k", "portable", "portable"),
         ("shard_b64_ragged", "auto", "portable")]


@pytest.mark.parametrize("name,kernel,expect", CASES)
@pytest.mark.parametrize("chunk", [0, 96])
def test_fp8_decode_small_ragged(name, kernel, expect, chunk):
    w = WORKLOADS[name].replace(batch=5)
    lens = np.array([333, 1, 0, 97, 1000], np.int32)
    inp = synth.fp8_inputs(make_inputs(w, lens=lens, max_len=1024))
    d = Dev(w, inp, fp8=True)
    cfg = config_for(w, kv_chunk=chunk, kernel=kernel)
    assert br.select_decode_kernel(cfg, d.cache(cfg)) == expect
    say(f"fp8 {name} {expect} chunk={chunk}: scales {inp['sc']:.4g} {inp['sr']:.4g}")
    got = host(d.decode(cfg))
    ref, _ = oracle_out(w, inp)
    err = row_rel_err(got, ref)
    say(f"  mlra_decode worst row rel err {err:.2e}")
    assert err <= TOL


# q_residue = 0 only with four branches: a one-softmax decode (MLA) on a
# query rounded to one bf16 sits at the bar at the pages' scales whatever the
# cache holds (the residue is what mla_absorb_q offers for it)
@pytest.mark.parametrize("name,kernel,residue", [("mlra4_b16_l32k", "auto", False),
                                                 ("mlra4_b16_l32k", "auto", True),
                                                 ("mla_b16_l4k", "auto", True),
                                                 ("mla_b16_l4k", "portable", True),
                                                 ("mlra4_b16_l32k", "portable", False)])
def test_fp8_step_calls(name, kernel, residue):
    # mla_absorb_q (no cache involved), then mla_decode_attn on the fp8 cache:
    # it scales a copy of the query and returns the latent of the dequantised
    # cache; then mla_out_proj
    w = WORKLOADS[name].replace(batch=4)
    lens = np.array([700, 33, 1, 256], np.int32)
    inp = synth.fp8_inputs(make_inputs(w, lens=lens, max_len=704))
    d = Dev(w, inp, fp8=True)
    cfg = config_for(w, kernel=kernel, q_residue=residue)
    qa = d.absorb(cfg)
    qa_before = qa.clone()
    lo = d.latent(cfg, qa)
    assert torch.equal(qa, qa_before), "mla_decode_attn changed the caller's query"
    ref, lo_ref = oracle_out(w, inp)
    err = row_rel_err(host(lo), lo_ref)
    say(f"fp8 {name} {kernel} residue={residue}: latent worst row rel err {err:.2e}")
    assert err <= TOL
    err = row_rel_err(host(d.out_proj(cfg, lo)), ref)
    say(f"  out_proj worst row rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mlra4_b16_l32k", "mla_b16_l32k"])
def test_fp8_full_size(name):
    # the workload at its full size: every sequence, all heads, against the
    # absorbed chain on the dequantised cache (16 sequences x 32K tokens)
    w = WORKLOADS[name]
    say(f"fp8 {name}: inputs")
    inp = synth.fp8_inputs(make_inputs(w))
    d = Dev(w, inp, fp8=True)
    cfg = config_for(w)
    say(f"  gpu ({br.select_decode_kernel(cfg, d.cache(cfg))})")
    got = host(d.decode(cfg))
    again = host(d.decode(cfg))
    assert np.array_equal(got, again), "not run-to-run deterministic"
    say("  oracle")
    ref, _ = oracle_out(w, inp)
    err = row_rel_err(got, ref)
    say(f"  worst row rel err over {w.batch} sequences x {w.heads} heads: {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("kernel", ["branch", "portable"])
def test_fp8_nan_codes_past_every_end(kernel):
    # rows at or past each sequence's length hold the NaN code; the workspace
    # is NaN bytes: nothing may reach the output
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=5)
    lens = np.array([333, 1, 0, 97, 500], np.int32)
    inp = synth.fp8_inputs(make_inputs(w, lens=lens, max_len=540))
    d = Dev(w, inp, fp8=True, poison=True)
    cfg = config_for(w, kernel=kernel)
    got = d.decode(cfg)
    assert torch.isfinite(got).all().item()
    err = row_rel_err(host(got), oracle_out(w, inp)[0])
    say(f"fp8 {kernel} with NaN codes past the ends: worst row rel err {err:.2e}")
    assert err <= TOL


def test_fp8_wide_nan_codes_past_every_end():
    w = WORKLOADS["mla_b16_l4k"].replace(batch=5)
    lens = np.array([333, 1, 0, 97, 500], np.int32)
    inp = synth.fp8_inputs(make_inputs(w, lens=lens, max_len=540))
    d = Dev(w, inp, fp8=True, poison=True)
    cfg = config_for(w, kernel="wide")
    got = d.decode(cfg)
    assert torch.isfinite(got).all().item()
    err = row_rel_err(host(got), oracle_out(w, inp)[0])
    say(f"fp8 wide with NaN codes past the ends: worst row rel err {err:.2e}")
    assert err <= TOL


def _near_tie(x):
    """True where x lies within a relative 2^-20 of a rounding boundary of
    E4M3 (a midpoint between neighbouring codes, or 448 + 16 for
    saturation): there the library's fp32 arithmetic before the rounding may
    pick the other neighbour."""
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    vals = np.unique(np.abs(vals[np.isfinite(vals)]))
    mids = 0.5 * (vals[1:] + vals[:-1])
    a = np.abs(x)
    i = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    near = np.minimum(np.abs(a - mids[i]), np.abs(a - mids[i - 1]))
    return near <= 2.0 ** -20 * np.maximum(a, 2.0 ** -9)


def test_fp8_append_codes():
    w = WORKLOADS["mlra4_b16_l32k"]
    Lmax = 24
    lens0 = np.array([0, 7, Lmax, Lmax - 1, 13, 1], np.int32)  # the third is full
    w = w.replace(batch=len(lens0))
    inp = synth.fp8_inputs(make_inputs(w, lens=lens0, max_len=Lmax))
    rng = np.random.default_rng(12)
    rows = (rng.standard_normal((w.batch, w.row)) * 3.0).astype(np.float32)
    gain = (1.0 + 0.1 * rng.standard_normal(w.d_c)).astype(np.float32)
    sc, sr = 0.0123, 0.0071
    d = Dev(w, inp, fp8=True)
    before = host(d.buf).astype(np.uint8)
    cfg = config_for(w)
    br.cache_append_fp8(cfg, torch.from_numpy(rows).cuda(), d.ckv, d.krope, d.lens, sc, sr,
                        gain=torch.from_numpy(gain).cuda(), eps=1e-6)
    torch.cuda.synchronize()
    after = d.buf.cpu().numpy()
    lens1 = d.lens.cpu().numpy()
    c_ref, k_ref, l_ref = oracle.cache_append_ref(np.zeros((w.batch, Lmax, w.d_c)),
                                                  np.zeros((w.batch, Lmax, w.d_r)), lens0,
                                                  rows[:, :w.d_c], rows[:, w.d_c:], Lmax,
                                                  gain=gain, eps=1e-6, theta=w.theta)
    assert lens1.tolist() == l_ref.tolist()
    checked = ties = 0
    for b in range(w.batch):
        p = int(lens0[b])
        for t in range(Lmax):
            if t != p:
                assert np.array_equal(after[b, t], before[b, t]), (b, t)
                continue
            for got, x, s in ((after[b, t, :w.d_c], c_ref[b, p], sc),
                              (after[b, t, w.d_c:], k_ref[b, p], sr)):
                want = oracle.fp8_quantize(x, s)
                tie = _near_tie(x / s)
                assert np.array_equal(got[~tie], want[~tie]), (b, t)
                # at a near-tie either neighbour is right
                alt = oracle.e4m3_decode(got[tie]) * s
                assert np.all(np.abs(alt - x[tie]) <= np.abs(oracle.fp8_dequantize(want[tie], s)
                                                             - x[tie]) * (1 + 2.0 ** -18) +
                              2.0 ** -30)
                checked += got.size
                ties += int(tie.sum())
    say(f"fp8 append: {checked} codes checked, {ties} near a tie")
    assert checked > 0
