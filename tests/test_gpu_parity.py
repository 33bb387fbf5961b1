"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Tolerance (maximum over output rows of the relative L2 error): 1e-5 for the
fp32 path, 1e-2 for bf16 caches, as the decode specification requires.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-5
BF16_TOL = 1e-2


def tiny_w(n, **kw):
    w = WORKLOADS["tiny_mla_fp32"].replace(n=n, **kw)
    return w


def oracle_out(w, inp, n=None, q_pos=None):
    return oracle.mlra_decode_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"],
                                  inp["ckv"], inp["krope"], inp["lens"], w.n if n is None else n,
                                  tau=w.tau, alpha_q=w.alpha_q, alpha_kv=w.alpha_kv,
                                  theta=w.theta, q_pos=q_pos)


@pytest.mark.parametrize("n", [1, 2, 4])
def test_tiny_fp32_end_to_end(n):
    w = tiny_w(n, alpha_q=1.3, alpha_kv=0.7)
    inp = make_inputs(w)
    say(f"tiny fp32 n={n}")
    d = Dev(w, inp)
    got = host(d.decode(config_for(w)))
    err = row_rel_err(got, oracle_out(w, inp))
    say(f"  rel err {err:.2e}")
    assert err <= FP32_TOL


@pytest.mark.parametrize("n", [1, 4])
def test_tiny_fp32_each_step(n):
    w = tiny_w(n, alpha_q=1.3, alpha_kv=0.7)
    inp = make_inputs(w)
    d = Dev(w, inp)
    cfg = config_for(w)
    pos = inp["lens"] - 1
    qa_ref = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], pos, w.tau, w.alpha_q)
    assert row_rel_err(host(d.absorb(cfg)), qa_ref) <= FP32_TOL
    # decode on the oracle's absorbed query
    lo_ref = oracle.latent_attn_ref(qa_ref, inp["ckv"], inp["krope"], inp["lens"], n)
    qa = torch.from_numpy(qa_ref.astype(np.float32)).cuda()
    assert row_rel_err(host(d.latent(cfg, qa)), lo_ref) <= FP32_TOL
    out_ref = oracle.out_proj_ref(lo_ref, inp["w_uv"], w.alpha_kv)
    lo = torch.from_numpy(lo_ref.astype(np.float32)).cuda()
    assert row_rel_err(host(d.out_proj(cfg, lo)), out_ref) <= FP32_TOL


@pytest.mark.parametrize("chunk", [0, 1, 5, 64, 300])
def test_tiny_ragged_lengths_and_split_sizes(chunk):
    # lengths 0 (empty), 1, a ragged tail and the full buffer; every split size
    # must give the oracle's answer
    w = tiny_w(2, batch=5)
    lens = np.array([37, 0, 1, 256, 129], np.int32)
    inp = make_inputs(w, lens=lens, max_len=256)
    say(f"ragged chunk={chunk}")
    got = host(Dev(w, inp).decode(config_for(w, kv_chunk=chunk)))
    ref = oracle_out(w, inp)
    assert np.all(got[1] == 0)
    assert row_rel_err(got, ref) <= FP32_TOL


def test_tiny_rope_shift_on_gpu():
    # keys rotated a further delta and the query moved by delta: same output
    w = tiny_w(4, init="rms", alpha_q=2.0)
    inp = make_inputs(w)
    delta = 100000
    B, Lmax = inp["ckv"].shape[:2]
    shifted = dict(inp, krope=oracle.rope(inp["krope"], np.full((B, Lmax), float(delta)))
                   .astype(np.float32))
    q_pos = torch.tensor(inp["lens"] - 1 + delta, dtype=torch.int32, device="cuda")
    base = host(Dev(w, inp).decode(config_for(w)))
    moved = host(Dev(w, shifted).decode(config_for(w), q_pos=q_pos))
    ref = oracle_out(w, inp)
    assert row_rel_err(base, ref) <= FP32_TOL
    assert row_rel_err(moved, ref) <= 2 * FP32_TOL


def test_tiny_bf16_out_dtype():
    w = tiny_w(1).replace(dtype="bf16")
    inp = make_inputs(w)
    d = Dev(w, inp)
    out = d.decode(config_for(w), out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    assert row_rel_err(host(out), oracle_out(w, inp)) <= BF16_TOL


def test_mla_b16_l4k_bf16_all_rows():
    w = WORKLOADS["mla_b16_l4k"]
    say("mla_b16_l4k: inputs")
    inp = make_inputs(w)
    d = Dev(w, inp)
    say("  gpu")
    got = host(d.decode(config_for(w)))
    again = host(d.decode(config_for(w)))
    assert np.array_equal(got, again), "not run-to-run deterministic"
    say("  oracle (absorbed chain, all rows)")
    pos = inp["lens"] - 1
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], pos, w.tau, w.alpha_q)
    lo = oracle.latent_attn_ref(qa, inp["ckv"], inp["krope"], inp["lens"], w.n)
    ref = oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv)
    err = row_rel_err(got, ref)
    say(f"  rel err {err:.2e}")
    assert err <= BF16_TOL
    # a few rows against the unabsorbed definition
    for b, h in ((0, 0), (15, 127), (7, 64)):
        sl = lambda a: a[b:b + 1]  # noqa: E731
        r = oracle.mlra_decode_ref(sl(inp["q_nope"])[:, h:h + 1], sl(inp["q_rope"])[:, h:h + 1],
                                   inp["w_uk"][h:h + 1], inp["w_uv"][h:h + 1], sl(inp["ckv"]),
                                   sl(inp["krope"]), sl(inp["lens"]), w.n, tau=w.tau,
                                   alpha_q=w.alpha_q, alpha_kv=w.alpha_kv)
        assert row_rel_err(got[b:b + 1, h:h + 1], r) <= BF16_TOL
