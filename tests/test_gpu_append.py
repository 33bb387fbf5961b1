"""GPU parity of the cache append (mlra_cache_append) and of a short decode
loop that appends a token and decodes, step after step, against the float64
oracle advancing the same state.

Appended rows are compared element by element with the oracle's float64
values within the storage type's rounding bound (bf16: unit roundoff 2^-8,
plus the fp32 arithmetic before it); rows that must not change are compared
bit for bit and the lengths exactly.
"""

import numpy as np
import pytest
import torch

import branch_rank_amd as br
import oracle
from synth import WORKLOADS, make_inputs, round_bf16
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _case(name, dtype):
    w = WORKLOADS[name]
    if dtype == "fp32":
        w = w.replace(dtype="fp32")
    return w


@pytest.mark.parametrize("name,dtype", [("mlra4_b16_l32k", "bf16"), ("mla_b16_l4k", "bf16"),
                                        ("tiny_mla_fp32", "fp32")])
def test_append_rows_against_oracle(name, dtype):
    w = _case(name, dtype)
    Lmax = 40
    lens0 = np.array([0, 7, Lmax, Lmax - 1, 13, 1], np.int32)  # the third is full
    w = w.replace(batch=len(lens0))
    inp = make_inputs(w, lens=lens0, max_len=Lmax)
    rng = np.random.default_rng(11)
    rows = (rng.standard_normal((w.batch, w.row)) * 3.0).astype(np.float32)
    gain = (1.0 + 0.1 * rng.standard_normal(w.d_c)).astype(np.float32)
    d = Dev(w, inp)
    before = host(d.buf).copy()
    cfg = config_for(w)
    say(f"append {name} {dtype}: lens {lens0.tolist()}")
    br.cache_append(cfg, torch.from_numpy(rows).cuda(), d.ckv, d.krope, d.lens,
                    gain=torch.from_numpy(gain).cuda(), eps=1e-6)
    torch.cuda.synchronize()
    after = host(d.buf)
    lens1 = host(d.lens)
    c_ref, k_ref, l_ref = oracle.cache_append_ref(before[..., :w.d_c], before[..., w.d_c:], lens0,
                                                  rows[:, :w.d_c], rows[:, w.d_c:], Lmax,
                                                  gain=gain, eps=1e-6, theta=w.theta)
    assert lens1.tolist() == l_ref.tolist()
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    for b in range(w.batch):
        p = int(lens0[b])
        for t in range(Lmax):
            if t == p:
                continue
            assert np.array_equal(after[b, t], before[b, t]), (b, t)
        if p >= Lmax:
            continue
        ref = np.concatenate([c_ref[b, p], k_ref[b, p]])
        got = after[b, p].astype(np.float64)
        bound = (u * 1.001 + 4e-6) * np.abs(ref) + 1e-30
        worst = float(np.max(np.abs(got - ref) / bound))
        say(f"  seq {b} row {p}: worst error / bound {worst:.3f}")
        assert worst <= 1.0


@pytest.mark.parametrize("name,n", [("mlra4_b16_l32k", 4), ("mla_b16_l4k", 1)])
def test_append_and_decode_loop(name, n):
    # three decode steps, each appending the new token first; the oracle
    # keeps its own cache (appended rows rounded to bf16 as stored)
    w = WORKLOADS[name]
    Lmax = 320
    lens = np.array([0, 5, 100, 300], np.int32)
    w = w.replace(batch=len(lens))
    inp = make_inputs(w, lens=lens, max_len=Lmax)
    d = Dev(w, inp)
    cfg = config_for(w, n=n)
    ckv = inp["ckv"].astype(np.float64)
    kr = inp["krope"].astype(np.float64)
    L = lens.copy()
    rng = np.random.default_rng(12)
    for step in range(3):
        rows = rng.standard_normal((w.batch, w.row)).astype(np.float32)
        br.cache_append(cfg, torch.from_numpy(rows).cuda(), d.ckv, d.krope, d.lens)
        got = host(d.decode(cfg, n=n))
        ckv, kr, L = oracle.cache_append_ref(ckv, kr, L, rows[:, :w.d_c], rows[:, w.d_c:], Lmax,
                                             theta=w.theta, round_to=round_bf16)
        assert host(d.lens).tolist() == L.tolist()
        qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], L - 1, w.tau,
                                 w.alpha_q)
        lo = oracle.latent_attn_ref(qa, ckv, kr, L, n)
        ref = oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv)
        err = row_rel_err(got, ref)
        say(f"{name} step {step}: lens {L.tolist()} rel err {err:.2e}")
        assert err <= TOL
