"""Value range of the MFMA decodes' split-KV partials.

The MFMA decodes (branch, head-group, wide) hand each work item's partial
latent output to the merge as acc / l in fp16: a weighted mean of cache rows,
so its magnitude is bounded by the rows' own, whatever the softmax's sums
reach. Scaling the latent cache by 2^12 and W_UK by 2^-12 (powers of two,
exact in bf16) leaves every score of the absorbed decode ("Multi-Head Low-Rank
Attention", 方法步骤详情 steps 1-2: q~ = W_UK q^N, s_t = q~ . c_t + rho . k^R_t)
unchanged and scales the output by 2^12: the cache then holds values near
+-2e4, where unnormalised fp16 accumulators would overflow, and every row must
still meet the 1e-2 bar against the float64 oracle. Beyond fp16's range
(2^17: values past 65504) the MFMA paths saturate, as the header documents,
and stay finite; the portable kernel (fp32 partials) still meets the bar.
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


def scaled_inputs(w, k, lens, max_len):
    inp = make_inputs(w, lens=lens, max_len=max_len)
    inp["ckv"] = (inp["ckv"] * np.float32(2.0 ** k)).astype(np.float32)
    inp["w_uk"] = (inp["w_uk"] * np.float32(2.0 ** -k)).astype(np.float32)
    return inp


def reference(w, inp):
    lens = inp["lens"]
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], np.maximum(lens - 1, 0),
                             w.tau, w.alpha_q)
    lo = oracle.latent_attn_ref(qa, inp["ckv"], inp["krope"], lens, w.n)
    return oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv)


CASES = [("mlra4_b16_l32k", "branch", False), ("mlra4_b16_l32k", "branch", True),
         ("mlra4_b16_l32k", "head_group", False), ("mla_b16_l4k", "wide", False),
         ("mla_b16_l4k", "head_group", False)]


@pytest.mark.parametrize("name,kernel,residue", CASES)
def test_large_latent_values_within_fp16(name, kernel, residue):
    w = WORKLOADS[name].replace(batch=5)
    lens = np.array([333, 1, 0, 97, 1000], np.int32)
    inp = scaled_inputs(w, 12, lens, 1024)
    assert 1e4 < np.abs(inp["ckv"]).max() < 65504
    d = Dev(w, inp)
    cfg = config_for(w, kernel=kernel, q_residue=residue)
    assert br.select_decode_kernel(cfg, d.cache(cfg)) == kernel
    got = host(d.decode(cfg))
    err = row_rel_err(got, reference(w, inp))
    say(f"{name} {kernel} residue={residue}, cache values up to {np.abs(inp['ckv']).max():.0f}: "
        f"worst row rel err {err:.2e}")
    assert err <= TOL


def test_latent_values_beyond_fp16_saturate():
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=3)
    lens = np.array([200, 37, 513], np.int32)
    inp = scaled_inputs(w, 17, lens, 520)
    assert np.abs(inp["ckv"]).max() > 65504
    d = Dev(w, inp)
    ref = reference(w, inp)
    got = d.decode(config_for(w, kernel="branch"))
    assert torch.isfinite(got).all().item(), "saturated partials must stay finite"
    err = row_rel_err(host(d.decode(config_for(w, kernel="portable"))), ref)
    say(f"cache values up to {np.abs(inp['ckv']).max():.0f}: portable worst row rel err {err:.2e}")
    assert err <= TOL
