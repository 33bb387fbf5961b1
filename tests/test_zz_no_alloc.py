"""The no-allocation decode step (mlra_decode_noalloc) against mlra_decode.

mlra_decode_noalloc runs the same kernels as mlra_decode on the library's
own per-GPU scratch array instead of a caller's workspace; its split-KV plan
is the same, so its output must equal mlra_decode's bit for bit (bf16 and
fp8 caches; every decode kernel that auto selection reaches). Two calls in
a row, the second on a smaller input, check that the scratch's contents left
by one call do not leak into the next. Called through the C ABI (the
binding only marshals pointers).
"""

import numpy as np
import pytest
import torch

import branch_rank_amd as br
import synth
from synth import WORKLOADS, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu


def run_both(w, inp, kernel="auto", fp8=False):
    d = Dev(w, inp, fp8=fp8)
    cfg = config_for(w, kernel=kernel)
    ref = d.decode(cfg)
    got = torch.full_like(ref, float("nan"))
    br.mlra_decode_noalloc(cfg, w.n, d.q_nope, d.q_rope, d.w_uk, d.w_uv, d.cache(cfg), got)
    torch.cuda.synchronize()
    return host(got), host(ref), br.select_decode_kernel(cfg, d.cache(cfg))


@pytest.mark.parametrize("name,fp8", [("mlra4_b16_l32k", False), ("mla_b16_l4k", False),
                                      ("mla_tp4_b16_l32k", False), ("mlra4_b16_l32k", True),
                                      ("mla_b16_l4k", True)])
def test_noalloc_matches_mlra_decode_twice_shrinking(name, fp8):
    base = WORKLOADS[name]
    prep = synth.fp8_inputs if fp8 else (lambda x: x)
    # first call: B=16 over ragged lengths up to 3000 tokens; second call:
    # B=5 with shorter sequences and an empty one
    w1 = base.replace(batch=16)
    rng = np.random.default_rng(11)
    lens1 = rng.integers(1, 3000, size=16).astype(np.int32)
    inp1 = prep(make_inputs(w1, lens=lens1, max_len=3000))
    got1, ref1, k1 = run_both(w1, inp1, fp8=fp8)
    e1 = row_rel_err(got1, ref1)
    say(f"{name} fp8={fp8} call 1 (B=16, {k1}): max row rel diff vs mlra_decode {e1:.2e}")
    assert np.isfinite(got1).all()
    assert np.array_equal(got1, ref1)
    w2 = base.replace(batch=5)
    lens2 = np.array([700, 0, 33, 512, 1], np.int32)
    inp2 = prep(make_inputs(w2, lens=lens2, max_len=700))
    got2, ref2, k2 = run_both(w2, inp2, fp8=fp8)
    e2 = row_rel_err(got2, ref2)
    say(f"{name} fp8={fp8} call 2 (B=5, {k2}): max row rel diff vs mlra_decode {e2:.2e}")
    assert np.isfinite(got2).all()
    assert np.array_equal(got2, ref2)
    assert not np.any(got2[1])


def test_noalloc_headline_size_fits_and_larger_is_refused():
    # the headline step (MLRA-4, B=16, L=32768) fits the scratch; a batch
    # whose plan needs more is refused with MLRA_ERR_WORKSPACE
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, lens=np.array([40, 9], np.int32), max_len=64)
    d = Dev(w, inp)
    cfg = config_for(w, kv_chunk=1)   # one work item per token: 130 slots of 256 KB
    out = torch.empty(2, w.heads, w.d_v, device="cuda")
    br.mlra_decode_noalloc(cfg, w.n, d.q_nope, d.q_rope, d.w_uk, d.w_uv, d.cache(cfg), out)
    assert torch.equal(out, d.decode(cfg))
    big = Dev(w.replace(batch=2), make_inputs(w, lens=np.array([4096, 4096], np.int32),
                                              max_len=4096))
    with pytest.raises(br.MlraError) as e:
        br.mlra_decode_noalloc(cfg, w.n, big.q_nope, big.q_rope, big.w_uk, big.w_uv,
                               big.cache(cfg), out)
    assert e.value.status == br.MLRA_ERR_WORKSPACE
    torch.cuda.synchronize()
