"""Every decode path through the debug build (device bounds checks).

Run as ``MLRA_LIB=<libmlra_debug.so> python -m tests._debug_bounds_run`` (by
tests/test_gpu_debug_bounds.py): each case runs mlra_decode, the step calls
(mla_absorb_q, mla_decode_attn) and mlra_decode_noalloc on ragged lengths
(an empty sequence, one token, tiles with ragged tails), split and unsplit;
a failed device check makes the call return MLRA_ERR_BOUNDS, which the
binding raises. The outputs are also held to the float64 oracle at the bf16
bar. Prints one line per case and exits non-zero on the first failure.
"""

import sys

import numpy as np
import torch

import branch_rank_amd as br
import oracle
import synth
from synth import WORKLOADS, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err

TOL = 1e-2
CASES = [("mlra4_b16_l32k", "branch", False), ("mlra4_b16_l32k", "head_group", False),
         ("mlra4_b16_l32k", "portable", False), ("mla_b16_l4k", "wide", False),
         ("mla_b16_l4k", "head_group", False), ("mla_tp4_b16_l32k", "wide", False),
         ("shard_b64_ragged", "branch", False), ("mlra4_b16_l32k", "branch", True),
         ("mla_b16_l4k", "wide", True), ("mlra4_b16_l32k", "portable", True)]


def reference(w, inp, fp8):
    ckv, kr = ((oracle.fp8_dequantize(inp["ckv8"], inp["sc"]),
                oracle.fp8_dequantize(inp["krope8"], inp["sr"])) if fp8
               else (inp["ckv"], inp["krope"]))
    lens = inp["lens"]
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], np.maximum(lens - 1, 0),
                             w.tau, w.alpha_q)
    lo = oracle.latent_attn_ref(qa, ckv, kr, lens, w.n)
    return oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv), lo


def main():
    assert br.bounds_checks(), "not the debug build"
    torch.cuda.set_device(0)
    for name, kernel, fp8 in CASES:
        w = WORKLOADS[name].replace(batch=5)
        lens = np.array([333, 1, 0, 97, 500], np.int32)
        inp = make_inputs(w, lens=lens, max_len=512)
        if fp8:
            inp = synth.fp8_inputs(inp)
        d = Dev(w, inp, fp8=fp8)
        ref, lo_ref = reference(w, inp, fp8)
        for chunk in (0, 96):
            cfg = config_for(w, kv_chunk=chunk, kernel=kernel, q_residue=True)
            assert br.select_decode_kernel(cfg, d.cache(cfg)) == kernel
            e1 = row_rel_err(host(d.decode(cfg)), ref)
            e2 = row_rel_err(host(d.latent(cfg, d.absorb(cfg))), lo_ref)
            out = torch.empty(w.batch, w.heads, w.d_v, dtype=torch.float32, device="cuda")
            br.mlra_decode_noalloc(cfg, w.n, d.q_nope, d.q_rope, d.w_uk, d.w_uv, d.cache(cfg), out)
            torch.cuda.synchronize()
            e3 = row_rel_err(host(out), ref)
            print(f"{name} {kernel} fp8={fp8} chunk={chunk}: checks passed; "
                  f"rel err {e1:.2e} / {e2:.2e} / {e3:.2e}", flush=True)
            assert max(e1, e2, e3) <= TOL
    print("ok", flush=True)


if __name__ == "__main__":
    sys.exit(main())
