"""GPU parity of the bf16 MFMA decode path at the DeepSeek-V3 attention shape.

Every case runs through the C ABI (mlra_decode or the step calls) and is
compared with the float64 oracle on the same seeded inputs; tolerance is the
bf16 bar, maximum row relative L2 error <= 1e-2. Full-size workloads are
checked on sampled sequences (all heads of each), which the oracle computes
exactly with its absorbed chain (pinned equal to the unabsorbed definition),
plus a few (sequence, head) rows against the unabsorbed definition itself.
"""

import math

import numpy as np
import pytest
import torch

import branch_rank_amd as br
import oracle
from synth import WORKLOADS, make_inputs
from tests._gpu import Dev, config_for, host, row_rel_err, say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def pages_alphas(w, n):
    """alpha_q = sqrt(d / d_c'), alpha_kv = sqrt(d / d_c) at model width 7168
    ("Multi-Head Low-Rank Attention", method steps)."""
    return dict(alpha_q=math.sqrt(7168 / (w.d_c // n)), alpha_kv=math.sqrt(7168 / w.d_c))


def absorbed_oracle(w, inp, seqs, n=None):
    n = w.n if n is None else n
    sel = lambda a: a[seqs]  # noqa: E731
    lens = inp["lens"][seqs]
    qa = oracle.absorb_q_ref(sel(inp["q_nope"]), sel(inp["q_rope"]), inp["w_uk"], lens - 1,
                             w.tau, w.alpha_q)
    lo = oracle.latent_attn_ref(qa, sel(inp["ckv"]), sel(inp["krope"]), lens, n)
    return oracle.out_proj_ref(lo, inp["w_uv"], w.alpha_kv)


def unabsorbed_rows(w, inp, rows, n=None):
    n = w.n if n is None else n
    out = []
    for b, h in rows:
        s = slice(b, b + 1)
        L = int(inp["lens"][b])
        r = oracle.mlra_decode_ref(inp["q_nope"][s, h:h + 1], inp["q_rope"][s, h:h + 1],
                                   inp["w_uk"][h:h + 1], inp["w_uv"][h:h + 1],
                                   inp["ckv"][s, :L], inp["krope"][s, :L], inp["lens"][s], n,
                                   tau=w.tau, alpha_q=w.alpha_q, alpha_kv=w.alpha_kv)
        out.append(r[0, 0])
    return np.stack(out)


def small(w, B=3, L=(300, 1, 77), Lmax=320):
    return w.replace(batch=B), np.array(L, np.int32), Lmax


# (workload, branches, decode kernel); "auto" picks the branch-per-wave kernel
# for MLRA-4 at d_c = 512 and the head-group kernel otherwise
KERNEL_CASES = [("mla_b16_l4k", 1, "auto"), ("mla_b16_l4k", 1, "head_group"),
                ("mla_unit_scales", 1, "auto"),
                ("mlra4_b16_l32k", 2, "auto"),
                ("mlra4_b16_l32k", 4, "branch"), ("mlra4_b16_l32k", 4, "head_group"),
                ("mlra4_b16_l32k", 4, "portable")]


@pytest.mark.parametrize("name,n,kernel", KERNEL_CASES)
@pytest.mark.parametrize("chunk", [0, 32, 100, 4096])
def test_small_ragged_every_split(name, n, kernel, chunk):
    # several tiles, a ragged tail, a one-token sequence; every split size
    # "mla_unit_scales": MLA with alpha_q = alpha_kv = 1 (the other MLA cases
    # take the pages' sqrt(7168 / 512))
    base = WORKLOADS["mla_b16_l4k"].replace(alpha_q=1.0, alpha_kv=1.0) \
        if name == "mla_unit_scales" else WORKLOADS[name]
    alphas = pages_alphas(base, n) if n > 1 else {}
    w, lens, Lmax = small(base.replace(n=n, **alphas))
    inp = make_inputs(w, lens=lens, max_len=Lmax)
    say(f"{name} n={n} kernel={kernel} chunk={chunk}")
    got = host(Dev(w, inp).decode(config_for(w, kv_chunk=chunk, kernel=kernel)))
    ref = absorbed_oracle(w, inp, np.arange(w.batch))
    err = row_rel_err(got, ref)
    say(f"  rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("kernel", ["branch", "head_group"])
def test_empty_sequences_give_zero(kernel):
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=4)
    lens = np.array([0, 64, 0, 33], np.int32)
    inp = make_inputs(w, lens=lens, max_len=64)
    got = host(Dev(w, inp).decode(config_for(w, kernel=kernel)))
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert row_rel_err(got, absorbed_oracle(w, inp, np.arange(4))) <= TOL


@pytest.mark.parametrize("kernel", ["branch", "head_group"])
def test_latent_step_against_oracle_query(kernel):
    # decode step alone, fed the oracle's absorbed query (rounded to bf16)
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, lens=np.array([1000, 517], np.int32), max_len=1024)
    d = Dev(w, inp)
    cfg = config_for(w, kernel=kernel)
    qa = oracle.absorb_q_ref(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["lens"] - 1, w.tau,
                             w.alpha_q)
    qa_dev = torch.from_numpy(qa.astype(np.float32)).cuda().to(torch.bfloat16)
    qa_b = qa_dev.float().cpu().numpy().astype(np.float64)
    lo_ref = oracle.latent_attn_ref(qa_b, inp["ckv"], inp["krope"], inp["lens"], w.n)
    # with the query rounding taken out, what remains is P in bf16 and fp32
    # accumulation: well below the end-to-end bar
    err = row_rel_err(host(d.latent(cfg, qa_dev)), lo_ref)
    say(f"decode step ({kernel}) on the oracle's bf16 query: rel err {err:.2e}")
    assert err <= 5e-3
    # absorbed query itself
    assert row_rel_err(host(d.absorb(cfg)), qa) <= TOL


def test_shard_sum_equals_four_branch_call():
    # MLRA-4 decomposes over branches: four one-branch calls on each latent
    # quarter (same shared K_RoPE, same alpha_q, alpha_kv) sum to the n=4 call
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, lens=np.array([2000, 777], np.int32), max_len=2048)
    full = host(Dev(w, inp).decode(config_for(w)))
    total = np.zeros_like(full)
    for j in range(4):
        sl = slice(128 * j, 128 * (j + 1))
        wj = w.replace(d_c=128, n=1)
        ij = dict(inp, ckv=np.ascontiguousarray(inp["ckv"][..., sl]),
                  w_uk=np.ascontiguousarray(inp["w_uk"][:, sl]),
                  w_uv=np.ascontiguousarray(inp["w_uv"][:, sl]))
        total += host(Dev(wj, ij).decode(config_for(wj)))
    assert row_rel_err(total, full) <= TOL


@pytest.mark.parametrize("kernel", ["branch", "head_group"])
def test_sixty_four_heads(kernel):
    # 64 heads: one workgroup holds every head of a work item
    w = WORKLOADS["mlra4_b16_l32k"].replace(heads=64)
    w, lens, Lmax = small(w)
    inp = make_inputs(w, lens=lens, max_len=Lmax)
    got = host(Dev(w, inp).decode(config_for(w, kernel=kernel)))
    err = row_rel_err(got, absorbed_oracle(w, inp, np.arange(w.batch)))
    say(f"H=64 {kernel}: rel err {err:.2e}")
    assert err <= TOL


def test_forced_kernel_outside_its_shapes_is_unsupported():
    w = WORKLOADS["mla_b16_l4k"]
    w, lens, Lmax = small(w)
    inp = make_inputs(w, lens=lens, max_len=Lmax)
    with pytest.raises(br.MlraError) as e:
        Dev(w, inp).decode(config_for(w, kernel="branch"))  # n = 1
    assert e.value.status == br.MLRA_ERR_UNSUPPORTED


@pytest.mark.slow
@pytest.mark.parametrize("name,kernel", [("mlra4_b16_l32k", "auto"),
                                         ("mlra4_b16_l32k", "head_group"),
                                         ("mla_b16_l32k", "auto"),
                                         ("mla_b16_l32k", "head_group")])
def test_headline_b16_l32k_sampled(name, kernel):
    w = WORKLOADS[name]
    say(f"{name} ({kernel}): inputs")
    inp = make_inputs(w)
    d = Dev(w, inp)
    say("  gpu")
    got = host(d.decode(config_for(w, kernel=kernel)))
    again = host(d.decode(config_for(w, kernel=kernel)))
    assert np.array_equal(got, again), "not run-to-run deterministic"
    # every sequence, all heads, against the absorbed chain; a few rows
    # against the unabsorbed definition itself
    seqs = np.arange(w.batch)
    say("  oracle")
    err = row_rel_err(got[seqs], absorbed_oracle(w, inp, seqs))
    say(f"  worst row rel err over {len(seqs)} sequences x {w.heads} heads: {err:.2e}")
    assert err <= TOL
    rows = [(0, 0), (7, 64), (15, 127)]
    err2 = row_rel_err(np.stack([got[b, h] for b, h in rows]), unabsorbed_rows(w, inp, rows))
    say(f"  unabsorbed rows {rows}: {err2:.2e}")
    assert err2 <= TOL


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mla_b2_l128k", "mlra4_b2_l128k"])
def test_long_context_b2_l128k(name):
    w = WORKLOADS[name]
    say(f"{name}: inputs")
    inp = make_inputs(w)
    got = host(Dev(w, inp).decode(config_for(w)))
    say("  oracle")
    err = row_rel_err(got, absorbed_oracle(w, inp, np.arange(2)))
    say(f"  worst row rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.slow
def test_shard_b64_ragged_sampled():
    w = WORKLOADS["shard_b64_ragged"]
    say("shard_b64_ragged: inputs")
    inp = make_inputs(w)
    lens = inp["lens"]
    got = host(Dev(w, inp).decode(config_for(w)))
    # all 64 sequences (the shortest, 1024 + a few tokens, and the longest
    # included), all heads
    seqs = np.arange(w.batch)
    say(f"  oracle on {len(seqs)} sequences, lengths {int(lens.min())}..{int(lens.max())}")
    err = row_rel_err(got[seqs], absorbed_oracle(w, inp, seqs))
    say(f"  worst row rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mla_tp4_b16_l32k", "mlra4_shard_b16_l32k"])
def test_tensor_parallel_shards_sampled(name):
    # one device's share under 4-way tensor parallelism: MLA with 32 heads over
    # 576-wide rows, one MLRA-4 branch with 128 heads over 192-wide rows
    w = WORKLOADS[name]
    say(f"{name}: inputs")
    inp = make_inputs(w)
    got = host(Dev(w, inp).decode(config_for(w)))
    seqs = np.arange(w.batch)
    say("  oracle")
    err = row_rel_err(got[seqs], absorbed_oracle(w, inp, seqs))
    say(f"  worst row rel err {err:.2e}")
    assert err <= TOL
    rows = [(3, 0), (12, w.heads - 1)]
    assert row_rel_err(np.stack([got[b, h] for b, h in rows]), unabsorbed_rows(w, inp, rows)) <= TOL


@pytest.mark.parametrize("batch", [16, 64, 3])
def test_out_proj_step_bf16(batch):
    # output projection alone on the oracle's fp32 latent: the fp32 latent is
    # split into bf16 hi + lo for the MFMA, so the result is fp32-accurate
    w = WORKLOADS["mlra4_b16_l32k"].replace(batch=batch)
    inp = make_inputs(w, lens=np.full(batch, 8, np.int32), max_len=8)
    rng = np.random.default_rng(5)
    lo = rng.standard_normal((batch, w.heads, w.d_c))
    d = Dev(w, inp)
    got = host(d.out_proj(config_for(w), torch.from_numpy(lo.astype(np.float32)).cuda()))
    ref = oracle.out_proj_ref(lo.astype(np.float32).astype(np.float64), inp["w_uv"], w.alpha_kv)
    err = row_rel_err(got, ref)
    say(f"out_proj bf16 B={batch}: rel err {err:.2e}")
    assert err <= 1e-4


@pytest.mark.parametrize("name,kernel", [("mlra4_b16_l32k", "branch"), ("mla_b16_l4k", "head_group"),
                                         ("mla_b16_l4k", "wide"), ("shard_b64_ragged", "head_group")])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fused_merge_matches_separate_calls(name, kernel, out_dtype):
    # mlra_decode merges the split-KV partials and projects them in one
    # kernel (blocks of 8 sequences, two per head); the separate calls
    # (mla_decode_attn, then mla_out_proj) merge into a latent in memory
    # first. 17 sequences cross the blocks; empty sequences give zero rows.
    w = WORKLOADS[name].replace(batch=17)
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 700, size=w.batch).astype(np.int32)
    lens[[3, 16]] = 0
    inp = make_inputs(w, lens=lens, max_len=700)
    # the separate calls carry q~'s residue as mlra_decode does internally
    cfg = config_for(w, kernel=kernel, q_residue=True)
    d = Dev(w, inp)
    assert br.select_decode_kernel(cfg, d.cache(cfg)) == kernel
    fused = host(d.decode(cfg, out_dtype=out_dtype))
    sep = host(d.out_proj(cfg, d.latent(cfg, d.absorb(cfg)), out_dtype=out_dtype))
    assert not np.any(fused[[3, 16]])
    tol = 1e-5 if out_dtype == torch.float32 else 2.0 ** -7  # one bf16 rounding apart
    err = row_rel_err(fused, sep)
    say(f"{name} {kernel} {out_dtype}: fused vs separate rel err {err:.2e}")
    assert err <= tol


@pytest.mark.parametrize("name,kernel", [("mlra4_b16_l32k", "branch"), ("mla_b16_l4k", "head_group"),
                                         ("mla_b16_l4k", "wide")])
def test_fused_merge_many_slots(name, kernel):
    # 64-token work items give up to 79 partial slots per sequence, so the
    # fused merge runs its weight table in several 32-slot passes; a
    # sequence of exactly one item, an empty one and one ending one token
    # into an item cross the pass and item edges
    w = WORKLOADS[name].replace(batch=5)
    lens = np.array([5000, 2100, 64, 0, 4097], np.int32)
    inp = make_inputs(w, lens=lens, max_len=5000)
    cfg = config_for(w, kernel=kernel, kv_chunk=64, q_residue=True)
    d = Dev(w, inp)
    fused = host(d.decode(cfg))
    sep = host(d.out_proj(cfg, d.latent(cfg, d.absorb(cfg))))
    assert not np.any(fused[3])
    err = row_rel_err(fused, sep)
    say(f"{name} {kernel} chunk 64: fused vs separate rel err {err:.2e}")
    assert err <= 1e-5
    ref = absorbed_oracle(w, inp, np.array([0, 2, 4]))
    assert row_rel_err(fused[[0, 2, 4]], ref) <= TOL


@pytest.mark.parametrize("d_c,n,heads", [(256, 2, 64), (256, 1, 128), (128, 1, 32)])
def test_other_latent_widths(d_c, n, heads):
    # the MFMA path's d_c = 256 and d_c = 128 instantiations (absorb_q,
    # head-group decode, fused merge + projection) against the oracle at the
    # pages' scales, alpha_q = sqrt(7168 / d_c') and alpha_kv = sqrt(7168 /
    # d_c), with W of std 1/sqrt(d_c): the scores spread wider than at
    # d_c = 512, and a query rounded to one bf16 alone would move these rows
    # past the bar (a numpy model of that rounding gives 1.08e-2 at d_c = 256,
    # n = 2), so the head-group kernel carries the query's rounding residue;
    # and the fused merge against the separate calls
    base = WORKLOADS["mla_b16_l4k"]
    w = base.replace(d_c=d_c, n=n, heads=heads, batch=5, **pages_alphas(base.replace(d_c=d_c), n))
    lens = np.array([300, 1, 0, 77, 129], np.int32)
    inp = make_inputs(w, lens=lens, max_len=320)
    cfg = config_for(w, q_residue=True)
    d = Dev(w, inp)
    kernel = br.select_decode_kernel(cfg, d.cache(cfg))
    say(f"d_c={d_c} n={n} H={heads}: kernel {kernel}")
    got = host(d.decode(cfg))
    err = row_rel_err(got[[0, 1, 3, 4]], absorbed_oracle(w, inp, np.array([0, 1, 3, 4])))
    say(f"  worst row rel err {err:.2e}")
    assert err <= TOL
    assert not np.any(got[2])
    sep = host(d.out_proj(cfg, d.latent(cfg, d.absorb(cfg))))
    assert row_rel_err(got, sep) <= 1e-5
