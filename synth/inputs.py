"""Seeded synthetic workloads for latent-KV decode attention.

Recipe (one numpy PCG64 stream per tensor, spawned from the workload seed in
the fixed order lens, ckv, krope, q_nope, q_rope, w_uk, w_uv):

* C_KV rows ~ N(0, 1), then divided by their own root-mean-square (unit RMS
  rows, as a latent that has passed an RMS norm) unless the workload uses
  fan-in scaling;
* K_RoPE rows ~ N(0, 1). The cache stores them already rotated; a rotation of
  an isotropic Gaussian is again isotropic Gaussian, so drawing them directly
  gives the same distribution as rotating fresh draws;
* q_nope, q_rope ~ N(0, 1); W_UK, W_UV ~ N(0, w_std^2);
* "fan_in" workloads scale every tensor by 1/sqrt(its last width) instead
  (C_KV, K_RoPE, q) and the weights by 1/sqrt(d_c);
* bf16 workloads round every tensor to bf16 (round to nearest even) here, so
  the oracle and the GPU see identical values.

Nothing here computes a step of the decode path.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


def round_bf16(x):
    """Round float32 values to the nearest bf16 (ties to even); returns
    float32 holding bf16-representable values. Inputs must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + (((b >> 16) & 1) + 0x7FFF)) & 0xFFFF0000
    return b.view(np.float32)


def bf16_bits(x):
    """bf16 bit patterns (uint16) of bf16-representable float32 values."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    d_c: int
    d_r: int
    d_n: int
    d_v: int
    n: int                      # branch count (1 = MLA)
    cache_len: int              # uniform length, or the upper end for ragged
    dtype: str = "bf16"         # "bf16" or "fp32"
    ragged_min: Optional[int] = None   # lengths ~ U{ragged_min..cache_len}
    alpha_q: float = 1.0
    alpha_kv: float = 1.0
    theta: float = 10000.0
    init: str = "rms"           # "rms" (unit-RMS latent rows, N(0,1) q) or "fan_in"
    w_std: Optional[float] = None  # default 1/sqrt(d_c)
    seed: int = 0

    @property
    def tau(self):
        return 1.0 / math.sqrt(self.d_n + self.d_r)

    @property
    def row(self):
        return self.d_c + self.d_r

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


def _mlra4_scales():
    # d = 7168 model width, d_c = 512, d_c' = 128 (four branches)
    return math.sqrt(7168 / 128), math.sqrt(7168 / 512)


_AQ4, _AKV4 = _mlra4_scales()
# MLA is one branch with d_c' = d_c = 512: alpha_q = alpha_kv = sqrt(7168 / 512)
_A1 = math.sqrt(7168 / 512)
MLA_SCALES = dict(alpha_q=_A1, alpha_kv=_A1)

DSV3 = dict(heads=128, d_c=512, d_r=64, d_n=128, d_v=128)

WORKLOADS = {
    # tiny fp32 MLA, fan-in scaled, positions 0..255
    "tiny_mla_fp32": Workload("tiny_mla_fp32", 1, 4, 64, 16, 32, 32, 1, 256,
                              dtype="fp32", init="fan_in", seed=1001),
    # MLA at the DeepSeek-V3 attention shape, B=16, L=4096; the variance
    # correction applies to MLA too (one branch: d_c' = d_c)
    "mla_b16_l4k": Workload("mla_b16_l4k", 16, n=1, cache_len=4096, seed=1002, **MLA_SCALES,
                            **DSV3),
    # MLRA-4 headline: B=16, L=32768
    "mlra4_b16_l32k": Workload("mlra4_b16_l32k", 16, n=4, cache_len=32768,
                               alpha_q=_AQ4, alpha_kv=_AKV4, seed=1003, **DSV3),
    # MLA at the headline shape
    "mla_b16_l32k": Workload("mla_b16_l32k", 16, n=1, cache_len=32768, seed=1003, **MLA_SCALES,
                             **DSV3),
    # long context, B=2, L=131072
    "mla_b2_l128k": Workload("mla_b2_l128k", 2, n=1, cache_len=131072, seed=1004, **MLA_SCALES,
                             **DSV3),
    "mlra4_b2_l128k": Workload("mlra4_b2_l128k", 2, n=4, cache_len=131072,
                               alpha_q=_AQ4, alpha_kv=_AKV4, seed=1004, **DSV3),
    # one MLRA-4 branch (one tensor-parallel shard): latent 128 + rope 64,
    # B=64, ragged lengths U{1024..65536}
    "shard_b64_ragged": Workload("shard_b64_ragged", 64, 128, 128, 64, 128, 128, 1,
                                 65536, ragged_min=1024, alpha_q=_AQ4, alpha_kv=_AKV4,
                                 w_std=1.0 / math.sqrt(512), seed=1005),
    # one GPU's share of 4-way tensor parallelism, per scheme: MLA splits heads
    # (32 of 128) but every device streams the full 576-wide rows; MLRA-4
    # splits branches (one 128-wide latent slice + the RoPE key, 192-wide
    # rows, all 128 heads). B=16 at L=32768 and L=131072
    "mla_tp4_b16_l32k": Workload("mla_tp4_b16_l32k", 16, 32, 512, 64, 128, 128, 1, 32768,
                                 seed=1006, **MLA_SCALES),
    "mlra4_shard_b16_l32k": Workload("mlra4_shard_b16_l32k", 16, 128, 128, 64, 128, 128, 1,
                                     32768, alpha_q=_AQ4, alpha_kv=_AKV4,
                                     w_std=1.0 / math.sqrt(512), seed=1006),
    # causal prefill of MLRA-4 at the DeepSeek-V3 attention shape: 4 prompts of
    # 4096 tokens, one query per position (q_rows = 4096)
    "mlra4_prefill_b4_t4k": Workload("mlra4_prefill_b4_t4k", 4, n=4, cache_len=4096,
                                     alpha_q=_AQ4, alpha_kv=_AKV4, seed=1008, **DSV3),
    # causal prefill of MLA (one branch) in the same shape
    "mla_prefill_b4_t4k": Workload("mla_prefill_b4_t4k", 4, n=1, cache_len=4096, seed=1009,
                                   **MLA_SCALES, **DSV3),
    "mla_tp4_b16_l128k": Workload("mla_tp4_b16_l128k", 16, 32, 512, 64, 128, 128, 1, 131072,
                                  seed=1007, **MLA_SCALES),
    "mlra4_shard_b16_l128k": Workload("mlra4_shard_b16_l128k", 16, 128, 128, 64, 128, 128, 1,
                                      131072, alpha_q=_AQ4, alpha_kv=_AKV4,
                                      w_std=1.0 / math.sqrt(512), seed=1007),
}


def ragged_lens(rng, batch, lo, hi):
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def make_inputs(w: Workload, seed: Optional[int] = None, lens=None, max_len=None,
                parts=("ckv", "krope", "q_nope", "q_rope", "w_uk", "w_uv"), q_rows=None):
    """Draw the inputs of workload ``w``.

    Returns a dict of float32 arrays (bf16-representable for bf16 workloads):
    ckv [B, L_max, d_c], krope [B, L_max, d_r], q_nope [B, H, d_n],
    q_rope [B, H, d_r], w_uk [H, d_c, d_n], w_uv [H, d_c, d_v], plus
    lens [B] int32. ``lens`` / ``max_len`` override the workload's lengths.
    ``parts`` limits which tensors are drawn (the others are skipped but the
    per-tensor streams stay the same). ``q_rows`` draws one query per
    position instead (a prompt): q_nope [B, q_rows, H, d_n], q_rope
    [B, q_rows, H, d_r].
    """
    ss = np.random.SeedSequence(w.seed if seed is None else seed)
    g = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(7)]
    B, H = w.batch, w.heads
    if lens is None:
        if w.ragged_min is not None:
            lens = ragged_lens(g[0], B, w.ragged_min, w.cache_len)
        else:
            lens = np.full(B, w.cache_len, dtype=np.int32)
    lens = np.asarray(lens, dtype=np.int32)
    if max_len is None:
        max_len = int(max(int(lens.max()) if lens.size else 0, 1))
    fan = w.init == "fan_in"
    rnd = round_bf16 if w.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    w_std = w.w_std if w.w_std is not None else 1.0 / math.sqrt(w.d_c)
    out = {"lens": lens}

    if "ckv" in parts:
        c = g[1].standard_normal((B, max_len, w.d_c), dtype=np.float32)
        if fan:
            c *= np.float32(1.0 / math.sqrt(w.d_c))
        else:
            ms = np.mean(np.square(c, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
            c /= np.sqrt(ms + np.float32(1e-6))
        out["ckv"] = rnd(c)
        del c
    if "krope" in parts:
        k = g[2].standard_normal((B, max_len, w.d_r), dtype=np.float32)
        if fan:
            k *= np.float32(1.0 / math.sqrt(w.d_r))
        out["krope"] = rnd(k)
    if "q_nope" in parts:
        qs = (B, H) if q_rows is None else (B, q_rows, H)
        q = g[3].standard_normal(qs + (w.d_n,), dtype=np.float32)
        out["q_nope"] = rnd(q / math.sqrt(w.d_n) if fan else q)
    if "q_rope" in parts:
        qs = (B, H) if q_rows is None else (B, q_rows, H)
        q = g[4].standard_normal(qs + (w.d_r,), dtype=np.float32)
        out["q_rope"] = rnd(q / math.sqrt(w.d_r) if fan else q)
    if "w_uk" in parts:
        out["w_uk"] = rnd(g[5].standard_normal((H, w.d_c, w.d_n), dtype=np.float32) * np.float32(w_std))
    if "w_uv" in parts:
        out["w_uv"] = rnd(g[6].standard_normal((H, w.d_c, w.d_v), dtype=np.float32) * np.float32(w_std))
    return out


def make_cache_device(w: Workload, seed: int, lens=None, device="cuda"):
    """The cache of workload ``w`` drawn on the device with torch (same recipe
    as ``make_inputs``: unit-RMS latent rows, N(0,1) K_RoPE rows, rounded to
    the workload dtype), as one interleaved buffer [B, L_max, d_c + d_r].

    For benchmark copies of large caches, where drawing on the host would
    take longer than the measurement. Values differ from ``make_inputs``
    (another generator); the distribution is the same.
    """
    import torch

    B = w.batch
    if lens is None:
        lens = make_inputs(w, seed=seed, parts=())["lens"]
    Lmax = int(max(int(np.max(lens)) if len(lens) else 0, 1))
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    buf = torch.empty(B, Lmax, w.d_c + w.d_r, dtype=dt, device=device)
    for b in range(B):  # one sequence at a time keeps the fp32 scratch small
        c = torch.randn(Lmax, w.d_c, generator=g, device=device, dtype=torch.float32)
        if w.init == "fan_in":
            c *= 1.0 / math.sqrt(w.d_c)
        else:
            c /= torch.sqrt(torch.mean(c * c, dim=-1, keepdim=True) + 1e-6)
        buf[b, :, :w.d_c] = c.to(dt)
        k = torch.randn(Lmax, w.d_r, generator=g, device=device, dtype=torch.float32)
        if w.init == "fan_in":
            k *= 1.0 / math.sqrt(w.d_r)
        buf[b, :, w.d_c:] = k.to(dt)
    return buf, np.asarray(lens, np.int32)


def fp8_codes(x, scale):
    """FP8 E4M3 codes (uint8) of the values x / scale, by torch's
    float8_e4m3fn cast (round to nearest even). With scale = fp8_scale(x) no
    value passes 448, so no code is NaN."""
    import torch

    t = torch.as_tensor(np.asarray(x, np.float32)) / float(scale)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_scale(x):
    """Per-tensor scale that maps the largest magnitude of x to 448, the
    largest finite E4M3 value (a plain max calibration)."""
    a = float(np.max(np.abs(x))) if np.size(x) else 0.0
    return a / 448.0 if a > 0 else 1.0


def fp8_inputs(inp):
    """Adds the quantised cache of a drawn input set: ckv8, krope8 (uint8
    codes) and their per-tensor scales sc, sr."""
    out = dict(inp)
    out["sc"], out["sr"] = fp8_scale(inp["ckv"]), fp8_scale(inp["krope"])
    out["ckv8"] = fp8_codes(inp["ckv"], out["sc"])
    out["krope8"] = fp8_codes(inp["krope"], out["sr"])
    return out


def fp8_device(buf, d_c):
    """The device version for an interleaved cache buffer [B, L_max, d_c + d_r]
    (bf16 or fp32): returns (codes [B, L_max, d_c + d_r] uint8, sc, sr), one
    scale per part. Converts one sequence at a time to bound the fp32
    scratch."""
    import torch

    sc = float(buf[..., :d_c].abs().amax()) / 448.0
    sr = float(buf[..., d_c:].abs().amax()) / 448.0
    sc, sr = sc if sc > 0 else 1.0, sr if sr > 0 else 1.0
    out = torch.empty(buf.shape, dtype=torch.uint8, device=buf.device)
    for b in range(buf.shape[0]):
        out[b, :, :d_c] = (buf[b, :, :d_c].float() / sc).to(torch.float8_e4m3fn).view(torch.uint8)
        out[b, :, d_c:] = (buf[b, :, d_c:].float() / sr).to(torch.float8_e4m3fn).view(torch.uint8)
    return out, sc, sr
