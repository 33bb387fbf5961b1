"""Helpers for the GPU tests: upload seeded inputs, call the library through the
Python binding (which calls the C ABI), compare with the oracle."""

import sys

import numpy as np
import torch

import branch_rank_amd as br


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def config_for(w, n=None, kv_chunk=0, kernel="auto", q_residue=False):
    return br.make_config(w.heads, w.d_c, w.d_r, w.d_n, w.d_v, n=w.n if n is None else n,
                          sm_scale=w.tau, alpha_q=w.alpha_q, alpha_kv=w.alpha_kv,
                          theta=w.theta, dtype=w.dtype, kv_chunk=kv_chunk, kernel=kernel,
                          q_residue=q_residue)


class Dev:
    """Device copies of one input set; the cache is one interleaved buffer of
    [c_t || k^R_t] rows.

    poison=True fills every row at or past a sequence's length (the rows in
    [L_b, L_max)) with NaN, and the decode calls fill their workspace with
    NaN bytes first, so that a kernel reading a row it must not read, or a
    workspace word before it was written, puts NaN into the output."""

    def __init__(self, w, inp, device="cuda", lens=None, poison=False, fp8=False):
        dt = torch_dtype(w)
        B, Lmax, _ = inp["ckv"].shape
        self.w = w
        # fp8: the cache holds the E4M3 codes inp["ckv8"], inp["krope8"] with
        # the scales inp["sc"], inp["sr"] (synth.fp8_inputs)
        self.fp8 = (inp["sc"], inp["sr"]) if fp8 else None
        if fp8:
            self.buf = torch.empty(B, Lmax, w.d_c + w.d_r, dtype=torch.uint8, device=device)
            self.buf[..., :w.d_c] = torch.from_numpy(inp["ckv8"]).to(device)
            self.buf[..., w.d_c:] = torch.from_numpy(inp["krope8"]).to(device)
        else:
            self.buf = torch.empty(B, Lmax, w.d_c + w.d_r, dtype=dt, device=device)
            self.buf[..., :w.d_c] = torch.from_numpy(inp["ckv"]).to(device).to(dt)
            self.buf[..., w.d_c:] = torch.from_numpy(inp["krope"]).to(device).to(dt)
        self.ckv = self.buf[..., :w.d_c]
        self.krope = self.buf[..., w.d_c:]
        L = inp["lens"] if lens is None else lens
        self.lens = torch.from_numpy(np.asarray(L, np.int32)).to(device)
        for k in ("q_nope", "q_rope", "w_uk", "w_uv"):
            setattr(self, k, torch.from_numpy(inp[k]).to(device).to(dt))
        self.B, self.Lmax = B, Lmax
        self.poison = poison
        if poison:
            for b, n in enumerate(np.asarray(L, np.int64)):
                # NaN (E4M3: code 0x7F)
                self.buf[b, max(int(n), 0):] = 0x7F if fp8 else float("nan")

    def workspace(self, cfg):
        ws = br.alloc_workspace(cfg, self.B, self.Lmax)
        if self.poison:
            ws.fill_(0xFF)  # every fp32 word NaN
        return ws

    def cache(self, cfg):
        return br.cache_view(self.ckv, self.krope, self.lens, cfg, fp8_scales=self.fp8)

    def decode(self, cfg, n=None, out_dtype=torch.float32, q_pos=None):
        n = cfg.num_branches if n is None else n
        out = torch.empty(self.B, self.w.heads, self.w.d_v, dtype=out_dtype, device=self.buf.device)
        ws = self.workspace(cfg if n == cfg.num_branches else _with_n(cfg, n))
        br.mlra_decode(cfg, n, self.q_nope, self.q_rope, self.w_uk, self.w_uv, self.cache(cfg), ws,
                       out, q_pos=q_pos)
        torch.cuda.synchronize()
        return out

    def absorb(self, cfg, q_pos=None):
        qa = torch.empty(self.B, self.w.heads, br.q_abs_width(cfg), dtype=torch_dtype(self.w),
                         device=self.buf.device)
        br.mla_absorb_q(cfg, self.q_nope, self.q_rope, self.w_uk, qa, q_pos=q_pos,
                        cache_lens=self.lens)
        torch.cuda.synchronize()
        return qa

    def latent(self, cfg, q_abs):
        lo = torch.empty(self.B, self.w.heads, self.w.d_c, dtype=torch.float32, device=self.buf.device)
        ws = self.workspace(cfg)
        br.mla_decode_attn(cfg, q_abs, self.cache(cfg), ws, lo)
        torch.cuda.synchronize()
        return lo

    def out_proj(self, cfg, latent, out_dtype=torch.float32):
        out = torch.empty(self.B, self.w.heads, self.w.d_v, dtype=out_dtype, device=self.buf.device)
        br.mla_out_proj(cfg, latent, self.w_uv, out)
        torch.cuda.synchronize()
        return out


def _with_n(cfg, n):
    c = br.Config.from_buffer_copy(cfg)
    c.num_branches = n
    return c


def host(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def row_rel_err(got, ref):
    """max over rows (last axis) of ||got - ref|| / ||ref||; rows whose
    reference is exactly zero must be exactly zero."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    zero = den == 0
    assert np.all(num[zero] == 0), "rows that must be zero are not"
    if np.all(zero):
        return 0.0
    return float(np.max(num[~zero] / den[~zero]))
