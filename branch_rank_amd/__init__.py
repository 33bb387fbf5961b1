"""Python binding of libmlra (include/mlra.h): latent-KV decode attention on MI355X.

Argument marshalling only: torch tensors supply device memory and the stream;
every step of the decode runs in the library's HIP kernels. The binding checks
shapes, dtypes, devices and contiguity so that no kernel is handed a buffer
smaller than the sizes it is told. There is no CPU fallback: if libmlra.so is
missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLRA_LIB points at another build of the same library: libmlra_debug.so (the
# device bounds checks), or a tuning build
LIB_PATH = os.environ.get("MLRA_LIB") or os.path.join(_HERE, "libmlra.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libmlra_debug.so")

MLRA_OK, MLRA_ERR_INVALID_ARG, MLRA_ERR_UNSUPPORTED, MLRA_ERR_WORKSPACE, \
    MLRA_ERR_NO_DEVICE, MLRA_ERR_HIP, MLRA_ERR_BOUNDS = range(7)
MLRA_BF16, MLRA_FP32 = 0, 1
MLRA_KERNEL_AUTO, MLRA_KERNEL_PORTABLE, MLRA_KERNEL_HEAD_GROUP, MLRA_KERNEL_BRANCH, \
    MLRA_KERNEL_WIDE = 0, 1, 2, 3, 4
KERNELS = {"auto": MLRA_KERNEL_AUTO, "portable": MLRA_KERNEL_PORTABLE,
           "head_group": MLRA_KERNEL_HEAD_GROUP, "branch": MLRA_KERNEL_BRANCH,
           "wide": MLRA_KERNEL_WIDE}

EXPORTS = ("mlra_workspace_size", "mla_absorb_q", "mla_decode_attn", "mla_out_proj",
           "mlra_decode", "mlra_decode_noalloc", "mlra_select_decode_kernel",
           "mlra_cache_append", "mlra_cache_append_fp8", "mlra_prefill",
           "mla_prefill_workspace_size", "mla_prefill",
           "mlra_set_kernel_timing", "mlra_status_string", "mlra_last_error_detail",
           "mlra_bounds_checks")


class MlraError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


class Config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("num_branches", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("alpha_q", ctypes.c_float),
                ("alpha_kv", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dtype", ctypes.c_int), ("kv_chunk", ctypes.c_int32),
                ("decode_kernel", ctypes.c_int), ("q_residue", ctypes.c_int32)]


class Cache(ctypes.Structure):
    _fields_ = [("ckv", ctypes.c_void_p), ("krope", ctypes.c_void_p),
                ("ckv_batch_stride", ctypes.c_int64), ("ckv_token_stride", ctypes.c_int64),
                ("krope_batch_stride", ctypes.c_int64), ("krope_token_stride", ctypes.c_int64),
                ("cache_lens", ctypes.c_void_p), ("max_len", ctypes.c_int32),
                ("fp8", ctypes.c_int32), ("ckv_scale", ctypes.c_float),
                ("krope_scale", ctypes.c_float)]


_lib = None


def lib():
    """Load libmlra.so (built in-tree by ``python -m branch_rank_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m branch_rank_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    CP, KP = ctypes.POINTER(Config), ctypes.POINTER(Cache)
    sigs = {
        "mlra_workspace_size": [CP, I32, I32, ctypes.POINTER(SZ)],
        "mla_absorb_q": [CP, I32, P, P, P, P, P, P, P],
        "mla_decode_attn": [CP, I32, P, KP, P, SZ, P, P],
        "mla_out_proj": [CP, I32, P, P, P, ctypes.c_int, P],
        "mlra_decode": [CP, I32, I32, P, P, P, P, P, KP, P, SZ, P, ctypes.c_int, P],
        "mlra_decode_noalloc": [CP, I32, I32, P, P, P, P, P, KP, P, ctypes.c_int, P],
        "mlra_select_decode_kernel": [CP, I32, KP, ctypes.POINTER(ctypes.c_int)],
        "mlra_cache_append": [CP, I32, P, P, ctypes.c_float, P, P, ctypes.c_int64,
                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, I32, P],
        "mlra_cache_append_fp8": [CP, I32, P, P, ctypes.c_float, P, P, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, I32,
                                  ctypes.c_float, ctypes.c_float, P],
        "mlra_prefill": [CP, I32, I32, P, P, P, P, KP, P, ctypes.c_int, P],
        "mla_prefill_workspace_size": [CP, I32, I32, ctypes.POINTER(SZ)],
        "mla_prefill": [CP, I32, P, P, P, P, KP, P, SZ, P, ctypes.c_int, P],
        "mlra_set_kernel_timing": [P, P],
        "mlra_status_string": [ctypes.c_int],
        "mlra_last_error_detail": [],
        "mlra_bounds_checks": [],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_char_p if name in ("mlra_status_string",
                                               "mlra_last_error_detail") else ctypes.c_int
    _lib = L
    return L


def _status_name(st):
    try:
        return lib().mlra_status_string(st).decode()
    except Exception:  # noqa: BLE001
        return f"status {st}"


def check(st):
    if st != MLRA_OK:
        raise MlraError(st, lib().mlra_last_error_detail().decode())


def bounds_checks():
    """True when the loaded library is the debug build (device bounds checks)."""
    return bool(lib().mlra_bounds_checks())


# ------------------------------------------------------------ config ----

def make_config(heads, d_latent, d_rope, d_nope, d_v, n=1, sm_scale=0.0, alpha_q=1.0,
                alpha_kv=1.0, theta=10000.0, dtype="bf16", kv_chunk=0, kernel="auto",
                q_residue=False):
    """kernel: "auto", "portable", "head_group", "branch" or "wide" (mlra_kernel_t).
    q_residue: the q_abs rows of mla_absorb_q / mla_decode_attn also carry
    the bf16 residue of q~ (bf16 only)."""
    return Config(heads, d_latent, d_rope, d_nope, d_v, n, sm_scale, alpha_q, alpha_kv, theta,
                  MLRA_BF16 if dtype == "bf16" else MLRA_FP32, kv_chunk, KERNELS[kernel],
                  1 if q_residue else 0)


def q_abs_width(cfg):
    """Elements per q_abs row: d_latent + d_rope (+ d_latent with q_residue)."""
    return cfg.d_latent + cfg.d_rope + (cfg.d_latent if cfg.q_residue else 0)


def workspace_size(cfg, batch, max_len):
    out = ctypes.c_size_t(0)
    check(lib().mlra_workspace_size(ctypes.byref(cfg), batch, max_len, ctypes.byref(out)))
    return out.value


def _torch():
    import torch
    return torch


def _dtype(cfg):
    t = _torch()
    return t.bfloat16 if cfg.dtype == MLRA_BF16 else t.float32


def _need(x, name, shape, dtype, contiguous=True):
    t = _torch()
    if not isinstance(x, t.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(x.shape)} != {tuple(shape)}")
    if x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype} != {dtype}")
    if contiguous and not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def cache_view(ckv, krope, cache_lens, cfg, fp8_scales=None):
    """Strided cache view from tensors ckv [B, L_max, d_c] and krope
    [B, L_max, d_r] (views into one interleaved buffer are fine; the last
    dimension must be dense) and cache_lens [B] int32. With
    fp8_scales = (ckv_scale, krope_scale) the tensors are uint8 FP8 E4M3
    codes of a quantised cache (values scale * e4m3(code))."""
    t = _torch()
    B, Lmax, dc = ckv.shape
    if dc != cfg.d_latent or tuple(krope.shape) != (B, Lmax, cfg.d_rope):
        raise ValueError("cache shapes do not match the config")
    want = t.uint8 if fp8_scales is not None else _dtype(cfg)
    for x, name in ((ckv, "ckv"), (krope, "krope")):
        if x.dtype != want or not x.is_cuda:
            raise ValueError(f"{name}: wrong dtype or device")
        if x.stride(2) != 1 and x.shape[2] > 1:
            raise ValueError(f"{name}: last dimension must be dense")
        if x.stride(0) < 0 or x.stride(1) < 1:
            raise ValueError(f"{name}: bad strides")
    _need(cache_lens, "cache_lens", (B,), t.int32)
    fp8 = fp8_scales is not None
    sc, sr = (float(fp8_scales[0]), float(fp8_scales[1])) if fp8 else (1.0, 1.0)
    c = Cache(ckv.data_ptr(), krope.data_ptr(), ckv.stride(0), ckv.stride(1), krope.stride(0),
              krope.stride(1), cache_lens.data_ptr(), Lmax, int(fp8), sc, sr)
    c._keep = (ckv, krope, cache_lens)  # keep the tensors alive with the view
    c._batch = B
    return c


def cache_append(cfg, new_rows, ckv, krope, cache_lens, gain=None, eps=1e-6, stream=None):
    """Append one token per sequence: new_rows [B, d_c + d_r] fp32 (latent,
    then the unrotated RoPE key) go to row L_b of ckv [B, L_max, d_c] and
    krope [B, L_max, d_r] (RMS-normalised latent, rotated key, cache dtype),
    and cache_lens [B] int32 is incremented in place (mlra_cache_append)."""
    t = _torch()
    B, Lmax, dc = ckv.shape
    if dc != cfg.d_latent or tuple(krope.shape) != (B, Lmax, cfg.d_rope):
        raise ValueError("cache shapes do not match the config")
    for x, name in ((ckv, "ckv"), (krope, "krope")):
        if x.dtype != _dtype(cfg) or not x.is_cuda:
            raise ValueError(f"{name}: wrong dtype or device")
        if x.stride(2) != 1 and x.shape[2] > 1:
            raise ValueError(f"{name}: last dimension must be dense")
    rows = _need(new_rows, "new_rows", (B, cfg.d_latent + cfg.d_rope), t.float32)
    g = _need(gain, "gain", (cfg.d_latent,), t.float32) if gain is not None else None
    lens = _need(cache_lens, "cache_lens", (B,), t.int32)
    check(lib().mlra_cache_append(ctypes.byref(cfg), B, rows, g, float(eps), ckv.data_ptr(),
                                  krope.data_ptr(), ckv.stride(0), ckv.stride(1),
                                  krope.stride(0), krope.stride(1), lens, Lmax, _stream(stream)))


def cache_append_fp8(cfg, new_rows, ckv, krope, cache_lens, ckv_scale, krope_scale, gain=None,
                     eps=1e-6, stream=None):
    """cache_append into a quantised cache: ckv [B, L_max, d_c] and krope
    [B, L_max, d_r] uint8 FP8 E4M3 codes; each value is stored as the code
    nearest value / scale (mlra_cache_append_fp8)."""
    t = _torch()
    B, Lmax, dc = ckv.shape
    if dc != cfg.d_latent or tuple(krope.shape) != (B, Lmax, cfg.d_rope):
        raise ValueError("cache shapes do not match the config")
    for x, name in ((ckv, "ckv"), (krope, "krope")):
        if x.dtype != t.uint8 or not x.is_cuda:
            raise ValueError(f"{name}: wrong dtype or device")
        if x.stride(2) != 1 and x.shape[2] > 1:
            raise ValueError(f"{name}: last dimension must be dense")
    rows = _need(new_rows, "new_rows", (B, cfg.d_latent + cfg.d_rope), t.float32)
    g = _need(gain, "gain", (cfg.d_latent,), t.float32) if gain is not None else None
    lens = _need(cache_lens, "cache_lens", (B,), t.int32)
    check(lib().mlra_cache_append_fp8(ctypes.byref(cfg), B, rows, g, float(eps), ckv.data_ptr(),
                                      krope.data_ptr(), ckv.stride(0), ckv.stride(1),
                                      krope.stride(0), krope.stride(1), lens, Lmax,
                                      float(ckv_scale), float(krope_scale), _stream(stream)))


def select_decode_kernel(cfg, cache):
    """Name of the decode kernel ("portable", "head_group", "branch" or "wide") that
    the decode calls run for this config and cache view (host-only)."""
    k = ctypes.c_int(-1)
    check(lib().mlra_select_decode_kernel(ctypes.byref(cfg), cache._batch, ctypes.byref(cache),
                                          ctypes.byref(k)))
    return {v: n for n, v in KERNELS.items()}[k.value]


# ------------------------------------------------------------ calls ----

def mla_absorb_q(cfg, q_nope, q_rope, w_uk, q_abs, q_pos=None, cache_lens=None, stream=None):
    t = _torch()
    B, H = q_nope.shape[:2]
    dt = _dtype(cfg)
    args = (_need(q_nope, "q_nope", (B, cfg.num_heads, cfg.d_nope), dt),
            _need(q_rope, "q_rope", (B, cfg.num_heads, cfg.d_rope), dt),
            _need(q_pos, "q_pos", (B,), t.int32) if q_pos is not None else None,
            _need(cache_lens, "cache_lens", (B,), t.int32) if cache_lens is not None else None,
            _need(w_uk, "w_uk", (cfg.num_heads, cfg.d_latent, cfg.d_nope), dt),
            _need(q_abs, "q_abs", (B, cfg.num_heads, q_abs_width(cfg)), dt))
    check(lib().mla_absorb_q(ctypes.byref(cfg), B, args[0], args[1], args[2], args[3], args[4],
                             args[5], _stream(stream)))


def _ws(workspace, cfg, B, max_len):
    t = _torch()
    need = workspace_size(cfg, B, max_len)
    if workspace.dtype != t.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, needs {need}")
    return workspace.data_ptr(), workspace.numel()


def alloc_workspace(cfg, batch, max_len, device="cuda"):
    t = _torch()
    return t.empty(max(workspace_size(cfg, batch, max_len), 256), dtype=t.uint8, device=device)


def mla_decode_attn(cfg, q_abs, cache, workspace, latent_out, stream=None):
    t = _torch()
    B = cache._batch
    qa = _need(q_abs, "q_abs", (B, cfg.num_heads, q_abs_width(cfg)), _dtype(cfg))
    lo = _need(latent_out, "latent_out", (B, cfg.num_heads, cfg.d_latent), t.float32)
    wp, wn = _ws(workspace, cfg, B, cache.max_len)
    check(lib().mla_decode_attn(ctypes.byref(cfg), B, qa, ctypes.byref(cache), wp, wn, lo,
                                _stream(stream)))


def mla_out_proj(cfg, latent_out, w_uv, out, stream=None):
    t = _torch()
    B = latent_out.shape[0]
    lo = _need(latent_out, "latent_out", (B, cfg.num_heads, cfg.d_latent), t.float32)
    wv = _need(w_uv, "w_uv", (cfg.num_heads, cfg.d_latent, cfg.d_v), _dtype(cfg))
    if out.dtype not in (t.float32, t.bfloat16):
        raise ValueError("out must be float32 or bfloat16")
    op = _need(out, "out", (B, cfg.num_heads, cfg.d_v), out.dtype)
    od = MLRA_BF16 if out.dtype == t.bfloat16 else MLRA_FP32
    check(lib().mla_out_proj(ctypes.byref(cfg), B, lo, wv, op, od, _stream(stream)))


def mlra_decode(cfg, num_branches, q_nope, q_rope, w_uk, w_uv, cache, workspace, out,
                q_pos=None, stream=None):
    t = _torch()
    B = cache._batch
    dt = _dtype(cfg)
    H = cfg.num_heads
    c2 = Config.from_buffer_copy(cfg)
    c2.num_branches = num_branches
    qn = _need(q_nope, "q_nope", (B, H, cfg.d_nope), dt)
    qr = _need(q_rope, "q_rope", (B, H, cfg.d_rope), dt)
    qp = _need(q_pos, "q_pos", (B,), t.int32) if q_pos is not None else None
    wk = _need(w_uk, "w_uk", (H, cfg.d_latent, cfg.d_nope), dt)
    wv = _need(w_uv, "w_uv", (H, cfg.d_latent, cfg.d_v), dt)
    if out.dtype not in (t.float32, t.bfloat16):
        raise ValueError("out must be float32 or bfloat16")
    op = _need(out, "out", (B, H, cfg.d_v), out.dtype)
    od = MLRA_BF16 if out.dtype == t.bfloat16 else MLRA_FP32
    wp, wn = _ws(workspace, c2, B, cache.max_len)
    check(lib().mlra_decode(ctypes.byref(cfg), num_branches, B, qn, qr, qp, wk, wv,
                            ctypes.byref(cache), wp, wn, op, od, _stream(stream)))


def mlra_decode_noalloc(cfg, num_branches, q_nope, q_rope, w_uk, w_uv, cache, out, q_pos=None,
                        stream=None):
    """mlra_decode with the library's own scratch instead of a workspace
    (mlra_decode_noalloc): allocates nothing; calls that overlap on one GPU
    race."""
    t = _torch()
    B = cache._batch
    dt = _dtype(cfg)
    H = cfg.num_heads
    qn = _need(q_nope, "q_nope", (B, H, cfg.d_nope), dt)
    qr = _need(q_rope, "q_rope", (B, H, cfg.d_rope), dt)
    qp = _need(q_pos, "q_pos", (B,), t.int32) if q_pos is not None else None
    wk = _need(w_uk, "w_uk", (H, cfg.d_latent, cfg.d_nope), dt)
    wv = _need(w_uv, "w_uv", (H, cfg.d_latent, cfg.d_v), dt)
    if out.dtype not in (t.float32, t.bfloat16):
        raise ValueError("out must be float32 or bfloat16")
    op = _need(out, "out", (B, H, cfg.d_v), out.dtype)
    od = MLRA_BF16 if out.dtype == t.bfloat16 else MLRA_FP32
    check(lib().mlra_decode_noalloc(ctypes.byref(cfg), num_branches, B, qn, qr, qp, wk, wv,
                                    ctypes.byref(cache), op, od, _stream(stream)))


def mlra_prefill(cfg, num_branches, q_nope, q_rope, w_uk, w_uv, cache, out, stream=None):
    """Causal prefill (mlra_prefill): q_nope [B][T][H][d_nope], q_rope
    [B][T][H][d_rope] for positions 0..T-1 of each sequence, T = cache.max_len;
    out [B][T][H][d_v] (float32 or bfloat16), zero for t >= cache_lens[b]."""
    t = _torch()
    B, T = cache._batch, cache.max_len
    dt = _dtype(cfg)
    H = cfg.num_heads
    qn = _need(q_nope, "q_nope", (B, T, H, cfg.d_nope), dt)
    qr = _need(q_rope, "q_rope", (B, T, H, cfg.d_rope), dt)
    wk = _need(w_uk, "w_uk", (H, cfg.d_latent, cfg.d_nope), dt)
    wv = _need(w_uv, "w_uv", (H, cfg.d_latent, cfg.d_v), dt)
    if out.dtype not in (t.float32, t.bfloat16):
        raise ValueError("out must be float32 or bfloat16")
    op = _need(out, "out", (B, T, H, cfg.d_v), out.dtype)
    od = MLRA_BF16 if out.dtype == t.bfloat16 else MLRA_FP32
    check(lib().mlra_prefill(ctypes.byref(cfg), num_branches, B, qn, qr, wk, wv,
                             ctypes.byref(cache), op, od, _stream(stream)))


def mla_prefill_workspace_size(cfg, batch, max_len):
    """Bytes of workspace mla_prefill needs (host only)."""
    n = ctypes.c_size_t(0)
    check(lib().mla_prefill_workspace_size(ctypes.byref(cfg), batch, max_len, ctypes.byref(n)))
    return n.value


def mla_prefill(cfg, q_nope, q_rope, w_uk, w_uv, cache, out, workspace=None, stream=None):
    """Causal prefill of MLA in the unabsorbed (multi-head) form (mla_prefill):
    arguments as for mlra_prefill; the up-projected keys and values live in
    `workspace` (a uint8 device tensor of mla_prefill_workspace_size bytes,
    allocated here when not given)."""
    t = _torch()
    B, T = cache._batch, cache.max_len
    dt = _dtype(cfg)
    H = cfg.num_heads
    qn = _need(q_nope, "q_nope", (B, T, H, cfg.d_nope), dt)
    qr = _need(q_rope, "q_rope", (B, T, H, cfg.d_rope), dt)
    wk = _need(w_uk, "w_uk", (H, cfg.d_latent, cfg.d_nope), dt)
    wv = _need(w_uv, "w_uv", (H, cfg.d_latent, cfg.d_v), dt)
    if out.dtype not in (t.float32, t.bfloat16):
        raise ValueError("out must be float32 or bfloat16")
    op = _need(out, "out", (B, T, H, cfg.d_v), out.dtype)
    od = MLRA_BF16 if out.dtype == t.bfloat16 else MLRA_FP32
    need = mla_prefill_workspace_size(cfg, B, T)
    if workspace is None:
        workspace = t.empty(max(need, 256), dtype=t.uint8, device=out.device)
    check(lib().mla_prefill(ctypes.byref(cfg), B, qn, qr, wk, wv, ctypes.byref(cache),
                            workspace.data_ptr(), workspace.numel(), op, od, _stream(stream)))
    return workspace


def set_kernel_timing(before=None, after=None):
    """Have the split-KV decode dispatch of later calls on this thread stamp
    torch.cuda.Event `before` at its start and `after` at its end (None, None
    stops). An event whose hipEvent does not exist yet is recorded once here
    to create it; record the events before a timed region so that this adds
    nothing to it."""
    if before is None or after is None:
        check(lib().mlra_set_kernel_timing(None, None))
        return
    for e in (before, after):
        if not e.cuda_event:
            e.record()  # torch creates the underlying hipEvent on first record
    check(lib().mlra_set_kernel_timing(ctypes.c_void_p(before.cuda_event),
                                       ctypes.c_void_p(after.cuda_event)))
