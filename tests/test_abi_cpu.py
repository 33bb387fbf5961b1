"""The C-ABI library loads, exports what include/mlra.h declares, and rejects bad
arguments with the documented status codes before touching a device.

No compute calls: pointers below are fake and every call is expected to fail
validation (or, with valid arguments, to report that no device is present).
"""

import ctypes
import os
import re

import pytest

import branch_rank_amd as br

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlra.h")
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MLRA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001
        return False


def test_library_exports_every_declared_symbol():
    L = br.lib()
    names = declared_functions()
    assert len(names) == 16, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(br.EXPORTS)


def test_debug_build_exports_the_same_symbols_and_says_so():
    # libmlra_debug.so: the same sources built with the device bounds checks
    # (the build makes both); only its mlra_bounds_checks() differs
    import ctypes
    assert os.path.exists(br.DEBUG_LIB_PATH), "libmlra_debug.so is not built"
    D = ctypes.CDLL(br.DEBUG_LIB_PATH)
    for n in declared_functions():
        assert hasattr(D, n), n
    D.mlra_bounds_checks.restype = ctypes.c_int
    assert D.mlra_bounds_checks() == 1
    if os.path.realpath(br.LIB_PATH) != os.path.realpath(br.DEBUG_LIB_PATH):
        assert not br.bounds_checks()
    D.mlra_status_string.restype = ctypes.c_char_p
    assert D.mlra_status_string(br.MLRA_ERR_BOUNDS) == b"MLRA_ERR_BOUNDS"


def cfg(**kw):
    base = dict(heads=128, d_latent=512, d_rope=64, d_nope=128, d_v=128, n=4)
    base.update(kw)
    return br.make_config(**base)


def test_workspace_size_is_host_only_and_grows():
    c = cfg()
    a = br.workspace_size(c, 16, 32768)
    b = br.workspace_size(c, 16, 65536)
    assert 0 < a <= b
    # plan header + prefix + partials + intermediates, 256-byte aligned parts
    assert a % 256 == 0
    assert br.workspace_size(c, 0, 0) > 0
    # a forced 16-token work item gives 512 items at 2 x 4096 tokens against the
    # automatic 128 (64-token minimum), so more partial slots
    c2 = cfg(kv_chunk=16)
    assert br.workspace_size(c2, 2, 4096) > br.workspace_size(cfg(), 2, 4096)


@pytest.mark.parametrize("kw,status", [
    (dict(n=3), br.MLRA_ERR_INVALID_ARG),            # 512 % 3
    (dict(d_rope=7), br.MLRA_ERR_INVALID_ARG),       # odd rope width
    (dict(heads=0), br.MLRA_ERR_INVALID_ARG),
    (dict(d_latent=2048), br.MLRA_ERR_UNSUPPORTED),
    (dict(n=16, d_latent=512, heads=128), br.MLRA_ERR_UNSUPPORTED),
    (dict(theta=0.0), br.MLRA_ERR_INVALID_ARG),
    (dict(kv_chunk=-1), br.MLRA_ERR_INVALID_ARG),
])
def test_config_validation(kw, status):
    c = cfg(**kw)
    out = ctypes.c_size_t(0)
    st = br.lib().mlra_workspace_size(ctypes.byref(c), 4, 128, ctypes.byref(out))
    assert st == status
    assert br.lib().mlra_last_error_detail().decode() != ""


@pytest.mark.parametrize("value", [-1, 5, 99])
def test_unknown_decode_kernel_is_invalid(value):
    c = cfg()
    c.decode_kernel = value
    out = ctypes.c_size_t(0)
    assert br.lib().mlra_workspace_size(ctypes.byref(c), 4, 128, ctypes.byref(out)) == \
        br.MLRA_ERR_INVALID_ARG


def _fake_cache(c, batch, max_len, ts=None):
    # host-only calls never dereference these (16-byte aligned) addresses
    ts = c.d_latent + c.d_rope if ts is None else ts
    k = br.Cache(0x100000, 0x100000 + 2 * c.d_latent, max_len * ts, ts, max_len * ts, ts,
                 0x200000, max_len)
    k._batch = batch
    return k


@pytest.mark.parametrize("kw,max_len,kernel,expect", [
    (dict(), 32768, "auto", "branch"),                            # MLRA-4, d_c = 512, H = 128
    (dict(heads=64), 4096, "auto", "branch"),
    (dict(n=1), 4096, "auto", "wide"),                            # MLA
    (dict(n=1, heads=64), 4096, "auto", "wide"),                 # MLA, 2-way TP share
    (dict(n=1, heads=32), 4096, "auto", "wide"),                 # MLA, 4-way TP share
    (dict(n=1, heads=32), 4096, "head_group", "head_group"),
    (dict(n=1), 4096, "head_group", "head_group"),
    (dict(n=2), 4096, "auto", "head_group"),
    (dict(n=1, d_latent=128), 4096, "auto", "branch"),            # one branch shard
    (dict(), 4096, "head_group", "head_group"),
    (dict(), 4096, "portable", "portable"),
    (dict(dtype="fp32"), 4096, "auto", "portable"),
    (dict(heads=96), 4096, "auto", "portable"),
    (dict(), 2_000_000, "auto", "portable"),                      # rows beyond 31-bit offsets
])
def test_kernel_selection_host_only(kw, max_len, kernel, expect):
    c = cfg(kernel=kernel, **kw)
    assert br.select_decode_kernel(c, _fake_cache(c, 2, max_len)) == expect


@pytest.mark.parametrize("kw,kernel", [(dict(n=1), "branch"), (dict(heads=96), "branch"),
                                       (dict(), "wide"), (dict(n=1, heads=96), "wide"),
                                       (dict(n=1, dtype="fp32"), "wide"),
                                       (dict(heads=96), "head_group"),
                                       (dict(dtype="fp32"), "head_group")])
def test_forced_kernel_outside_its_shapes(kw, kernel):
    c = cfg(kernel=kernel, **kw)
    with pytest.raises(br.MlraError) as e:
        br.select_decode_kernel(c, _fake_cache(c, 2, 4096))
    assert e.value.status == br.MLRA_ERR_UNSUPPORTED


def test_null_config_and_bad_batch():
    out = ctypes.c_size_t(0)
    L = br.lib()
    assert L.mlra_workspace_size(None, 1, 1, ctypes.byref(out)) == br.MLRA_ERR_INVALID_ARG
    c = cfg()
    assert L.mlra_workspace_size(ctypes.byref(c), -1, 1, ctypes.byref(out)) == br.MLRA_ERR_INVALID_ARG
    assert L.mlra_workspace_size(ctypes.byref(c), 1, -5, ctypes.byref(out)) == br.MLRA_ERR_INVALID_ARG
    assert L.mlra_workspace_size(ctypes.byref(c), 65536, 65536, ctypes.byref(out)) != br.MLRA_OK
    assert L.mlra_status_string(br.MLRA_ERR_WORKSPACE) == b"MLRA_ERR_WORKSPACE"


def cache(max_len=128, ckv=FAKE, krope=FAKE + 1024, ts=576, bs=576 * 128, lens=FAKE):
    return br.Cache(ckv, krope, bs, ts, bs, ts, lens, max_len)


def decode(c, k, ws=FAKE, ws_bytes=None, q=FAKE, out=FAKE, B=4):
    if ws_bytes is None:
        ws_bytes = br.workspace_size(c, B, k.max_len)
    return br.lib().mla_decode_attn(ctypes.byref(c), B, q, ctypes.byref(k), ws, ws_bytes, out, None)


def test_decode_argument_validation():
    c = cfg()
    assert decode(c, cache(ckv=0)) == br.MLRA_ERR_INVALID_ARG           # null cache
    assert decode(c, cache(ckv=FAKE + 2)) == br.MLRA_ERR_INVALID_ARG    # misaligned
    assert decode(c, cache(ts=577)) == br.MLRA_ERR_INVALID_ARG          # stride not 16 B
    assert decode(c, cache(ts=0)) == br.MLRA_ERR_INVALID_ARG
    # token strides below the row widths (16-byte multiples, so only the width
    # check rejects them): rows would overlap, and the kernels would disagree
    # on how much of the last row exists
    assert decode(c, cache(ts=256)) == br.MLRA_ERR_INVALID_ARG         # < d_latent 512
    k = cache()
    k.krope_token_stride = 32                                           # < d_rope 64
    assert decode(c, k) == br.MLRA_ERR_INVALID_ARG
    assert prefill(c, k=cache(ts=256)) == br.MLRA_ERR_INVALID_ARG
    assert decode(c, cache(lens=0)) == br.MLRA_ERR_INVALID_ARG
    assert decode(c, cache(), q=0) == br.MLRA_ERR_INVALID_ARG
    assert decode(c, cache(), out=FAKE + 4) == br.MLRA_ERR_INVALID_ARG
    assert decode(c, cache(), ws_bytes=100) == br.MLRA_ERR_WORKSPACE
    assert decode(c, cache(), ws=0) == br.MLRA_ERR_WORKSPACE
    assert decode(c, cache(), ws=FAKE + 16) == br.MLRA_ERR_INVALID_ARG  # 256-B alignment
    # batch 0 is a no-op that succeeds without a device
    assert decode(c, cache(), B=0) == br.MLRA_OK


def test_other_entry_points_validate():
    L = br.lib()
    c = cfg()
    assert L.mla_absorb_q(ctypes.byref(c), 4, FAKE, FAKE, None, None, FAKE, FAKE, None) == br.MLRA_ERR_INVALID_ARG
    assert L.mla_absorb_q(ctypes.byref(c), 4, 0, FAKE, None, FAKE, FAKE, FAKE, None) == br.MLRA_ERR_INVALID_ARG
    assert L.mla_out_proj(ctypes.byref(c), 4, FAKE, FAKE, FAKE, 7, None) == br.MLRA_ERR_INVALID_ARG
    assert L.mla_out_proj(ctypes.byref(c), 4, FAKE + 8, FAKE, FAKE, 0, None) == br.MLRA_ERR_INVALID_ARG
    k = cache()
    ws = br.workspace_size(c, 4, 128)
    assert L.mlra_decode(ctypes.byref(c), 3, 4, FAKE, FAKE, None, FAKE, FAKE, ctypes.byref(k),
                         FAKE, ws, FAKE, 0, None) == br.MLRA_ERR_INVALID_ARG
    assert L.mlra_decode(ctypes.byref(c), 4, 4, FAKE, FAKE, None, FAKE, FAKE, ctypes.byref(k),
                         FAKE, 8, FAKE, 0, None) == br.MLRA_ERR_WORKSPACE
    # the no-allocation step validates like mlra_decode
    assert L.mlra_decode_noalloc(ctypes.byref(c), 3, 4, FAKE, FAKE, None, FAKE, FAKE,
                                 ctypes.byref(k), FAKE, 0, None) == br.MLRA_ERR_INVALID_ARG
    assert L.mlra_decode_noalloc(ctypes.byref(c), 4, 4, FAKE, FAKE, None, FAKE, FAKE,
                                 ctypes.byref(k), 0, 0, None) == br.MLRA_ERR_INVALID_ARG
    assert L.mlra_decode_noalloc(ctypes.byref(c), 4, 4, FAKE, FAKE, None, FAKE, FAKE,
                                 ctypes.byref(k), FAKE, 9, None) == br.MLRA_ERR_INVALID_ARG
    assert L.mlra_decode_noalloc(ctypes.byref(c), 4, 0, FAKE, FAKE, None, FAKE, FAKE,
                                 ctypes.byref(k), FAKE, 0, None) == br.MLRA_OK
    assert L.mlra_set_kernel_timing(FAKE, None) == br.MLRA_ERR_INVALID_ARG
    assert L.mlra_set_kernel_timing(None, None) == br.MLRA_OK


def append(c, rows=FAKE, gain=None, eps=1e-6, ckv=FAKE, kr=FAKE, ts=576, kts=576, lens=FAKE,
           B=4, max_len=128):
    return br.lib().mlra_cache_append(ctypes.byref(c), B, rows, gain, eps, ckv, kr, 128 * 576, ts,
                                      128 * 576, kts, lens, max_len, None)


def test_cache_append_validation():
    c = cfg()
    assert append(c, rows=0) == br.MLRA_ERR_INVALID_ARG
    assert append(c, lens=0) == br.MLRA_ERR_INVALID_ARG
    assert append(c, ckv=0) == br.MLRA_ERR_INVALID_ARG
    assert append(c, kr=0) == br.MLRA_ERR_INVALID_ARG
    assert append(c, eps=-1.0) == br.MLRA_ERR_INVALID_ARG
    assert append(c, eps=float("nan")) == br.MLRA_ERR_INVALID_ARG
    assert append(c, ts=100) == br.MLRA_ERR_INVALID_ARG       # token stride below d_latent
    assert append(c, kts=10) == br.MLRA_ERR_INVALID_ARG       # below d_rope
    assert append(c, B=-1) == br.MLRA_ERR_INVALID_ARG
    assert append(c, max_len=-1) == br.MLRA_ERR_INVALID_ARG
    # nothing to do: succeeds without a device
    assert append(c, B=0) == br.MLRA_OK
    assert append(c, max_len=0) == br.MLRA_OK
    # a RoPE-free config needs no krope buffer
    assert append(cfg(d_rope=0), kr=0, kts=0) in (br.MLRA_OK, br.MLRA_ERR_NO_DEVICE)


def prefill(c, n=4, q=FAKE, out=FAKE, od=0, k=None, B=4):
    k = cache() if k is None else k
    return br.lib().mlra_prefill(ctypes.byref(c), n, B, q, FAKE, FAKE, FAKE, ctypes.byref(k), out,
                                 od, None)


def test_prefill_validation():
    c = cfg()
    assert prefill(c, n=3) == br.MLRA_ERR_INVALID_ARG             # 3 does not divide d_latent
    assert prefill(c, n=1) == br.MLRA_ERR_UNSUPPORTED              # MLA: no prefill kernel
    assert prefill(cfg(dtype="fp32")) == br.MLRA_ERR_UNSUPPORTED
    assert prefill(cfg(d_rope=32)) == br.MLRA_ERR_UNSUPPORTED
    assert prefill(cfg(d_v=64)) == br.MLRA_ERR_UNSUPPORTED
    assert prefill(c, q=0) == br.MLRA_ERR_INVALID_ARG
    assert prefill(c, out=0) == br.MLRA_ERR_INVALID_ARG
    assert prefill(c, out=FAKE + 4) == br.MLRA_ERR_INVALID_ARG      # 16-byte alignment
    assert prefill(c, od=7) == br.MLRA_ERR_INVALID_ARG
    assert prefill(c, k=cache(ckv=0)) == br.MLRA_ERR_INVALID_ARG
    assert prefill(c, B=-1) == br.MLRA_ERR_INVALID_ARG
    big = cache(max_len=65536, bs=576 * 65536)
    assert prefill(c, k=big, B=65) == br.MLRA_ERR_UNSUPPORTED        # over 2^22 prompt rows
    # nothing to do: succeeds without a device
    assert prefill(c, B=0) == br.MLRA_OK
    assert prefill(c, k=cache(max_len=0)) == br.MLRA_OK


@pytest.mark.skipif(gpu_present(), reason="valid arguments would launch on a real device")
def test_valid_arguments_without_device_report_no_device():
    c = cfg()
    assert decode(c, cache()) == br.MLRA_ERR_NO_DEVICE
    L = br.lib()
    assert L.mla_out_proj(ctypes.byref(c), 4, FAKE, FAKE, FAKE, 0, None) == br.MLRA_ERR_NO_DEVICE
    assert append(c) == br.MLRA_ERR_NO_DEVICE
    assert prefill(c) == br.MLRA_ERR_NO_DEVICE
    k = cache()
    assert L.mlra_decode_noalloc(ctypes.byref(c), 4, 4, FAKE, FAKE, None, FAKE, FAKE,
                                 ctypes.byref(k), FAKE, 0, None) == br.MLRA_ERR_NO_DEVICE


def test_read_probe_library_exports_and_validates():
    # the benchmark's read-ceiling probe (include/mlra_probe.h): its own
    # library; invalid arguments are refused before any HIP call
    path = os.path.join(ROOT, "branch_rank_amd", "libmlra_probe.so")
    L = ctypes.CDLL(path)
    text = open(os.path.join(ROOT, "include", "mlra_probe.h")).read()
    names = re.findall(r"MLRA_PROBE_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)
    assert names == ["mlra_probe_read"]
    f = L.mlra_probe_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    n = 1 << 20
    assert f(None, n, 0, 256, 4, 4, FAKE, None) == -1           # null buffer
    assert f(FAKE + 4, n, 0, 256, 4, 4, FAKE, None) == -1       # misaligned
    assert f(FAKE, n, 0, 256, 4, 4, None, None) == -1           # null sink
    assert f(FAKE, n + 16, 0, 256, 4, 4, FAKE, None) == -1      # not 1 KB per workgroup
    assert f(FAKE, n, 0, 256, 17, 4, FAKE, None) == -1          # > 16 waves
    assert f(FAKE, n, 0, 256, 4, 3, FAKE, None) == -1           # depth not offered
    assert f(FAKE, n, 1, 256, 4, 5, FAKE, None) == -1
    assert f(FAKE, n, 2, 256, 4, 4, FAKE, None) == -1           # unknown mode


def test_q_residue_validation_and_row_width():
    out = ctypes.c_size_t(0)
    L = br.lib()
    c = cfg(q_residue=True)
    assert L.mlra_workspace_size(ctypes.byref(c), 4, 128, ctypes.byref(out)) == br.MLRA_OK
    assert br.q_abs_width(c) == 512 + 64 + 512
    assert br.q_abs_width(cfg()) == 512 + 64
    c.q_residue = 2
    assert L.mlra_workspace_size(ctypes.byref(c), 4, 128, ctypes.byref(out)) == br.MLRA_ERR_INVALID_ARG
    c = cfg(q_residue=True, dtype="fp32")   # the residue is a bf16 notion
    assert L.mlra_workspace_size(ctypes.byref(c), 4, 128, ctypes.byref(out)) == br.MLRA_ERR_INVALID_ARG


# ---- fp8 (E4M3) caches: validation and kernel choice, host only ----

def _fp8_cache(c, batch, max_len, sc=0.01, sr=0.02, fp8=1, ts=None):
    ts = c.d_latent + c.d_rope if ts is None else ts  # bytes
    k = br.Cache(0x100000, 0x100000 + c.d_latent, max_len * ts, ts, max_len * ts, ts,
                 0x200000, max_len, fp8, sc, sr)
    k._batch = batch
    return k


@pytest.mark.parametrize("kw,kernel,expect", [
    (dict(), "auto", "branch"),                    # MLRA-4, 128 heads
    (dict(n=1), "auto", "wide"),                   # MLA
    (dict(heads=64), "auto", "portable"),          # MLRA-4 at 64 heads: no fp8 MFMA kernel
    (dict(n=2), "auto", "portable"),
    (dict(n=1, d_latent=128), "auto", "portable"),  # one branch shard
    (dict(), "portable", "portable"),
])
def test_fp8_kernel_selection(kw, kernel, expect):
    c = cfg(kernel=kernel, **kw)
    assert br.select_decode_kernel(c, _fp8_cache(c, 2, 4096)) == expect


def test_fp8_head_group_is_unsupported():
    c = cfg(kernel="head_group", n=2)
    with pytest.raises(br.MlraError) as e:
        br.select_decode_kernel(c, _fp8_cache(c, 2, 4096))
    assert e.value.status == br.MLRA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,cache_kw", [
    (dict(dtype="fp32"), dict()),                  # fp8 needs bf16 queries and weights
    (dict(), dict(sc=0.0)),
    (dict(), dict(sr=-1.0)),
    (dict(), dict(sc=float("inf"))),
    (dict(), dict(sc=float("nan"))),
    (dict(), dict(sr=2.0 ** 40)),
    (dict(), dict(fp8=2)),
    (dict(), dict(ts=584)),                        # byte stride not a multiple of 16
])
def test_fp8_cache_validation(kw, cache_kw):
    c = cfg(**kw)
    k = _fp8_cache(c, 4, 128, **cache_kw)
    assert decode(c, k) == br.MLRA_ERR_INVALID_ARG


def test_fp8_byte_strides_accepted():
    c = cfg()
    k = _fp8_cache(c, 4, 128)  # 576-byte rows: a multiple of 16 bytes
    out = ctypes.c_int(-1)
    assert br.lib().mlra_select_decode_kernel(ctypes.byref(c), 4, ctypes.byref(k),
                                              ctypes.byref(out)) == br.MLRA_OK


def test_fp8_prefill_is_unsupported():
    c = cfg()
    k = _fp8_cache(c, 2, 128)
    assert br.lib().mlra_prefill(ctypes.byref(c), 4, 2, FAKE, FAKE, FAKE, FAKE, ctypes.byref(k),
                                 FAKE, br.MLRA_FP32, None) == br.MLRA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,sc,sr", [(dict(dtype="fp32"), 0.1, 0.1), (dict(), 0.0, 0.1),
                                      (dict(), 0.1, float("inf")), (dict(), 2.0 ** -40, 0.1)])
def test_fp8_append_validation(kw, sc, sr):
    c = cfg(**kw)
    L = br.lib()
    assert L.mlra_cache_append_fp8(ctypes.byref(c), 2, FAKE, None, 1e-6, FAKE, FAKE, 576 * 8,
                                   576, 576 * 8, 576, FAKE, 8, sc, sr, None) == \
        br.MLRA_ERR_INVALID_ARG


# ---- mla_prefill (MLA in the unabsorbed form), host only ----

def test_mla_prefill_workspace_size():
    c = cfg(n=1)
    n = br.mla_prefill_workspace_size(c, 4, 4096)
    assert n >= 2 * 4 * 4096 * (256 * 128 + 64)
    assert br.mla_prefill_workspace_size(c, 0, 4096) == 0


@pytest.mark.parametrize("kw,expect", [(dict(n=1, dtype="fp32"), br.MLRA_ERR_UNSUPPORTED),
                                       (dict(n=1, d_latent=256), br.MLRA_ERR_UNSUPPORTED),
                                       (dict(n=1, d_v=64), br.MLRA_ERR_UNSUPPORTED)])
def test_mla_prefill_unsupported_shapes(kw, expect):
    c = cfg(**kw)
    k = br.Cache(FAKE, FAKE + 1024, 576 * 128, 576, 576 * 128, 576, FAKE, 128)
    assert br.lib().mla_prefill(ctypes.byref(c), 2, FAKE, FAKE, FAKE, FAKE, ctypes.byref(k),
                                FAKE, 1 << 40, FAKE, br.MLRA_FP32, None) == expect


def test_mla_prefill_workspace_checked():
    c = cfg(n=1)
    k = br.Cache(FAKE, FAKE + 1024, 576 * 128, 576, 576 * 128, 576, FAKE, 128)
    L = br.lib()
    assert L.mla_prefill(ctypes.byref(c), 2, FAKE, FAKE, FAKE, FAKE, ctypes.byref(k), FAKE, 1024,
                         FAKE, br.MLRA_FP32, None) == br.MLRA_ERR_WORKSPACE
    assert L.mla_prefill(ctypes.byref(c), 2, FAKE, FAKE, FAKE, FAKE, ctypes.byref(k), FAKE + 16,
                         1 << 40, FAKE, br.MLRA_FP32, None) == br.MLRA_ERR_INVALID_ARG
