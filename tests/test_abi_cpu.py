"""The C-ABI library on the host (no GPU): it loads, exports every function include/mimo_attn.h
declares, and rejects every invalid argument with its code before anything is enqueued."""
import ctypes
import os
import re

import pytest

import global_attention_rope_amd as mimo
from global_attention_rope_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("mimo_attn.h", "mimo_router.h")]


def _declared_functions():
    names = set()
    for hdr in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
        names |= set(re.findall(r"\b(mimo_(?:attn|router)_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 7
    lib = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in mimo_attn.h but not exported"
    assert set(names) == set(binding.EXPORTS)
    assert mimo.lib().mimo_attn_abi_version() == 2


def test_probe_library_exports_its_declared_functions():
    """The latency-reference library beside the layer's (a measurement aid) loads and exports what
    include/mimo_probe.h declares."""
    from global_attention_rope_amd import build as hb
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mimo_probe.h")).read(),
                  flags=re.S)
    names = set(re.findall(r"\b(mimo_probe_\w+)\s*\(", text))
    assert names == {"mimo_probe_empty", "mimo_probe_tile_read", "mimo_probe_stream_read",
                     "mimo_probe_mfma"}
    lib = ctypes.CDLL(hb.PROBE_LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_arguments_checked_before_any_launch():
    """The ceiling probes reject NULL buffers, empty grids and bad sizes on the host (no device call
    is made, so this runs without a GPU)."""
    from global_attention_rope_amd import build as hb
    lib = ctypes.CDLL(hb.PROBE_LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mimo_probe_stream_read.argtypes = [vp, i64, i32, vp, i32, vp]
    lib.mimo_probe_mfma.argtypes = [vp, i32, i32, vp]
    fake = vp(0x1000)
    assert lib.mimo_probe_stream_read(None, 1 << 20, 0, fake, 8, None) == -1
    assert lib.mimo_probe_stream_read(fake, 1 << 20, 0, None, 8, None) == -1
    assert lib.mimo_probe_stream_read(fake, 1 << 20, 1, fake, 0, None) == -1
    for bad in (0, 8, (1 << 20) + 4):
        assert lib.mimo_probe_stream_read(fake, bad, 0, fake, 8, None) == -2
    assert lib.mimo_probe_stream_read(fake, 3 * 4096, 2, fake, 2, None) == -2   # uneven slices
    assert lib.mimo_probe_mfma(None, 8, 10, None) == -1
    assert lib.mimo_probe_mfma(fake, 0, 10, None) == -1
    assert lib.mimo_probe_mfma(fake, 8, 0, None) == -2


def _swa(**kw):
    d = dict(batch=1, num_q_heads=64, num_kv_heads=8, qk_head_dim=192, v_head_dim=128,
             rope_dims=64, layer_kind=mimo.LAYER_SWA, window=128, rope_theta=1e4,
             v_scale=0.70710678, dtype=mimo.BF16)
    d.update(kw)
    return mimo.Params(**d)


def _ga(**kw):
    d = dict(num_kv_heads=4, layer_kind=mimo.LAYER_GLOBAL, window=0, rope_theta=5e6)
    d.update(kw)
    return _swa(**d)


@pytest.mark.parametrize("p", [_swa(), _ga(), _swa(rope_dims=0), _ga(rope_dims=192),
                               _swa(dtype=mimo.F32, qk_head_dim=32, v_head_dim=16, rope_dims=10,
                                    num_q_heads=4, num_kv_heads=1, window=16),
                               _ga(batch=0)])
def test_valid_params(p):
    assert mimo.check_params(p) == mimo.MIMO_OK, mimo.last_error()
    assert mimo.last_error() == ""


@pytest.mark.parametrize("p,code", [
    (_swa(rope_dims=63), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(rope_dims=194), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(rope_dims=-2), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(num_kv_heads=7), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(num_kv_heads=0), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(window=0), mimo.MIMO_ERR_INVALID_ARG),
    (_ga(window=128), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(layer_kind=2), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(rope_theta=0.0), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(rope_theta=float("inf")), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(v_scale=float("nan")), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(softmax_scale=-1.0), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(batch=-1), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(dtype=7), mimo.MIMO_ERR_INVALID_ARG),
    (_swa(qk_head_dim=128), mimo.MIMO_ERR_UNSUPPORTED),
    (_swa(v_head_dim=192), mimo.MIMO_ERR_UNSUPPORTED),
    (_swa(rope_dims=40), mimo.MIMO_ERR_UNSUPPORTED),
    (_swa(dtype=mimo.F32, qk_head_dim=512), mimo.MIMO_ERR_UNSUPPORTED),
])
def test_invalid_params_rejected_with_code_and_message(p, code):
    assert mimo.check_params(p) == code
    assert mimo.last_error() != ""


def test_cache_dtype_and_scales_are_checked():
    fp8 = dict(cache_dtype=mimo.CACHE_FP8_E4M3, k_cache_scale=0.05, v_cache_scale=2.0)
    assert mimo.check_params(_swa(**fp8)) == mimo.MIMO_OK
    assert mimo.check_params(_ga(**fp8)) == mimo.MIMO_OK
    cp = _swa().c()
    cp.cache_dtype = 1
    assert mimo.lib().mimo_attn_check_params(ctypes.byref(cp)) == mimo.MIMO_ERR_INVALID_ARG
    assert mimo.lib().mimo_attn_check_params(None) == mimo.MIMO_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert mimo.check_params(_swa(**dict(fp8, k_cache_scale=bad))) == mimo.MIMO_ERR_INVALID_ARG
        assert mimo.check_params(_swa(**dict(fp8, v_cache_scale=bad))) == mimo.MIMO_ERR_INVALID_ARG
    # scales are ignored for caches of the layer dtype
    assert mimo.check_params(_swa(k_cache_scale=0.0)) == mimo.MIMO_OK
    # fp8 caches belong to bf16 layers
    assert mimo.check_params(_swa(dtype=mimo.F32, qk_head_dim=32, v_head_dim=16, rope_dims=10,
                                  num_q_heads=4, num_kv_heads=1, window=16, **fp8)) == \
        mimo.MIMO_ERR_UNSUPPORTED
    # extend over fp8 caches lays their rows out widened in its workspace (global layers too)
    assert _extend(_swa(**fp8), ws=None) == mimo.MIMO_ERR_WORKSPACE
    assert _extend(_ga(**fp8), ws=None, cap=200) == mimo.MIMO_ERR_WORKSPACE
    assert mimo.extend_workspace_size(_ga(batch=2, **fp8), 1000, 5000) == \
        2 * 4 * (5000 + 1000) * (192 + 128) * 2
    assert mimo.extend_workspace_size(_swa(batch=2, **fp8), 1000, 5000) == \
        mimo.extend_workspace_size(_swa(batch=2), 1000, 5000)
    # an fp8 cache slice may be twice as long as a bf16 one under the 4 GiB bound
    # (passes the bound, then stops at the missing workspace: nothing is launched)
    assert _decode(_ga(**fp8), maxp=100_000, cap=12_000_000, ws=None) == mimo.MIMO_ERR_WORKSPACE
    assert _decode(_ga(**fp8), maxp=10, cap=23_000_000) == mimo.MIMO_ERR_UNSUPPORTED


def test_workspace_sizes():
    assert mimo.prefill_workspace_size(_swa(), 4096) == 1 * 8 * 4096 * 192 * 2
    assert mimo.prefill_workspace_size(_swa(dtype=mimo.F32, qk_head_dim=32, v_head_dim=16, rope_dims=10,
                                            num_q_heads=4, num_kv_heads=1, window=16), 64) == 0
    assert mimo.prefill_workspace_size(_ga(), 8192) == 1 * 4 * 8192 * 192 * 2
    assert mimo.prefill_workspace_size(_ga(rope_dims=63), 8192) == 0  # invalid -> 0
    # the 128-slot ring fits one split: no partials
    assert mimo.decode_workspace_size(_swa(batch=64), 40000) == 0
    ws = mimo.decode_workspace_size(_ga(batch=64), 32768)
    assert ws > 0 and ws % (64 * 64 * 130 * 4) == 0
    assert mimo.decode_workspace_size(_ga(batch=64), 100) == 0
    # more (sequence, KV head) pairs than the split policy's grid budget: one split each
    assert mimo.decode_workspace_size(_ga(batch=2048), 2000) == 0
    assert mimo.decode_workspace_size(_ga(batch=1100, cache_dtype=mimo.CACHE_FP8_E4M3), 70000) == 0
    # extend: sliding layers lay out window + S rows of K and V; global layers read a bf16 cache
    assert mimo.extend_workspace_size(_swa(batch=2), 1000, 5000) == 2 * 8 * (128 + 1000) * (192 + 128) * 2
    assert mimo.extend_workspace_size(_ga(batch=2), 1000, 5000) == 0
    assert mimo.extend_workspace_size(_swa(), -1, 0) == 0
    assert mimo.extend_workspace_size(_swa(), 4, -1) == 0
    # a few new tokens: the multi-token tile kernel, split partials for long global caches
    assert mimo.extend_workspace_size(_ga(batch=2), 4, 100) == 0
    # 64 sequences x 4 KV heads fill the chip's two workgroups per CU at 2 splits; splits are at
    # most 4096 rows, so 32772 key rows take 9 (of 3648 rows)
    assert mimo.extend_workspace_size(_ga(batch=64), 4, 32768) == 64 * 4 * 64 * 9 * 130 * 4
    assert mimo.extend_workspace_size(_ga(batch=64), 4, 4092) == 64 * 4 * 64 * 2 * 130 * 4
    rows = 8 * (128 + 4) * (192 + 128) * 2
    assert mimo.extend_workspace_size(_swa(), 4, 30000) == (rows + 255) // 256 * 256
    # one sequence, 4 KV heads, 4 tokens after 30000 positions: 30004 key rows in 256-row splits,
    # 118 of them (more than one combine prefetch block of 96 holds)
    assert mimo.extend_workspace_size(_ga(), 4, 30000) == 1 * 4 * 64 * 118 * 130 * 4


_L = None


def _lib():
    global _L
    _L = mimo.lib()
    return _L


def _prefill(p, S=16, q=1, k=1, v=1, sp=1, out=1, kc=None, vc=None, cap=0, ws=None, wsb=0):
    cp = p.c()
    P = ctypes.c_void_p
    ptr = lambda x: None if x is None else P(0x1000 * x)  # never dereferenced: rejected first
    return _lib().mimo_attn_prefill(ctypes.byref(cp), S, ptr(q), ptr(k), ptr(v), ptr(sp), None,
                                    ptr(out), ptr(kc), ptr(vc), cap, ptr(ws), wsb, None)


def _decode(p, maxp=10, q=1, kn=1, vn=1, pos=1, kc=1, vc=1, cap=128, out=1, ws=None, wsb=0):
    cp = p.c()
    P = ctypes.c_void_p
    ptr = lambda x: None if x is None else P(0x1000 * x)
    return _lib().mimo_attn_decode(ctypes.byref(cp), ptr(q), ptr(kn), ptr(vn), ptr(pos), maxp,
                                   ptr(kc), ptr(vc), cap, None, ptr(out), ptr(ws), wsb, None)


def _decode_noalloc(p, maxp=10, q=1, kn=1, vn=1, pos=1, kc=1, vc=1, cap=128, out=1):
    cp = p.c()
    P = ctypes.c_void_p
    ptr = lambda x: None if x is None else P(0x1000 * x)
    return _lib().mimo_attn_decode_noalloc(ctypes.byref(cp), ptr(q), ptr(kn), ptr(vn), ptr(pos),
                                           maxp, ptr(kc), ptr(vc), cap, None, ptr(out), None)


def test_decode_noalloc_limits_checked_before_any_device_call():
    """The allocation-free decode validates like mimo_attn_decode, and rejects partials beyond its
    fixed scratch array with a workspace error, before touching any device."""
    E = mimo.MIMO_ERR_INVALID_ARG
    assert mimo.decode_noalloc_max_bytes() == 32 << 20
    assert _decode_noalloc(_swa(), maxp=-1) == E
    assert _decode_noalloc(_swa(), kc=None) == E
    assert _decode_noalloc(_swa(), cap=100) == E
    assert _decode_noalloc(_ga(), maxp=500, cap=500) == E
    assert _decode_noalloc(_swa(batch=0), q=None) == mimo.MIMO_OK
    # 512 sequences x 4 KV heads over 4096 positions: 2 splits, 34 MB of partials > 32 MiB
    big = _ga(batch=512)
    assert mimo.decode_workspace_size(big, 4095) > mimo.decode_noalloc_max_bytes()
    assert _decode_noalloc(big, maxp=4095, cap=4096) == mimo.MIMO_ERR_WORKSPACE
    assert "scratch" in mimo.last_error()


def _extend(p, S=16, q=1, k=1, v=1, sp=1, maxs=100, out=1, kc=1, vc=1, cap=128, ws=None, wsb=0):
    cp = p.c()
    P = ctypes.c_void_p
    ptr = lambda x: None if x is None else P(0x1000 * x)
    return _lib().mimo_attn_extend(ctypes.byref(cp), S, ptr(q), ptr(k), ptr(v), ptr(sp), maxs,
                                   None, ptr(out), ptr(kc), ptr(vc), cap, ptr(ws), wsb, None)


def test_prefill_argument_errors_return_before_any_launch():
    E = mimo.MIMO_ERR_INVALID_ARG
    assert _prefill(_swa(rope_dims=5)) == E
    assert _prefill(_swa(), S=-1) == E
    assert _prefill(_swa(), q=None) == E
    assert _prefill(_swa(), out=None) == E
    assert _prefill(_swa(), sp=None) == E
    assert _prefill(_swa(), kc=3, vc=None, cap=128) == E
    assert _prefill(_swa(), kc=3, vc=4, cap=64) == E       # ring capacity != window
    assert _prefill(_ga(), kc=3, vc=4, cap=0) == E
    assert _prefill(_ga(), ws=None) == mimo.MIMO_ERR_WORKSPACE
    assert _prefill(_swa(), ws=None) == mimo.MIMO_ERR_WORKSPACE
    assert _prefill(_ga(), S=16, ws=5, wsb=100) == mimo.MIMO_ERR_WORKSPACE
    assert "workspace" in mimo.last_error()
    # nothing to do: success without touching any pointer
    assert _prefill(_swa(), S=0, q=None, k=None, v=None, sp=None, out=None) == mimo.MIMO_OK
    assert _prefill(_swa(batch=0), q=None) == mimo.MIMO_OK


def test_decode_argument_errors_return_before_any_launch():
    E = mimo.MIMO_ERR_INVALID_ARG
    assert _decode(_swa(), maxp=-1) == E
    assert _decode(_swa(), kc=None) == E
    assert _decode(_swa(), pos=None) == E
    assert _decode(_swa(), cap=100) == E                   # ring capacity != window
    assert _decode(_ga(), maxp=500, cap=500) == E          # linear cache too short
    assert _decode(_ga(batch=64), maxp=32768, cap=40000) == mimo.MIMO_ERR_WORKSPACE
    assert _decode(_ga(num_q_heads=68, num_kv_heads=2), cap=40) == mimo.MIMO_ERR_UNSUPPORTED
    assert _decode(_swa(batch=0), q=None) == mimo.MIMO_OK
    # a bf16 cache slice is addressed with a 32-bit byte bound
    assert _decode(_ga(), maxp=10, cap=12_000_000) == mimo.MIMO_ERR_UNSUPPORTED
    assert "4 GiB" in mimo.last_error()


def test_extend_argument_errors_return_before_any_launch():
    E = mimo.MIMO_ERR_INVALID_ARG
    assert _extend(_swa(), S=-1) == E
    assert _extend(_swa(), maxs=-1) == E
    assert _extend(_swa(), kc=None) == E                   # extend reads the cache
    assert _extend(_swa(), vc=None) == E
    assert _extend(_swa(), q=None) == E
    assert _extend(_swa(), sp=None) == E
    assert _extend(_swa(), cap=64) == E                    # ring capacity != window
    assert _extend(_ga(), maxs=100, S=16, cap=115) == E    # linear cache cannot hold 116 positions
    assert "max_start" in mimo.last_error()
    assert _extend(_ga(), maxs=0x7ffffff0, S=100, cap=128) == E   # positions overflow int32
    assert _extend(_swa(), ws=None) == mimo.MIMO_ERR_WORKSPACE
    assert _extend(_swa(), ws=5, wsb=100) == mimo.MIMO_ERR_WORKSPACE
    assert _extend(_swa(dtype=mimo.F32, qk_head_dim=32, v_head_dim=16, rope_dims=10,
                        num_q_heads=4, num_kv_heads=1, window=16), cap=16) == mimo.MIMO_ERR_UNSUPPORTED
    # nothing to do: success without touching any pointer
    assert _extend(_swa(), S=0, q=None, k=None, v=None, sp=None, out=None) == mimo.MIMO_OK
    assert _extend(_ga(batch=0), q=None, cap=116) == mimo.MIMO_OK


def _layer(p, hidden=4096, S=16, x=1, w=1, sp=1, out=1, ws=None, wsb=0, out_dim=4096, kc=None,
           vc=None, cap=0):
    cp = p.c()
    P = ctypes.c_void_p
    ptr = lambda v: None if v is None else P(0x1000 * v)
    return _lib().mimo_attn_layer_prefill(ctypes.byref(cp), hidden, S, ptr(x), ptr(w), ptr(w),
                                          ptr(w), ptr(w), out_dim, ptr(sp), None, ptr(out), ptr(kc),
                                          ptr(vc), cap, ptr(ws), wsb, None)


def test_layer_argument_errors_return_before_any_launch():
    E = mimo.MIMO_ERR_INVALID_ARG
    assert _layer(_swa(), hidden=0) == E
    assert _layer(_swa(), out_dim=0) == E
    assert _layer(_swa(), S=-1) == E
    assert _layer(_swa(), x=None) == E
    assert _layer(_swa(), w=None) == E
    assert _layer(_swa(), ws=None) == mimo.MIMO_ERR_WORKSPACE
    assert "workspace" in mimo.last_error()
    assert _layer(_swa(rope_dims=5)) == E
    assert _layer(_swa(dtype=mimo.F32, qk_head_dim=32, v_head_dim=16, rope_dims=10, num_q_heads=4,
                       num_kv_heads=1, window=16)) == mimo.MIMO_ERR_UNSUPPORTED
    assert _layer(_swa(), S=0, x=None, w=None, sp=None, out=None) == mimo.MIMO_OK
    # cache arguments are checked before anything is enqueued too
    assert _layer(_swa(), kc=1, vc=None, cap=128) == E
    assert _layer(_swa(), kc=1, vc=1, cap=100) == E          # ring capacity != window
    assert _layer(_swa(), kc=1, vc=1, cap=0) == E
    # the projection kernel's shape limits
    assert _layer(_swa(), hidden=100) == mimo.MIMO_ERR_UNSUPPORTED
    assert _layer(_swa(), out_dim=100) == mimo.MIMO_ERR_UNSUPPORTED
    # q, k, v, attention output and the prefill workspace
    T = 2 * 100
    need = mimo.layer_workspace_size(_ga(batch=2), 4096, 100)
    parts = T * (64 * 192 + 4 * 192 + 4 * 128 + 64 * 128) * 2 + mimo.prefill_workspace_size(_ga(batch=2), 100)
    assert parts <= need <= parts + 5 * 256


def test_router_params_are_checked_on_the_host():
    ok = mimo.RouterParams()
    assert mimo.router_check_params(ok, 100) == mimo.MIMO_OK
    E = mimo.MIMO_ERR_INVALID_ARG
    bad = [dict(n_group=3), dict(topk_group=0), dict(topk_group=9), dict(top_k=0),
           dict(top_k=129), dict(routed_scaling_factor=float("inf")), dict(num_experts=256, n_group=256)]
    for kw in bad:
        p = mimo.RouterParams(**kw)
        assert mimo.router_check_params(p, 10) == E, kw
        assert mimo.last_error() != ""
    assert mimo.router_check_params(ok, -1) == E
    U = mimo.MIMO_ERR_UNSUPPORTED
    assert mimo.router_check_params(mimo.RouterParams(num_experts=96, n_group=8), 4) == U
    assert mimo.router_check_params(mimo.RouterParams(n_group=128, num_experts=512, topk_group=4), 4) == U
    cp = ok.c(4)
    cp.reserved = 1
    assert _lib().mimo_router_check_params(ctypes.byref(cp)) == E
    assert _lib().mimo_router_check_params(None) == E
    # missing pointers are rejected before any launch; no tokens: nothing to do
    cp = ok.c(4)
    assert _lib().mimo_router_topk(ctypes.byref(cp), None, None, None, None, None) == E
    cp = ok.c(0)
    assert _lib().mimo_router_topk(ctypes.byref(cp), None, None, None, None, None) == mimo.MIMO_OK
