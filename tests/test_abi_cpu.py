"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments synchronously without touching a
GPU (every call here returns before any HIP call)."""
import ctypes
import os
import re

import pytest

import bit_moe_amd as bm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitmoe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bm.LIB_PATH):
        from bit_moe_amd import build
        build.build()
    return bm.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("moe_route", "moe_expert_ffn", "engram_gather", "bitmoe_workspace_size"):
        assert n in names
    assert sorted(names) == sorted(bm.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def _layer(**kw):
    fake = 0x10000  # 16-byte aligned host value; never dereferenced by validation
    base = dict(d_model=4096, d_ff=2048, n_experts=384, top_k=6, wfmt=bm.WFMT_Q2SB, shared_wfmt=bm.WFMT_Q8_0,
                w_gate=fake, w_up=fake, w_down=fake, w_router=fake, ws_gate=fake, ws_up=fake, ws_down=fake)
    base.update(kw)
    return bm._LayerC(**base)


def _ws_size(lib, layer, T, mode=bm.MODE_AUTO):
    n = ctypes.c_size_t(0)
    rc = lib.bitmoe_workspace_size(ctypes.byref(layer), T, mode, ctypes.byref(n))
    return rc, n.value


def test_workspace_size_valid_layer(lib):
    rc, n = _ws_size(lib, _layer(), 1)
    assert rc == bm.OK and n > 0
    rc5, n5 = _ws_size(lib, _layer(), 5)
    assert rc5 == bm.OK and n5 > n
    rcp, npf = _ws_size(lib, _layer(), 4096)
    assert rcp == bm.OK and npf > 4096 * 6 * 4096 * 4  # holds the per-pair outputs


@pytest.mark.parametrize("field,value,code", [
    ("d_model", 300, bm.EUNSUPPORTED), ("d_model", 8192, bm.EUNSUPPORTED), ("d_ff", 96, bm.EUNSUPPORTED),
    ("d_model", 3072, bm.EUNSUPPORTED), ("d_ff", 1536, bm.EUNSUPPORTED),  # multiples of 256, not powers of two
    ("n_experts", 0, bm.EUNSUPPORTED), ("n_experts", 2000, bm.EUNSUPPORTED), ("top_k", 0, bm.EINVAL),
    ("top_k", 9, bm.EINVAL), ("wfmt", 7, bm.EUNSUPPORTED), ("shared_wfmt", 5, bm.EUNSUPPORTED),
    ("w_gate", 0, bm.EINVAL), ("w_up", 0x10004, bm.EINVAL), ("w_router", 0, bm.EINVAL), ("ws_down", 0, bm.EINVAL),
    ("layout_flags", 1, bm.EUNSUPPORTED), ("layout_flags", -1, bm.EUNSUPPORTED),
])
def test_layer_validation(lib, field, value, code):
    rc, _ = _ws_size(lib, _layer(**{field: value}), 1)
    assert rc == code
    assert lib.bitmoe_last_error().decode()  # a named message


def test_topk_above_experts_rejected(lib):
    rc, _ = _ws_size(lib, _layer(n_experts=4, top_k=6), 1)
    assert rc == bm.EINVAL and b"top_k" in lib.bitmoe_last_error()


def test_route_rejects_bad_args(lib):
    L = _layer()
    P = ctypes.c_void_p
    assert lib.moe_route(None, P(0x10000), bm.BF16, 1, None, P(0x10000), P(0x10000), P(0x10000), 1 << 30,
                         None) == bm.EINVAL
    assert lib.moe_route(ctypes.byref(L), None, bm.BF16, 1, None, P(0x10000), P(0x10000), P(0x10000), 1 << 30,
                         None) == bm.EINVAL
    assert lib.moe_route(ctypes.byref(L), P(0x10000), 7, 1, None, P(0x10000), P(0x10000), P(0x10000), 1 << 30,
                         None) == bm.EUNSUPPORTED
    # workspace too small
    assert lib.moe_route(ctypes.byref(L), P(0x10000), bm.BF16, 1, None, P(0x10000), P(0x10000), P(0x10000), 64,
                         None) == bm.EWORKSPACE
    # empty batch is a no-op
    assert lib.moe_route(ctypes.byref(L), None, bm.BF16, 0, None, None, None, None, 0, None) == bm.OK
    assert lib.moe_route(ctypes.byref(L), None, bm.BF16, -1, None, None, None, None, 0, None) == bm.EINVAL


def test_route_ex_rejects_bad_args(lib):
    L = _layer()
    P = ctypes.c_void_p
    f = P(0x10000)

    def call(opts, T=1, x=f, ws_bytes=1 << 30):
        return lib.moe_route_ex(ctypes.byref(L), x, bm.BF16, T, None if opts is None else ctypes.byref(opts), f, f,
                                f, ws_bytes, None)

    assert call(None) == bm.EINVAL
    assert call(bm._RouteOptsC(score=5)) == bm.EUNSUPPORTED
    assert call(bm._RouteOptsC(hash_table=0x10000)) == bm.EINVAL  # table without token ids
    assert call(bm._RouteOptsC(hash_table=0x10000, token_ids=0x10000, vocab=0)) == bm.EINVAL
    assert call(bm._RouteOptsC(select_bias=0x10002)) == bm.EINVAL  # misaligned option array
    assert call(bm._RouteOptsC(), ws_bytes=64) == bm.EWORKSPACE
    assert call(bm._RouteOptsC(), x=None) == bm.EINVAL
    assert call(bm._RouteOptsC(), T=0, x=None) == bm.OK


def test_engram_inject_rejects_bad_args(lib):
    f = ctypes.c_void_p(0x10000)
    n = ctypes.c_size_t(0)
    assert lib.engram_inject_workspace_size(5, 4096, ctypes.byref(n)) == bm.OK and n.value >= 5 * 5 * 4096 * 4
    assert lib.engram_inject_workspace_size(5, 300, ctypes.byref(n)) == bm.EINVAL

    def call(T=5, n_rows=8, W=4096, eps=1e-6, rows=f, qn=f, ws_bytes=1 << 30):
        return lib.engram_inject(rows, T, n_rows, f, W, qn, f, ctypes.c_float(eps), None, f, None, f, ws_bytes, None)

    assert call(n_rows=7) == bm.EUNSUPPORTED
    assert call(n_rows=34) == bm.EUNSUPPORTED
    assert call(W=4000) == bm.EUNSUPPORTED
    assert call(eps=-1.0) == bm.EINVAL
    assert call(rows=None) == bm.EINVAL
    assert call(rows=ctypes.c_void_p(0x10008)) == bm.EINVAL
    assert call(qn=ctypes.c_void_p(0x10004)) == bm.EINVAL  # the norm weights are read 16 bytes at a time
    assert call(ws_bytes=1024) == bm.EWORKSPACE
    assert call(T=0, rows=None) == bm.OK
    assert call(T=-1) == bm.EINVAL


def test_expert_ffn_rejects_bad_args(lib):
    L = _layer()
    P = ctypes.c_void_p
    args = lambda **k: [ctypes.byref(L), k.get("x", P(0x10000)), bm.BF16, k.get("T", 1), P(0x10000), P(0x10000),
                        k.get("y", P(0x10000)), k.get("yd", bm.BF16), k.get("mode", bm.MODE_AUTO),
                        k.get("ws", P(0x10000)), k.get("wsb", 64), None]
    assert lib.moe_expert_ffn(*args(y=None, wsb=1 << 40)) == bm.EINVAL
    assert lib.moe_expert_ffn(*args(yd=9, wsb=1 << 40)) == bm.EUNSUPPORTED
    assert lib.moe_expert_ffn(*args(mode=5, wsb=1 << 40)) == bm.EINVAL
    assert lib.moe_expert_ffn(*args(wsb=64)) == bm.EWORKSPACE
    assert lib.moe_expert_ffn(*args(ws=P(0x10010), wsb=1 << 40)) == bm.EINVAL  # not 256-aligned
    assert lib.moe_expert_ffn(*args(T=9, mode=bm.MODE_DECODE, wsb=1 << 40)) == bm.EUNSUPPORTED
    assert lib.moe_expert_ffn(*args(T=9, mode=bm.MODE_DECODE_INT8, wsb=1 << 40)) == bm.EUNSUPPORTED
    assert lib.moe_expert_ffn(*args(mode=6, wsb=1 << 40)) == bm.EINVAL  # 4 is MODE_PREFILL_INT8
    assert lib.moe_expert_ffn(*args(mode=bm.MODE_DECODE_INT8, wsb=64)) == bm.EWORKSPACE
    assert lib.moe_expert_ffn(*args(T=0, x=None, y=None)) == bm.OK


def test_layer_residual_rejects_bad_args(lib):
    # moe_layer_residual checks the layer, x_next and its aliasing before
    # anything reaches moe_layer's launches
    P = ctypes.c_void_p
    args = lambda L=None, **k: [ctypes.byref(L or _layer()), P(0x10000), k.get("T", 1), None, P(0x10000),
                                P(0x10000), k.get("y", P(0x20000)), bm.BF16, k.get("xn", P(0x30000)), bm.MODE_AUTO,
                                P(0x10000), 1 << 40, None]
    assert lib.moe_layer_residual(*args(xn=None)) == bm.EINVAL
    assert lib.moe_layer_residual(*args(xn=P(0x30008))) == bm.EINVAL  # not 16-byte aligned
    assert lib.moe_layer_residual(*args(xn=P(0x20000))) == bm.EINVAL  # aliases y
    assert lib.moe_layer_residual(*args(L=_layer(top_k=400))) == bm.EINVAL
    assert lib.moe_layer_residual(*args(T=-1)) == bm.EINVAL
    assert lib.moe_layer_residual(*args(T=0, xn=None)) == bm.OK


def test_engram_gather_tables_rejects_bad_args(lib):
    P = ctypes.c_void_p
    tabs = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    rows = (ctypes.c_int64 * 2)(1 << 22, 1 << 22)
    call = lambda t=tabs, r=rows, nt=2, ids=P(0x30000), g=5, per=8, out=P(0x40000), st=None: \
        lib.engram_gather_tables(t, r, nt, ids, g, per, out, st, None)
    assert call(nt=0) == bm.EINVAL
    assert call(nt=5) == bm.EINVAL
    assert call(t=None) == bm.EINVAL
    assert call(t=(ctypes.c_void_p * 2)(0x10000, 0x20004)) == bm.EINVAL  # table 1 not 8-byte aligned
    assert call(r=(ctypes.c_int64 * 2)(1, -1)) == bm.EINVAL
    assert call(per=0) == bm.EINVAL
    assert call(g=-1) == bm.EINVAL
    assert call(ids=None) == bm.EINVAL
    assert call(out=P(0x40008)) == bm.EINVAL
    assert call(st=P(0x50004)) == bm.EINVAL
    assert call(g=1 << 40) == bm.EUNSUPPORTED
    assert call(g=0, ids=None, out=None) == bm.OK


def test_int8_mode_workspace_and_shape_limits(lib):
    L = _layer()
    n8, n1 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.bitmoe_workspace_size(ctypes.byref(L), 5, bm.MODE_DECODE_INT8, ctypes.byref(n8)) == bm.OK
    assert lib.bitmoe_workspace_size(ctypes.byref(L), 5, bm.MODE_DECODE, ctypes.byref(n1)) == bm.OK
    # float32 h in place of its two bf16 parts: the same size
    assert n8.value == n1.value
    assert lib.bitmoe_workspace_size(ctypes.byref(L), 5, 6, ctypes.byref(n8)) == bm.EINVAL
    # the int8 mode needs d_ff >= 256 (two 16-value halves per 32-value block of h, whole super-blocks per row)
    Ls = _layer(d_ff=128)
    P = ctypes.c_void_p
    f = P(0x10000)
    assert lib.moe_expert_ffn(ctypes.byref(Ls), f, bm.BF16, 1, f, f, f, bm.BF16, bm.MODE_DECODE_INT8, f, 1 << 40,
                              None) == bm.EUNSUPPORTED


def test_quantize_rejects_bad_args(lib):
    P = ctypes.c_void_p
    f = P(0x10000)
    assert lib.moe_quantize_q8_1(f, bm.BF16, 4, 48, f, f, f, None) == bm.EINVAL  # cols not a multiple of 32
    assert lib.moe_quantize_q8_1(f, bm.BF16, 4, 0, f, f, f, None) == bm.EINVAL
    assert lib.moe_quantize_q8_1(f, 7, 4, 64, f, f, f, None) == bm.EUNSUPPORTED
    assert lib.moe_quantize_q8_1(None, bm.BF16, 4, 64, f, f, f, None) == bm.EINVAL
    assert lib.moe_quantize_q8_1(f, bm.BF16, 4, 64, P(0x10004), f, f, None) == bm.EINVAL  # q misaligned
    assert lib.moe_quantize_q8_1(f, bm.F32, -1, 64, f, f, f, None) == bm.EINVAL
    assert lib.moe_quantize_q8_1(None, bm.F32, 0, 64, None, None, None, None) == bm.OK


def test_engram_gather_rejects_bad_args(lib):
    P = ctypes.c_void_p
    assert lib.engram_gather(P(0x10000), 10, P(0x10000), 0, None, None, None) == bm.OK  # empty
    assert lib.engram_gather(None, 10, P(0x10000), 4, P(0x10000), None, None) == bm.EINVAL
    assert lib.engram_gather(P(0x10004), 10, P(0x10000), 4, P(0x10000), None, None) == bm.EINVAL
    assert lib.engram_gather(P(0x10000), 10, P(0x10000), 4, P(0x10008), None, None) == bm.EINVAL
    assert lib.engram_gather(P(0x10000), 10, P(0x10000), -1, P(0x10000), None, None) == bm.EINVAL


def test_dequant_and_fill_reject_bad_args(lib):
    P = ctypes.c_void_p
    assert lib.moe_dequant(P(0x10000), 9, 256, P(0x10000), bm.F32, None) == bm.EUNSUPPORTED
    assert lib.moe_dequant(P(0x10000), bm.WFMT_Q2SB, 100, P(0x10000), bm.F32, None) == bm.EINVAL
    assert lib.moe_dequant(P(0x10000), bm.WFMT_Q8_0, 0, P(0x10000), bm.F32, None) == bm.OK
    assert lib.bitmoe_fill(P(0x10000), 85, 1, bm.FILL_Q2, P(0x10000), None) == bm.EINVAL
    assert lib.bitmoe_fill(P(0x10000), 84, 1, bm.FILL_Q2, None, None) == bm.EINVAL
    assert lib.bitmoe_fill(P(0x10000), 84, 1, 9, None, None) == bm.EINVAL


def test_plan_rejects_bad_args(lib):
    P = ctypes.c_void_p
    assert lib.moe_plan(P(0x10000), 4, 2, 0, P(1), P(1), P(1), P(1), P(1), None, P(1), 1 << 20, None) == bm.EINVAL
    assert lib.moe_plan(P(0x10000), 4, 2, 16, None, P(1), P(1), P(1), P(1), None, P(1), 1 << 20, None) == bm.EINVAL
    assert lib.moe_plan(P(0x10000), 4, 2, 16, P(1), P(1), P(1), P(1), P(1), None, P(1), 0, None) == bm.EWORKSPACE


def test_strerror_names_every_code(lib):
    for code in (bm.OK, bm.EINVAL, bm.EUNSUPPORTED, bm.EWORKSPACE, bm.EHIP, bm.EDEVICE):
        assert lib.bitmoe_strerror(code).startswith(b"BITMOE_")


def test_residual_rescale_rejects_bad_args(lib):
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert lib.bitmoe_residual_rescale(fake, fake, bm.BF16, 4, 4097, fake, None) == bm.EINVAL
    assert lib.bitmoe_residual_rescale(fake, fake, bm.BF16, 4, 8, fake, None) == bm.EINVAL
    assert lib.bitmoe_residual_rescale(fake, fake, 7, 4, 4096, fake, None) == bm.EUNSUPPORTED
    assert lib.bitmoe_residual_rescale(None, fake, bm.BF16, 4, 4096, fake, None) == bm.EINVAL
    assert lib.bitmoe_residual_rescale(None, None, bm.BF16, 0, 4096, None, None) == bm.OK
    assert lib.bitmoe_residual_rescale(ctypes.c_void_p((1 << 20) + 4), fake, bm.F32, 4, 4096, fake, None) == bm.EINVAL
    assert lib.bitmoe_residual_rescale(fake, fake, bm.F32, -1, 4096, fake, None) == bm.EINVAL


def test_build_rejects_spilling_kernels():
    # the build parses the compiler's resource report and refuses spills
    from bit_moe_amd import build as b
    report = "\n".join([
        "x.hip:1:1: remark: Function Name: k_ok [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark: Function Name: k_bad [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     SGPRs Spill: 30 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
    ])
    bad = b._spills(report)
    assert bad == ["k_bad: SGPRs Spill 30", "k_bad: ScratchSize [bytes/lane] 12"]
