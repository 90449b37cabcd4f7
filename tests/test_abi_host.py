"""Host-side checks of libmoeq: it loads, exports every entry point declared in
include/moeq.h, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest
import torch

import bit_quantized_moe_top_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moeq.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, DEVICE, LAUNCH = range(6)
FAKE = ctypes.c_void_p(4096)          # a non-null, aligned address never dereferenced


def declared_functions():
    text = open(HEADER).read()
    body = text[text.index('extern "C" {'):]
    text_no_comments = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text_no_comments,
                      flags=re.M)


def test_header_and_binding_agree():
    names = declared_functions()
    assert len(names) == 24
    assert set(names) == set(mq.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(mq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(handle, name), name


def test_version_and_status_strings():
    assert mq.moe_abi_version() == 3
    assert mq.moe_status_string(0) == "ok"
    for s in range(1, 7):
        assert mq.moe_status_string(s) not in ("ok", "unknown status")
    assert mq.moe_status_string(99) == "unknown status"


def test_plan_size_formula():
    for E, R in [(8, 32), (256, 24), (256, 12288), (384, 12288), (1, 0)]:
        max_tiles = (R + 63) // 64 + min(E, R)
        chunks = max(1, (R + 1023) // 1024)
        words = 16 + (E + 1) + 2 * R + E + 2 * max_tiles + chunks * E
        assert mq.moe_plan_size(E, R) == 4 * words
    assert mq.moe_plan_size(0, 5) == 0 and mq.moe_plan_size(4, -1) == 0


def test_argument_errors_are_reported_without_a_gpu():
    L = mq.lib
    N = None
    # route
    assert L.moe_route_topk(N, N, 1, 8, 2, 1, FAKE, FAKE, N) == INVALID
    assert L.moe_route_topk(FAKE, N, 1, 8, 9, 1, FAKE, FAKE, N) == INVALID        # k > E
    assert L.moe_route_topk(FAKE, N, 1, 2048, 2, 1, FAKE, FAKE, N) == UNSUPPORTED  # E > 1024
    assert L.moe_route_topk(FAKE, N, 1, 64, 9, 1, FAKE, FAKE, N) == UNSUPPORTED    # k > 8
    assert L.moe_route_topk(N, N, 0, 8, 2, 1, N, N, N) == OK                        # empty
    # router logits
    assert L.moe_router_logits(FAKE, 1, 4, 24, FAKE, 8, FAKE, N) == UNSUPPORTED        # H % 16
    assert L.moe_router_logits(FAKE, 5, 4, 32, FAKE, 8, FAKE, N) == INVALID            # dtype
    assert L.moe_router_logits(N, 1, 4, 32, FAKE, 8, FAKE, N) == INVALID               # null x
    assert L.moe_router_logits(ctypes.c_void_p(4100), 1, 4, 32, FAKE, 8, FAKE, N) == INVALID
    assert L.moe_router_logits(N, 1, 0, 32, N, 8, N, N) == OK                           # T = 0
    # quant
    assert L.quant_fp8_per_token(FAKE, 1, 4, 12, 12, FAKE, FAKE, N) == UNSUPPORTED  # K % 8
    assert L.quant_fp8_per_token(FAKE, 7, 4, 16, 16, FAKE, FAKE, N) == INVALID      # dtype
    assert L.quant_fp8_per_token(FAKE, 1, 4, 16, 8, FAKE, FAKE, N) == INVALID       # ld < K
    assert L.quant_fp8_per_token(ctypes.c_void_p(4100), 1, 4, 16, 16, FAKE, FAKE, N) == INVALID
    assert L.quant_fp8_per_token(N, 1, 0, 16, 16, N, N, N) == OK
    # FNUZ -> OCP requantization
    assert L.moe_requant_fp8_fnuz(FAKE, FAKE, 4, 12, FAKE, FAKE, N) == UNSUPPORTED    # K % 8
    assert L.moe_requant_fp8_fnuz(N, FAKE, 4, 16, FAKE, FAKE, N) == INVALID           # null
    assert L.moe_requant_fp8_fnuz(FAKE, FAKE, -1, 16, FAKE, FAKE, N) == INVALID       # rows < 0
    assert L.moe_requant_fp8_fnuz(ctypes.c_void_p(4100), FAKE, 4, 16, FAKE, FAKE, N) == INVALID
    assert L.moe_requant_fp8_fnuz(N, N, 0, 16, N, N, N) == OK                          # empty
    # permute
    small = mq.moe_plan_size(8, 32) - 4
    assert L.moe_permute(FAKE, 16, 2, 8, N, N, 0, N, N, FAKE, small, N) == WORKSPACE
    assert L.moe_permute(FAKE, 16, 2, 8, FAKE, N, 64, FAKE, FAKE, FAKE, 1 << 20, N) == INVALID
    assert L.moe_permute(FAKE, 16, 2, 8, FAKE, FAKE, 24, FAKE, FAKE, FAKE, 1 << 20, N) == UNSUPPORTED
    assert L.moe_permute(FAKE, 16, 9, 8, N, N, 0, N, N, FAKE, 1 << 20, N) == UNSUPPORTED
    # fused front end
    big = 1 << 20
    assert L.moe_route_quant_permute(FAKE, N, 4, 8, 2, 1, FAKE, 1, 24, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, big, N) == UNSUPPORTED                  # H % 16
    assert L.moe_route_quant_permute(FAKE, N, 4, 8, 2, 1, FAKE, 5, 32, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, big, N) == INVALID                      # dtype
    assert L.moe_route_quant_permute(FAKE, N, 4, 8, 2, 1, N, 1, 32, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, big, N) == INVALID                      # x null
    assert L.moe_route_quant_permute(FAKE, N, 4, 8, 2, 1, FAKE, 1, 32, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, 64, N) == WORKSPACE
    # pack
    assert L.pack_int4_g128(FAKE, 4, 100, FAKE, FAKE, N) == UNSUPPORTED
    assert L.pack_int4_g128(N, 4, 128, FAKE, FAKE, N) == INVALID
    # read probe: null, misaligned or ragged buffers; zero bytes is a no-op
    assert L.moe_read_bandwidth_probe(N, 1024, FAKE, N) == INVALID
    assert L.moe_read_bandwidth_probe(FAKE, 1000, FAKE, N) == INVALID
    assert L.moe_read_bandwidth_probe(ctypes.c_void_p(FAKE.value + 4), 1024, FAKE, N) == INVALID
    assert L.moe_read_bandwidth_probe(FAKE, 1024, N, N) == INVALID
    assert L.moe_read_bandwidth_probe(N, 0, N, N) == OK
    # tiled order: rows % 16, K % 128, null, misaligned and overlapping buffers
    other = ctypes.c_void_p(FAKE.value + (1 << 20))
    assert L.moe_tile_int4_weights(FAKE, 8, 128, other, N) == UNSUPPORTED
    assert L.moe_tile_int4_weights(FAKE, 16, 100, other, N) == UNSUPPORTED
    assert L.moe_tile_int4_weights(FAKE, -16, 128, other, N) == INVALID
    assert L.moe_tile_int4_weights(N, 16, 128, other, N) == INVALID
    assert L.moe_tile_int4_weights(FAKE, 16, 128, ctypes.c_void_p(FAKE.value + 8), N) == INVALID
    assert L.moe_tile_int4_weights(FAKE, 16, 128, ctypes.c_void_p(FAKE.value + 512), N) == INVALID
    assert L.moe_tile_int4_weights(FAKE, 0, 128, other, N) == OK
    # grouped GEMMs (plan_bytes after the plan)
    pb = mq.moe_plan_size(8, 32)
    for fn in (L.moe_grouped_gemm_w4a8, L.moe_grouped_gemm_fp8row, L.moe_grouped_gemm_w4a8_bf16s):
        assert fn(FAKE, FAKE, FAKE, pb, 8, 32, FAKE, FAKE, 100, 256, 0, FAKE, 1, N) == UNSUPPORTED
        assert fn(FAKE, FAKE, FAKE, pb, 8, 32, FAKE, FAKE, 256, 200, 0, FAKE, 1, N) == UNSUPPORTED
        assert fn(FAKE, FAKE, FAKE, pb, 8, 32, FAKE, FAKE, 256, 256, 1, FAKE, 0, N) == INVALID
        assert fn(FAKE, FAKE, FAKE, pb, 8, 32, FAKE, FAKE, 256, 256, 5, FAKE, 1, N) == INVALID
        assert fn(N, FAKE, FAKE, pb, 8, 32, FAKE, FAKE, 256, 256, 0, FAKE, 1, N) == INVALID
        assert fn(N, N, N, 0, 8, 0, N, N, 256, 256, 0, N, 1, N) == OK
        # a plan buffer smaller than moe_plan_size(E, R): too few bytes, or built for a smaller R
        assert fn(FAKE, FAKE, FAKE, pb - 4, 8, 32, FAKE, FAKE, 256, 256, 0, FAKE, 1, N) == WORKSPACE
        assert fn(FAKE, FAKE, FAKE, mq.moe_plan_size(8, 16), 8, 32, FAKE, FAKE, 256, 256, 0, FAKE,
                  1, N) == WORKSPACE
        assert fn(FAKE, FAKE, FAKE, mq.moe_plan_size(4, 32), 8, 32, FAKE, FAKE, 256, 256, 0, FAKE,
                  1, N) == WORKSPACE
        assert fn(FAKE, FAKE, ctypes.c_void_p(4098), pb, 8, 32, FAKE, FAKE, 256, 256, 0, FAKE, 1,
                  N) == INVALID                                                   # plan misaligned
    # NVFP4 / AQLM: plan bytes and the slab count S
    nv = lambda pbytes, E, slab, S: L.moe_grouped_gemm_nvfp4(  # noqa: E731
        FAKE, FAKE, FAKE, pbytes, E, 32, slab, S, FAKE, FAKE, FAKE, 256, 256, 0, FAKE, 1, N)
    assert nv(pb - 4, 8, FAKE, 3) == WORKSPACE
    assert nv(pb, 8, N, 3) == INVALID                 # identity slab map with fewer slabs than E
    assert nv(pb, 8, FAKE, -1) == INVALID
    assert nv(pb, 8, FAKE, 0) == OK                   # no expert in this format: nothing to do
    books = (ctypes.c_void_p * 1)(FAKE)
    ents = (ctypes.c_int * 1)(65536)
    aq = lambda pbytes, E, slab, S: L.moe_grouped_gemm_aqlm(  # noqa: E731
        FAKE, FAKE, FAKE, pbytes, E, 32, slab, S, 1, books, ents, books, FAKE, 256, 256, 0, FAKE,
        1, N)
    assert aq(pb - 4, 8, FAKE, 3) == WORKSPACE
    assert aq(pb, 8, N, 3) == INVALID
    assert aq(pb, 8, FAKE, 0) == OK
    bad_ents = (ctypes.c_int * 1)(65537)
    assert L.moe_grouped_gemm_aqlm(FAKE, FAKE, FAKE, pb, 8, 32, FAKE, 3, 1, books, bad_ents, books,
                                   FAKE, 256, 256, 0, FAKE, 1, N) == UNSUPPORTED
    # fused expert MLP
    for fn in (L.moe_expert_mlp_w4a8, L.moe_expert_mlp_fp8row):
        ok = (FAKE, FAKE, FAKE, big, 8, 24, FAKE, FAKE, FAKE, FAKE, 4096, 2048, FAKE, FAKE, FAKE,
              FAKE, N)
        assert fn(*ok[:10], 4000, *ok[11:]) == UNSUPPORTED                  # H % 128
        assert fn(*ok[:11], 2000, *ok[12:]) == UNSUPPORTED                  # I % 128
        assert fn(*ok[:4], 2000, *ok[5:]) == UNSUPPORTED                    # E > 1024
        assert fn(*ok[:12], N, *ok[13:]) == INVALID                         # h null
        assert fn(*ok[:3], 64, *ok[4:]) == WORKSPACE                        # plan too small
        assert fn(ctypes.c_void_p(4100), *ok[1:]) == INVALID                # xp_q misaligned
        assert fn(N, N, N, 0, 8, 0, N, N, N, N, 4096, 2048, N, N, N, N, N) == OK   # R = 0
    # combine / shared (plan_bytes and E after the plan)
    cb = mq.moe_plan_size(8, 8)
    assert L.moe_combine(FAKE, FAKE, cb, 8, FAKE, N, 4, 2, 12, FAKE, N) == UNSUPPORTED
    assert L.moe_combine(FAKE, N, cb, 8, FAKE, N, 4, 2, 16, FAKE, N) == INVALID
    assert L.moe_combine(FAKE, FAKE, cb, 8, FAKE, N, 4, 9, 16, FAKE, N) == UNSUPPORTED   # k > 8
    assert L.moe_combine(FAKE, FAKE, cb, 0, FAKE, N, 4, 2, 16, FAKE, N) == INVALID       # E = 0
    assert L.moe_combine(FAKE, FAKE, cb - 4, 8, FAKE, N, 4, 2, 16, FAKE, N) == WORKSPACE
    assert L.moe_combine(FAKE, FAKE, cb, 8, FAKE, N, 8, 2, 16, FAKE, N) == WORKSPACE      # R = 16
    # more 2048-column blocks than the grid's second dimension holds
    assert L.moe_combine(FAKE, FAKE, cb, 8, FAKE, N, 0, 2, 1 << 28, FAKE, N) == UNSUPPORTED
    assert L.moe_shared_gemm_bf16(FAKE, FAKE, 4, 100, 64, 0, FAKE, N) == UNSUPPORTED
    assert L.moe_shared_gemm_bf16(FAKE, FAKE, 4, 128, 48, 0, FAKE, N) == UNSUPPORTED


@pytest.mark.skipif(torch.cuda.is_available(), reason="would launch on fake pointers")
def test_valid_call_without_gpu_reports_device_error():
    L = mq.lib
    assert L.moe_route_topk(FAKE, None, 4, 8, 2, 1, FAKE, FAKE, None) == DEVICE
    assert L.moe_combine(FAKE, FAKE, mq.moe_plan_size(8, 8), 8, FAKE, None, 4, 2, 16, FAKE,
                         None) == DEVICE
    assert L.moe_grouped_gemm_w4a8(FAKE, FAKE, FAKE, mq.moe_plan_size(8, 32), 8, 32, FAKE, FAKE,
                                   256, 256, 0, FAKE, 1, None) == DEVICE
    assert L.moe_expert_mlp_w4a8(FAKE, FAKE, FAKE, 1 << 20, 8, 24, FAKE, FAKE, FAKE, FAKE, 256,
                                 128, FAKE, FAKE, FAKE, FAKE, None) == DEVICE


def test_python_binding_raises_on_bad_input():
    with pytest.raises(TypeError):
        mq.moe_route_topk(torch.zeros(2, 8, dtype=torch.float64), 2)
    with pytest.raises(ValueError):
        mq.moe_route_topk(torch.zeros(2, 8), 2)        # host tensor


def test_binding_plan_shape_check():
    # a plan tensor remembers the (E, R) it was built for; calls with other sizes
    # are rejected in Python, before the C ABI (no device memory is read)
    plan = torch.zeros(mq.moe_plan_size(8, 32) // 4, dtype=torch.int32)
    mq._mark_plan(plan, 8, 32)
    with pytest.raises(ValueError, match="built for"):
        mq._plan_shape_ok(plan, 8, 16)
    with pytest.raises(ValueError, match="built for"):
        mq._plan_shape_ok(plan, 4, 32)
    mq._plan_shape_ok(plan, 8, 32)
    unmarked = torch.zeros(4, dtype=torch.int32)
    mq._plan_shape_ok(unmarked, 8, 32)                 # no record: nothing to compare


def test_binding_views_int32_packed_weights():
    # the checkpoint's int32 [N, K/8] .weight_packed words are the GEMM's [N, K/2] bytes
    words = torch.tensor([[0x76543210, -0x1234568]], dtype=torch.int32)
    b = words.view(torch.uint8)
    assert b.shape == (1, 8)
    assert b.tolist() == [[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]]
