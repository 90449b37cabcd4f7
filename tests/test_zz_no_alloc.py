"""moe_expert_mlp_w4a8_noalloc: the expert MLP with its intermediates in the
library's per-GPU scratch array, called through the C ABI, against
moe_expert_mlp_w4a8 on the same inputs (bit-identical o), on two calls in a row
of which the second is smaller; and its size limit, checked on the host."""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_moe_top_amd as mq


def _case(T, k, E, H, I, seed, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    ids = torch.stack([torch.randperm(E, generator=g, device=dev)[:k] for _ in range(T)]).to(
        torch.int32)
    x = torch.randn(T, H, generator=g, device=dev).to(torch.bfloat16)
    x_q, x_s = mq.quant_fp8_per_token(x)
    plan, xp_q, xp_s = mq.moe_permute(ids, E, x_q, x_s)
    w13, s13 = mq.pack_int4_g128(torch.randn(E, 2 * I, H, generator=g, device=dev) * 0.02,
                                 tiled=True)
    w2, s2 = mq.pack_int4_g128(torch.randn(E, H, I, generator=g, device=dev) * 0.02, tiled=True)
    return plan, xp_q, xp_s, w13, s13, w2, s2


@pytest.mark.gpu
def test_noalloc_expert_mlp_matches_two_calls_smaller_second():
    dev = torch.device("cuda:0")
    E, H, I = 8, 4096, 2048
    # 300 routed rows (64-row tile kernels, three launches), then 24 (decode
    # units, the down GEMM quantizing h itself, two launches)
    for T, k in ((50, 6), (4, 6)):
        print(f"[noalloc] T={T} k={k} E={E} H={H} I={I}", flush=True)
        plan, xp_q, xp_s, w13, s13, w2, s2 = _case(T, k, E, H, I, 1000 + T, dev)
        ref = mq.moe_expert_mlp_w4a8(xp_q, xp_s, plan, w13, s13, w2, s2)["o"]
        got = torch.full_like(ref, float("nan"))
        rc = mq.lib.moe_expert_mlp_w4a8_noalloc(
            ctypes.c_void_p(xp_q.data_ptr()), ctypes.c_void_p(xp_s.data_ptr()),
            ctypes.c_void_p(plan.data_ptr()), plan.numel() * 4, E, T * k,
            ctypes.c_void_p(w13.data_ptr()), ctypes.c_void_p(s13.data_ptr()),
            ctypes.c_void_p(w2.data_ptr()), ctypes.c_void_p(s2.data_ptr()), H, I,
            ctypes.c_void_p(got.data_ptr()),
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        assert rc == 0, mq.moe_status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        # the binding's wrapper of the same call
        got2 = mq.moe_expert_mlp_w4a8_noalloc(xp_q, xp_s, plan, w13, s13, w2, s2)
        torch.cuda.synchronize()
        assert torch.equal(got2, ref)


def test_noalloc_size_limit_on_the_host():
    # argument checks run before any HIP call: R * I beyond the scratch array
    # is rejected with its own status, on any machine
    fake = ctypes.c_void_p(4096)
    E, H, I = 8, 4096, 2048
    big = 5458 * 1
    rc = mq.lib.moe_expert_mlp_w4a8_noalloc(fake, fake, fake, 1 << 30, E, big, fake, fake, fake,
                                            fake, H, I, fake, None)
    assert rc == 6 and "scratch" in mq.moe_status_string(rc)
    rc = mq.lib.moe_expert_mlp_w4a8_noalloc(fake, fake, fake, 1 << 30, E, 24, fake, fake, fake,
                                            fake, H, I, None, None)
    assert rc == 1                                    # o is required
    assert mq.lib.moe_expert_mlp_w4a8_noalloc(None, None, None, 0, E, 0, None, None, None, None,
                                              H, I, None, None) == 0     # R = 0: nothing to do
    _ = np
