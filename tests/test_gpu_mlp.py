"""The routed experts' MLP in one call (moe_expert_mlp_w4a8 / _fp8row) against
the three separate calls it replaces: gate/up GEMM with SiLU, per-row FP8
quantization of h, down GEMM.  The results must be bit-identical.  The layer
tests compare the same path with the oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_moe_top_amd as mq

pytestmark = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


def _ids(T, k, E, rng, hot):
    rows = []
    for _ in range(T):
        if hot is not None:
            rest = [e for e in range(E) if e != hot]
            rows.append(np.r_[hot, rng.choice(rest, k - 1, replace=False)] if k > 1 else [hot])
        else:
            rows.append(rng.choice(E, k, replace=False))
    return np.stack(rows).astype(np.int32)


def _setup(T, k, E, H, I, fmt, hot, seed):
    rng = np.random.default_rng(seed)
    g = torch.Generator(device=_dev()).manual_seed(seed)
    ids = torch.from_numpy(_ids(T, k, E, rng, hot)).to(_dev())
    x = torch.randn(T, H, device=_dev(), generator=g).to(torch.bfloat16)
    x_q, x_s = mq.quant_fp8_per_token(x)
    plan, xp_q, xp_s = mq.moe_permute(ids, E, x_q, x_s)
    w13 = torch.randn(E, 2 * I, H, device=_dev(), generator=g) * 0.02
    w2 = torch.randn(E, H, I, device=_dev(), generator=g) * 0.02
    if fmt in ("w4a8", "w4a8_bf16s"):
        sdt = torch.bfloat16 if fmt == "w4a8_bf16s" else torch.float32
        q13, s13 = mq.pack_int4_g128(w13, scale_dtype=sdt, tiled=True)
        q2, s2 = mq.pack_int4_g128(w2, scale_dtype=sdt, tiled=True)
    else:
        q13, s13 = mq.quant_fp8_per_token(w13)
        q2, s2 = mq.quant_fp8_per_token(w2)
    del w13, w2
    return dict(plan=plan, xp_q=xp_q, xp_s=xp_s, w13=q13, s13=s13, w2=q2, s2=s2, R=T * k)


def _separate(c, fmt):
    gemm = mq.moe_grouped_gemm_fp8row if fmt == "fp8row" else mq.moe_grouped_gemm_w4a8
    h = gemm(c["xp_q"], c["xp_s"], c["plan"], c["w13"], c["s13"], epilogue=mq.EPI_SILU_MUL)
    h_q, h_s = mq.quant_fp8_per_token(h)
    o = gemm(h_q, h_s, c["plan"], c["w2"], c["s2"], epilogue=mq.EPI_NONE)
    return dict(h=h, h_q=h_q, h_s=h_s, o=o)


def _fused(c, fmt):
    mlp = mq.moe_expert_mlp_fp8row if fmt == "fp8row" else mq.moe_expert_mlp_w4a8
    return mlp(c["xp_q"], c["xp_s"], c["plan"], c["w13"], c["s13"], c["w2"], c["s2"])


@pytest.mark.parametrize("fmt", ["w4a8", "fp8row", "w4a8_bf16s"])
@pytest.mark.parametrize("T,k,E,H,I,hot", [
    (4, 6, 24, 4096, 2048, None),   # decode shape: the unrolled K sweeps
    (4, 6, 64, 512, 256, None),     # decode-like, looped K sweeps
    (16, 2, 8, 256, 128, None),     # the tiny layer
    (40, 1, 3, 256, 256, 1),        # one expert with > 16 rows: several row blocks
    (64, 1, 2, 128, 128, 0),        # R = 64: a full 64-row tile
    (12, 4, 8, 4096, 256, None),    # H = 4096 with a narrow expert (unrolled gate/up sweep)
    (4, 6, 8, 256, 2048, 3),        # I = 2048 (unrolled down sweep), a hot expert
    (60, 1, 4, 128, 1024, None),    # many rows per expert: row blocks past four rows
    (30, 4, 16, 256, 128, None),    # R = 120: 64-row tiles of the two-launch path
    (50, 4, 16, 256, 128, None),    # R = 200 > 192: the tile kernels, three launches
    (4, 2, 8, 128, 2560, None),     # I > 2048: the three-launch path
    (4, 6, 24, 256, 640, None),     # I = 640: uneven K quarters (1, 1, 1, 2 groups)
])
def test_expert_mlp_matches_separate_calls(fmt, T, k, E, H, I, hot):
    c = _setup(T, k, E, H, I, fmt, hot, seed=T * 7 + E + H + I)
    ref = _separate(c, fmt)
    out = _fused(c, fmt)
    again = _fused(c, fmt)                  # repeatable, plan unchanged
    torch.cuda.synchronize()
    for name in ("h", "h_q", "h_s", "o"):
        assert torch.equal(out[name], ref[name]), name
        assert torch.equal(again[name], ref[name]), name + " (second call)"


def test_expert_mlp_argument_errors():
    z = torch.zeros(4, 128, dtype=torch.uint8, device=_dev())
    s = torch.zeros(4, device=_dev())
    ids = torch.zeros(1, 4, dtype=torch.int32, device=_dev())
    plan, _, _ = mq.moe_permute(ids, 8)
    w13 = torch.zeros(8, 16, 1, 16, 64, dtype=torch.uint8, device=_dev())   # tiled, N=256, K=128
    s13 = torch.zeros(8, 256, 1, device=_dev())
    w2 = torch.zeros(8, 8, 1, 16, 64, dtype=torch.uint8, device=_dev())     # tiled, N=128, K=128
    s2 = torch.zeros(8, 128, 1, device=_dev())
    with pytest.raises(mq.MoeqError):                   # plan too small for R = 4
        mq.moe_expert_mlp_w4a8(z, s, plan[:8], w13, s13, w2, s2)
    with pytest.raises(ValueError):
        mq.moe_expert_mlp_w4a8(z, s, plan, w13, s13, w2[:, :4], s2)
    with pytest.raises(ValueError):                     # packed rows not in the tiled order
        mq.moe_expert_mlp_w4a8(z, s, plan, torch.zeros(8, 256, 64, dtype=torch.uint8,
                                                       device=_dev()), s13, w2, s2)
    # output buffers the caller passes are checked, not trusted
    for bad in ({"h": torch.empty(4, 64, dtype=torch.bfloat16, device=_dev())},      # shape
                {"h_q": torch.empty(4, 128, dtype=torch.int8, device=_dev())},        # dtype
                {"o": torch.empty(128, 4, dtype=torch.bfloat16, device=_dev()).t()},  # strides
                {"h_s": torch.empty(4)}):                                             # host
        with pytest.raises(ValueError):
            mq.moe_expert_mlp_w4a8(z, s, plan, w13, s13, w2, s2, out=bad)
    logits = torch.zeros(1, 8, device=_dev())
    x = torch.zeros(1, 128, dtype=torch.bfloat16, device=_dev())
    with pytest.raises(ValueError):
        mq.moe_route_quant_permute(logits, x, 4, out={"xp_q": torch.empty(4, 64, dtype=torch.uint8,
                                                                         device=_dev())})
    with pytest.raises(TypeError):                     # a float plan buffer
        mq.moe_route_quant_permute(logits, x, 4, out={"plan": torch.empty(8, device=_dev())})
