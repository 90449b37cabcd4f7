"""One quantized MoE expert layer as a fixed sequence of libmoeq calls.

    [router logits, when the layer holds the router weights]
      -> route + quantize x + permute (one call; one launch for T <= 16)
      -> expert MLP: gate/up GEMM (+SiLU) -> quantize h -> down GEMM (one call;
         two launches for decode-sized batches)
      -> combine (+ shared experts)

Only orchestration lives here: buffers are torch allocations, reused across
calls with the same token count, and every step is a C-ABI call into libmoeq.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (EPI_NONE, EPI_SILU_MUL, moe_combine, moe_expert_mlp_fp8row, moe_expert_mlp_w4a8,
               moe_grouped_gemm_aqlm, moe_grouped_gemm_fp8row, moe_grouped_gemm_nvfp4,
               moe_grouped_gemm_w4a8, moe_plan_size,
               moe_requant_fp8_fnuz, moe_route_quant_permute, moe_router_logits, moe_shared_gemm_bf16, pack_int4_g128,
               quant_fp8_per_token)


class MoELayer:
    """Routed experts (W4A8 INT4-g128 or row-scaled FP8) plus optional bf16 shared experts.

    weight_format: "w4a8" (INT4 g128, fp32 group scales), "w4a8_bf16s" (INT4
    g128, bfloat16 group scales) or "fp8row" (E4M3, one fp32 scale per row).
    Weights: w13 [E, 2I, H] (gate rows then up rows), w2 [E, H, I].
    """

    def __init__(self, H: int, I: int, E: int, k: int, weight_format: str = "w4a8",
                 renormalize: bool = True, device="cuda"):
        if weight_format not in ("w4a8", "w4a8_bf16s", "fp8row"):
            raise ValueError(weight_format)
        self.H, self.I, self.E, self.k = H, I, E, k
        self.weight_format = weight_format
        self.renormalize = renormalize
        self.device = torch.device(device)
        self.w13 = self.s13 = self.w2 = self.s2 = None
        self.ws13 = self.ws2 = None
        self.w_router = None
        self._bufs = {}

    # --------------------------------------------------------------- weights
    def set_weights(self, w13, s13, w2, s2):
        """Already-quantized weights: INT4 in the GEMMs' tiled order (tile_int4_weights)
        with group scales, or E4M3 with row scales."""
        self.w13, self.s13, self.w2, self.s2 = w13, s13, w2, s2

    def quantize_weights(self, w13_f32: torch.Tensor, w2_f32: torch.Tensor):
        """Quantize fp32 weights on the device with the library's own kernels."""
        if self.weight_format in ("w4a8", "w4a8_bf16s"):
            sdt = torch.bfloat16 if self.weight_format == "w4a8_bf16s" else torch.float32
            self.w13, self.s13 = pack_int4_g128(w13_f32, scale_dtype=sdt, tiled=True)
            self.w2, self.s2 = pack_int4_g128(w2_f32, scale_dtype=sdt, tiled=True)
        else:
            self.w13, self.s13 = quant_fp8_per_token(w13_f32)
            self.w2, self.s2 = quant_fp8_per_token(w2_f32)

    def set_weights_fnuz(self, w13_fnuz, s13_fnuz, w2_fnuz, s2_fnuz):
        """Row-scaled E4M3FNUZ expert weights (the MI300X checkpoint layout: scales
        [E, out_channels], max|row| / 240), converted on the device to the
        row-scaled OCP E4M3 weights this layer runs on."""
        if self.weight_format != "fp8row":
            raise ValueError("E4M3FNUZ weights are row-scaled FP8 experts (weight_format='fp8row')")
        self.w13, self.s13 = moe_requant_fp8_fnuz(w13_fnuz, s13_fnuz)
        self.w2, self.s2 = moe_requant_fp8_fnuz(w2_fnuz, s2_fnuz)

    def set_router(self, w_router: Optional[torch.Tensor]):
        """fp32 router weights [E, H]; forward() then takes logits=None and computes
        them with moe_router_logits."""
        self.w_router = w_router

    def set_shared(self, ws13: Optional[torch.Tensor], ws2: Optional[torch.Tensor]):
        self.ws13, self.ws2 = ws13, ws2

    # ---------------------------------------------------------------- buffers
    def buffers(self, T: int) -> dict:
        b = self._bufs.get(T)
        if b is None:
            H, I, E, k, d = self.H, self.I, self.E, self.k, self.device
            R = T * k
            b = {
                "logits": torch.empty(T, E, dtype=torch.float32, device=d),
                "ids": torch.empty(T, k, dtype=torch.int32, device=d),
                "w": torch.empty(T, k, dtype=torch.float32, device=d),
                "x_q": torch.empty(T, H, dtype=torch.uint8, device=d),
                "x_s": torch.empty(T, dtype=torch.float32, device=d),
                "plan": torch.empty((moe_plan_size(E, R) + 3) // 4, dtype=torch.int32, device=d),
                "xp_q": torch.empty(R, H, dtype=torch.uint8, device=d),
                "xp_s": torch.empty(R, dtype=torch.float32, device=d),
                "h": torch.empty(R, I, dtype=torch.bfloat16, device=d),
                "h_q": torch.empty(R, I, dtype=torch.uint8, device=d),
                "h_s": torch.empty(R, dtype=torch.float32, device=d),
                "o": torch.empty(R, H, dtype=torch.bfloat16, device=d),
                "y": torch.empty(T, H, dtype=torch.bfloat16, device=d),
            }
            if self.ws13 is not None:
                S = self.ws2.shape[1]
                b["sh_h"] = torch.empty(T, S, dtype=torch.bfloat16, device=d)
                b["shared"] = torch.empty(T, H, dtype=torch.bfloat16, device=d)
            self._bufs[T] = b
        return b

    # ---------------------------------------------------------------- forward
    def forward(self, x: torch.Tensor, logits: Optional[torch.Tensor] = None,
                bias: Optional[torch.Tensor] = None,
                return_all: bool = False, events: Optional[list] = None,
                split_mlp: bool = False):
        """y = layer(x).  logits=None: the router's logits are computed from x and the
        weights given to set_router.  With `events` (a list), each call is bracketed by a pair of
        timing events on the current stream, appended as (name, start, end).
        split_mlp runs the expert MLP as its three separate calls (same results)."""
        T = x.shape[0]
        b = self.buffers(T)
        w4 = self.weight_format != "fp8row"      # INT4 (scale dtype picks the entry point)
        gemm = moe_grouped_gemm_w4a8 if w4 else moe_grouped_gemm_fp8row
        mlp = moe_expert_mlp_w4a8 if w4 else moe_expert_mlp_fp8row

        def step(name, fn, *args, **kw):
            if events is None:
                return fn(*args, **kw)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            r = fn(*args, **kw)
            e.record()
            events.append((name, s, e))
            return r

        if logits is None:
            if self.w_router is None:
                raise ValueError("logits=None needs router weights (set_router)")
            logits = step("router", moe_router_logits, x, self.w_router, out=b["logits"])
        step("route_quant_permute", moe_route_quant_permute, logits, x, self.k, bias,
             self.renormalize, out=b)
        if split_mlp:
            step("gemm_gate_up", gemm, b["xp_q"], b["xp_s"], b["plan"], self.w13, self.s13,
                 epilogue=EPI_SILU_MUL, out=b["h"])
            step("quant_h", quant_fp8_per_token, b["h"], q=b["h_q"], scale=b["h_s"])
            step("gemm_down", gemm, b["h_q"], b["h_s"], b["plan"], self.w2, self.s2,
                 epilogue=EPI_NONE, out=b["o"])
        else:
            step("expert_mlp", mlp, b["xp_q"], b["xp_s"], b["plan"], self.w13, self.s13, self.w2,
                 self.s2, out=b)
        shared = None
        if self.ws13 is not None:
            # the shared experts are bf16 MLPs of the bf16 model: their input is x itself
            if x.dtype != torch.bfloat16:
                raise TypeError("shared experts take bfloat16 x")
            step("shared_gate_up", moe_shared_gemm_bf16, x, self.ws13, EPI_SILU_MUL, out=b["sh_h"])
            shared = step("shared_down", moe_shared_gemm_bf16, b["sh_h"], self.ws2, EPI_NONE,
                          out=b["shared"])
        step("combine", moe_combine, b["o"], b["plan"], b["w"], shared, y=b["y"], E=self.E)
        return b if return_all else b["y"]

    __call__ = forward


class HybridMoELayer(MoELayer):
    """The NVFP4 + AQLM hybrid expert layer: each routed expert is either hot
    (an NVFP4 slab) or cold (an AQLM slab).  hot_ids / cold_ids list the routed
    expert of each slab and together partition 0 .. E-1.

    Hot slabs:  w13 [n_hot, 2I, H/2] E2M1 pairs, w13_bs [n_hot, 2I, H/16] E4M3,
                w13_s2 [n_hot] fp32; w2 [n_hot, H, I/2], w2_bs [n_hot, H, I/16], w2_s2.
    Cold slabs: per projection a list of code tensors ([n_cold, out, in/8], one
                per book), the list of fp16 codebooks [entries, 8], and the fp16
                row scales [n_cold, out].
    Each GEMM step runs both formats' kernels; each fills only its experts' rows.
    """

    def __init__(self, H: int, I: int, E: int, k: int, renormalize: bool = True, device="cuda"):
        super().__init__(H, I, E, k, "w4a8", renormalize, device)
        self.weight_format = "hybrid"
        self.hot = self.cold = None

    def set_hybrid_weights(self, hot_ids, cold_ids, hot: dict, cold: dict):
        """hot: w13, w13_bs, w13_s2, w2, w2_bs, w2_s2; cold: w13_codes (list), w13_books
        (list), w13_scale, w2_codes, w2_books, w2_scale."""
        d = self.device
        hot_ids = torch.as_tensor(hot_ids, dtype=torch.int64)
        cold_ids = torch.as_tensor(cold_ids, dtype=torch.int64)
        if torch.cat([hot_ids, cold_ids]).sort().values.tolist() != list(range(self.E)):
            raise ValueError("hot_ids and cold_ids must partition the experts")
        hot_of = torch.full((self.E,), -1, dtype=torch.int32)
        cold_of = torch.full((self.E,), -1, dtype=torch.int32)
        hot_of[hot_ids] = torch.arange(len(hot_ids), dtype=torch.int32)
        cold_of[cold_ids] = torch.arange(len(cold_ids), dtype=torch.int32)
        self.hot_of, self.cold_of = hot_of.to(d), cold_of.to(d)
        self.hot, self.cold = hot, cold

    def _gemm_both(self, a_q, a_s, plan, proj: str, epilogue, out):
        h, c = self.hot, self.cold
        if h is not None and h[proj].shape[0] > 0:
            moe_grouped_gemm_nvfp4(a_q, a_s, plan, h[proj], h[proj + "_bs"], h[proj + "_s2"],
                                   epilogue=epilogue, out=out, slab_of=self.hot_of)
        if c is not None and c[proj + "_scale"].shape[0] > 0:
            moe_grouped_gemm_aqlm(a_q, a_s, plan, c[proj + "_codes"], c[proj + "_books"],
                                  c[proj + "_scale"], epilogue=epilogue, out=out,
                                  slab_of=self.cold_of)
        return out

    def forward(self, x: torch.Tensor, logits: Optional[torch.Tensor] = None,
                bias: Optional[torch.Tensor] = None, return_all: bool = False,
                events: Optional[list] = None, split_mlp: bool = True):
        T = x.shape[0]
        b = self.buffers(T)

        def step(name, fn, *args, **kw):
            if events is None:
                return fn(*args, **kw)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            r = fn(*args, **kw)
            e.record()
            events.append((name, s, e))
            return r

        if logits is None:
            if self.w_router is None:
                raise ValueError("logits=None needs router weights (set_router)")
            logits = step("router", moe_router_logits, x, self.w_router, out=b["logits"])
        step("route_quant_permute", moe_route_quant_permute, logits, x, self.k, bias,
             self.renormalize, out=b)
        step("gemm_gate_up", self._gemm_both, b["xp_q"], b["xp_s"], b["plan"], "w13",
             EPI_SILU_MUL, b["h"])
        step("quant_h", quant_fp8_per_token, b["h"], q=b["h_q"], scale=b["h_s"])
        step("gemm_down", self._gemm_both, b["h_q"], b["h_s"], b["plan"], "w2", EPI_NONE, b["o"])
        step("combine", moe_combine, b["o"], b["plan"], b["w"], None, y=b["y"], E=self.E)
        return b if return_all else b["y"]

    __call__ = forward
