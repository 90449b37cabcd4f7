"""Python binding of libmoeq, the quantized MoE expert layer for MI355X (gfx950).

Argument marshalling only: every function below checks dtypes/shapes, allocates
outputs with torch (device memory and streams are all torch is used for), and
calls the C ABI declared in include/moeq.h, which enqueues the HIP kernels on the
current torch stream.  No computation happens here, and there is no fallback:
if libmoeq.so is missing, importing this package raises ImportError.

Build the library first:  python bit_quantized_moe_top_amd/build.py
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "LIB_PATH", "lib", "MOEQ_F32", "MOEQ_BF16", "EPI_NONE", "EPI_SILU_MUL", "TILE_M",
    "MAX_EXPERTS", "MAX_TOPK", "MoeqError", "moe_abi_version", "moe_status_string",
    "moe_plan_size", "moe_router_logits", "moe_route_topk", "quant_fp8_per_token", "moe_permute",
    "moe_route_quant_permute", "pack_int4_g128", "tile_int4_weights", "moe_requant_fp8_fnuz",
    "moe_read_bandwidth_probe", "READ_PROBE_BLOCKS",
    "moe_grouped_gemm_w4a8", "moe_grouped_gemm_w4a8_bf16s", "moe_grouped_gemm_nvfp4",
    "moe_grouped_gemm_aqlm",
    "moe_expert_mlp_w4a8", "moe_expert_mlp_w4a8_noalloc", "NOALLOC_SCRATCH_BYTES",
    "moe_expert_mlp_w4a8_bf16s", "moe_expert_mlp_fp8row", "pack_int4_g128_bf16s", "moe_grouped_gemm_fp8row", "moe_combine", "moe_shared_gemm_bf16",
    "plan_fields", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoeq.so")

MOEQ_F32, MOEQ_BF16 = 0, 1
EPI_NONE, EPI_SILU_MUL = 0, 1
TILE_M = 64
MAX_EXPERTS, MAX_TOPK = 1024, 8
PLAN_HEADER = 16
NOALLOC_SCRATCH_BYTES = 32 << 20     # MOEQ_NOALLOC_SCRATCH_BYTES
READ_PROBE_BLOCKS = 8192             # MOEQ_READ_PROBE_BLOCKS

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); the exact list of entry points in include/moeq.h
_SIGNATURES = {
    "moe_abi_version": (_I, []),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_plan_size": (_SZ, [_I, _I]),
    "moe_router_logits": (_I, [_P, _I, _I, _I, _P, _I, _P, _P]),
    "moe_route_topk": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "quant_fp8_per_token": (_I, [_P, _I, _I64, _I, _I64, _P, _P, _P]),
    "moe_permute": (_I, [_P, _I, _I, _I, _P, _P, _I, _P, _P, _P, _SZ, _P]),
    "moe_route_quant_permute": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P,
                                     _P, _SZ, _P]),
    "pack_int4_g128": (_I, [_P, _I64, _I, _P, _P, _P]),
    "pack_int4_g128_bf16s": (_I, [_P, _I64, _I, _P, _P, _P]),
    "moe_tile_int4_weights": (_I, [_P, _I64, _I, _P, _P]),
    "moe_read_bandwidth_probe": (_I, [_P, _SZ, _P, _P]),
    "moe_requant_fp8_fnuz": (_I, [_P, _P, _I64, _I, _P, _P, _P]),
    "moe_grouped_gemm_w4a8": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _P, _I, _I, _I, _P, _I, _P]),
    "moe_grouped_gemm_fp8row": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _P, _I, _I, _I, _P, _I, _P]),
    "moe_grouped_gemm_w4a8_bf16s": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _P, _I, _I, _I, _P, _I,
                                         _P]),
    "moe_grouped_gemm_nvfp4": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _I, _P, _P, _P, _I, _I, _I, _P,
                                    _I, _P]),
    "moe_grouped_gemm_aqlm": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _I, _I, _P, _P, _P, _P, _I, _I,
                                   _I, _P, _I, _P]),
    "moe_expert_mlp_w4a8": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P,
                                 _P]),
    "moe_expert_mlp_w4a8_bf16s": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P,
                                       _P, _P]),
    "moe_expert_mlp_fp8row": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P,
                                   _P, _P]),
    "moe_expert_mlp_w4a8_noalloc": (_I, [_P, _P, _P, _SZ, _I, _I, _P, _P, _P, _P, _I, _I, _P,
                                         _P]),
    "moe_combine": (_I, [_P, _P, _SZ, _I, _P, _P, _I, _I, _I, _P, _P]),
    "moe_shared_gemm_bf16": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run: python bit_quantized_moe_top_amd/build.py")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


class MoeqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {lib.moe_status_string(status).decode()} (status {status})")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeqError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _req(t: torch.Tensor, name: str, dtype, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _out(o: dict, name: str, shape: tuple, dtype, dev: torch.device) -> torch.Tensor:
    """o[name]: the caller's tensor, checked against the shape and dtype the call
    writes, or a new one (allocated only when o has none)."""
    t = o.get(name)
    if t is None:
        t = o[name] = torch.empty(shape, dtype=dtype, device=dev)
    elif (t.dtype != dtype or t.shape != shape or t.device != dev or
          not t.is_contiguous()):
        raise ValueError(f"out[{name!r}] must be a contiguous {dtype} tensor of shape {shape} "
                         f"on {dev}, got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _weight_bytes(t: torch.Tensor, name: str) -> torch.Tensor:
    """Packed INT4 weights as bytes: uint8 [..., K/2] as they are, or the checkpoint's
    int32 [..., K/8] .weight_packed words viewed as their little-endian bytes."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.int32:
        _req(t, name, torch.int32)
        return t.view(torch.uint8)
    _req(t, name, torch.uint8)
    return t


def _tiled_int4(t: torch.Tensor, name: str) -> Tuple[int, int, int]:
    """(E, N, K) of INT4 weights in the GEMMs' tiled order, uint8
    [E, N/16, K/128, 16, 64] as tile_int4_weights returns them."""
    if isinstance(t, torch.Tensor) and t.dim() != 5:
        raise ValueError(f"{name} must be INT4 weights in the tiled order [E, N/16, K/128, 16, 64] "
                         f"(pass the packed rows through tile_int4_weights first), got {tuple(t.shape)}")
    _req(t, name, torch.uint8, 5)
    E, nb, G, r, c = t.shape
    if (r, c) != (16, 64):
        raise ValueError(f"{name}: the last two dims of the tiled order are (16, 64)")
    return E, 16 * nb, 128 * G


def _mark_plan(plan: torch.Tensor, E: int, R: int) -> None:
    # the (E, R) a plan tensor was last built for, so that later calls can check
    # theirs without reading device memory
    plan._moeq_shape = (E, R)


def _plan_shape_ok(plan: torch.Tensor, E: int, R: int) -> None:
    built = getattr(plan, "_moeq_shape", None)
    if built is not None and built != (E, R):
        raise ValueError(f"plan was built for (E, R) = {built}, the call has ({E}, {R})")


def _check_plan(plan: torch.Tensor, E: int, R: int) -> None:
    _req(plan, "plan", torch.int32, 1)
    _plan_shape_ok(plan, E, R)


def moe_abi_version() -> int:
    return lib.moe_abi_version()


def moe_status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def moe_plan_size(E: int, R: int) -> int:
    return lib.moe_plan_size(E, R)


def plan_fields(plan: torch.Tensor, E: int, R: int) -> dict:
    """Views of the plan's arrays (the layout documented in include/moeq.h)."""
    max_tiles = (R + TILE_M - 1) // TILE_M + min(E, R)
    chunks = max(1, (R + 1023) // 1024)
    o = PLAN_HEADER
    f = {"header": plan[:PLAN_HEADER]}
    for name, n in (("row_pos", R), ("sorted_rows", R), ("offsets", E + 1), ("active", E),
                    ("tile_expert", max_tiles), ("tile_row0", max_tiles), ("scratch", chunks * E)):
        f[name] = plan[o:o + n]
        o += n
    return f


# ----------------------------------------------------------------------- calls
def moe_router_logits(x: torch.Tensor, w_router: torch.Tensor,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [T, H] fp32/bf16, w_router [E, H] fp32 -> logits [T, E] fp32 = x . w_router^T."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _req(x, "x", x.dtype, 2)
    _req(w_router, "w_router", torch.float32, 2)
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("w_router must be [E, H]")
    if out is None:
        out = torch.empty(T, E, dtype=torch.float32, device=x.device)
    dt = MOEQ_BF16 if x.dtype == torch.bfloat16 else MOEQ_F32
    _check("moe_router_logits", lib.moe_router_logits(_ptr(x), dt, T, H, _ptr(w_router), E,
                                                      _ptr(out), _stream(x.device)))
    return out


def moe_route_topk(logits: torch.Tensor, k: int, bias: Optional[torch.Tensor] = None,
                   renormalize: bool = True, ids: Optional[torch.Tensor] = None,
                   weights: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    _req(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    if bias is not None:
        _req(bias, "bias", torch.float32, 1)
    if ids is None:
        ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _check("moe_route_topk", lib.moe_route_topk(_ptr(logits), _ptr(bias), T, E, k,
                                                1 if renormalize else 0, _ptr(ids), _ptr(weights),
                                                _stream(logits.device)))
    return ids, weights


def quant_fp8_per_token(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                        scale: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _req(x, "x", x.dtype)
    K = x.shape[-1]
    x2 = x.reshape(-1, K)
    M = x2.shape[0]
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    dt = MOEQ_BF16 if x.dtype == torch.bfloat16 else MOEQ_F32
    _check("quant_fp8_per_token", lib.quant_fp8_per_token(_ptr(x2), dt, M, K, K, _ptr(q),
                                                          _ptr(scale), _stream(x.device)))
    return q, scale


def moe_permute(topk_ids: torch.Tensor, E: int, x_q: Optional[torch.Tensor] = None,
                x_s: Optional[torch.Tensor] = None, plan: Optional[torch.Tensor] = None,
                xp_q: Optional[torch.Tensor] = None, xp_s: Optional[torch.Tensor] = None):
    """Returns (plan int32 tensor, xp_q, xp_s) -- the last two None without x_q."""
    _req(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    R = T * k
    dev = topk_ids.device
    nbytes = moe_plan_size(E, R)
    if plan is None:
        plan = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device=dev)
    H = 0
    if x_q is not None:
        _req(x_q, "x_q", torch.uint8, 2)
        _req(x_s, "x_s", torch.float32, 1)
        H = x_q.shape[1]
        if xp_q is None:
            xp_q = torch.empty(R, H, dtype=torch.uint8, device=dev)
        if xp_s is None:
            xp_s = torch.empty(R, dtype=torch.float32, device=dev)
    _check("moe_permute", lib.moe_permute(_ptr(topk_ids), T, k, E, _ptr(x_q), _ptr(x_s), H,
                                          _ptr(xp_q), _ptr(xp_s), _ptr(plan), plan.numel() * 4,
                                          _stream(dev)))
    _mark_plan(plan, E, R)
    return plan, xp_q, xp_s


def moe_route_quant_permute(logits: torch.Tensor, x: torch.Tensor, k: int,
                            bias: Optional[torch.Tensor] = None, renormalize: bool = True,
                            out: Optional[dict] = None) -> dict:
    """Routing, FP8 quantization of x and the permutation (with gather) in one call.
    Returns a dict with ids, w, x_q, x_s, plan, xp_q, xp_s (reusing `out`'s tensors)."""
    _req(logits, "logits", torch.float32, 2)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _req(x, "x", x.dtype, 2)
    T, E = logits.shape
    H = x.shape[1]
    R = T * k
    dev = x.device
    if bias is not None:
        _req(bias, "bias", torch.float32, 1)
    o = dict(out) if out is not None else {}
    _out(o, "ids", (T, k), torch.int32, dev)
    _out(o, "w", (T, k), torch.float32, dev)
    _out(o, "x_q", (T, H), torch.uint8, dev)
    _out(o, "x_s", (T,), torch.float32, dev)
    if o.get("plan") is None:
        o["plan"] = torch.empty((moe_plan_size(E, R) + 3) // 4, dtype=torch.int32, device=dev)
    else:
        _req(o["plan"], "out['plan']", torch.int32, 1)
    _out(o, "xp_q", (R, H), torch.uint8, dev)
    _out(o, "xp_s", (R,), torch.float32, dev)
    dt = MOEQ_BF16 if x.dtype == torch.bfloat16 else MOEQ_F32
    _check("moe_route_quant_permute", lib.moe_route_quant_permute(
        _ptr(logits), _ptr(bias), T, E, k, 1 if renormalize else 0, _ptr(x), dt, H, _ptr(o["ids"]),
        _ptr(o["w"]), _ptr(o["x_q"]), _ptr(o["x_s"]), _ptr(o["xp_q"]), _ptr(o["xp_s"]),
        _ptr(o["plan"]), o["plan"].numel() * 4, _stream(dev)))
    _mark_plan(o["plan"], E, R)
    return o


def moe_read_bandwidth_probe(buf: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Streams every byte of the contiguous device tensor buf (a measurement helper,
    not a layer step); returns sink, READ_PROBE_BLOCKS * 4 uint32 words (as int32)
    whose XOR is the XOR of buf's 32-bit words."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(READ_PROBE_BLOCKS * 4, dtype=torch.int32, device=buf.device)
    _req(sink, "sink", torch.int32, 1)
    if sink.numel() < READ_PROBE_BLOCKS * 4:
        raise ValueError("sink too small")
    _check("moe_read_bandwidth_probe", lib.moe_read_bandwidth_probe(
        _ptr(buf), nbytes, _ptr(sink), _stream(buf.device)))
    return sink


def tile_int4_weights(w_packed: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed INT4 rows uint8 [..., N, K/2] (or the checkpoint's int32 [..., N, K/8]
    words) -> the GEMMs' tiled order uint8 [..., N/16, K/128, 16, 64]
    (moe_tile_int4_weights; a permutation of whole bytes)."""
    w_packed = _weight_bytes(w_packed, "w_packed")
    if w_packed.dim() < 2:
        raise ValueError("w_packed must be [..., N, K/2]")
    N, K = w_packed.shape[-2], 2 * w_packed.shape[-1]
    shape = tuple(w_packed.shape[:-2]) + (N // 16, K // 128, 16, 64)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=w_packed.device)
    _req(out, "out", torch.uint8)
    if N % 16 or K % 128 or tuple(out.shape) != shape:
        raise ValueError(f"tiled INT4 weights need N % 16 == 0, K % 128 == 0 and out {shape}")
    rows = w_packed.numel() // (K // 2) if K else 0
    _check("moe_tile_int4_weights", lib.moe_tile_int4_weights(
        _ptr(w_packed), rows, K, _ptr(out), _stream(w_packed.device)))
    return out


def pack_int4_g128(w: torch.Tensor, packed: Optional[torch.Tensor] = None,
                   scales: Optional[torch.Tensor] = None,
                   scale_dtype=torch.float32, tiled: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """w [..., K] fp32 -> packed uint8 [..., K/2], scales [..., K/128] of scale_dtype
    (fp32: pack_int4_g128; bfloat16: pack_int4_g128_bf16s).
    tiled=True: the packed rows go through tile_int4_weights (into `packed`, then
    [..., N/16, K/128, 16, 64]), the order the GEMMs read."""
    _req(w, "w", torch.float32)
    if scales is not None:
        scale_dtype = scales.dtype
    if scale_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("scale_dtype must be float32 or bfloat16")
    if tiled:
        rows_packed, scales = pack_int4_g128(w, None, scales, scale_dtype)
        return tile_int4_weights(rows_packed, packed), scales
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    if packed is None:
        packed = torch.empty(*w.shape[:-1], K // 2, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(*w.shape[:-1], K // 128, dtype=scale_dtype, device=w.device)
    _req(scales, "scales", scale_dtype)
    name = "pack_int4_g128" if scale_dtype == torch.float32 else "pack_int4_g128_bf16s"
    _check(name, getattr(lib, name)(_ptr(w), rows, K, _ptr(packed), _ptr(scales),
                                    _stream(w.device)))
    return packed, scales


def pack_int4_g128_bf16s(w: torch.Tensor, packed: Optional[torch.Tensor] = None,
                         scales: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """pack_int4_g128 with bfloat16 scales."""
    return pack_int4_g128(w, packed, scales, scale_dtype=torch.bfloat16)


def moe_requant_fp8_fnuz(w_fnuz: torch.Tensor, s_fnuz: torch.Tensor,
                         w_ocp: Optional[torch.Tensor] = None,
                         s_ocp: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Row-scaled E4M3FNUZ weights w_fnuz uint8 [..., K] with scales s_fnuz fp32
    [...] -> row-scaled OCP E4M3 weights uint8 [..., K] and scales fp32 [...]."""
    _req(w_fnuz, "w_fnuz", torch.uint8)
    _req(s_fnuz, "s_fnuz", torch.float32)
    K = w_fnuz.shape[-1]
    rows = w_fnuz.numel() // K if K else 0
    if tuple(s_fnuz.shape) != tuple(w_fnuz.shape[:-1]):
        raise ValueError("s_fnuz must have shape w_fnuz.shape[:-1]")
    if w_ocp is None:
        w_ocp = torch.empty_like(w_fnuz)
    if s_ocp is None:
        s_ocp = torch.empty_like(s_fnuz)
    _check("moe_requant_fp8_fnuz", lib.moe_requant_fp8_fnuz(
        _ptr(w_fnuz), _ptr(s_fnuz), rows, K, _ptr(w_ocp), _ptr(s_ocp), _stream(w_fnuz.device)))
    return w_ocp, s_ocp


def _gemm(fn_name: str, a_q, a_s, plan, E, w, w_scale, N, K, epilogue, out_dtype, out):
    _req(a_q, "a_q", torch.uint8, 2)
    _req(a_s, "a_s", torch.float32, 1)
    R = a_q.shape[0]
    _check_plan(plan, E, R)
    if a_q.shape[1] != K:
        raise ValueError("a_q has the wrong K")
    n_out = N // 2 if epilogue == EPI_SILU_MUL else N
    if out is None:
        out = torch.empty(R, n_out, dtype=out_dtype, device=a_q.device)
    odt = MOEQ_BF16 if out.dtype == torch.bfloat16 else MOEQ_F32
    fn = getattr(lib, fn_name)
    _check(fn_name, fn(_ptr(a_q), _ptr(a_s), _ptr(plan), plan.numel() * 4, E, R, _ptr(w),
                       _ptr(w_scale), N, K, epilogue, _ptr(out), odt, _stream(a_q.device)))
    return out


def moe_grouped_gemm_w4a8(a_q: torch.Tensor, a_s: torch.Tensor, plan: torch.Tensor,
                          w_packed: torch.Tensor, w_scales: torch.Tensor,
                          epilogue: int = EPI_NONE, out_dtype=torch.bfloat16,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w_packed: INT4 weights in the tiled order, uint8 [E, N/16, K/128, 16, 64]
    (tile_int4_weights of the packed [E, N, K/2] rows or of the checkpoint's int32
    [E, N, K/8] words), w_scales [E, N, K/128] fp32 (or bfloat16: then
    moe_grouped_gemm_w4a8_bf16s)."""
    E, N, K = _tiled_int4(w_packed, "w_packed")
    bf16 = w_scales.dtype == torch.bfloat16
    _req(w_scales, "w_scales", torch.bfloat16 if bf16 else torch.float32, 3)
    if tuple(w_scales.shape) != (E, N, K // 128):
        raise ValueError("w_scales shape does not match w_packed")
    name = "moe_grouped_gemm_w4a8_bf16s" if bf16 else "moe_grouped_gemm_w4a8"
    return _gemm(name, a_q, a_s, plan, E, w_packed, w_scales, N, K, epilogue, out_dtype, out)


def moe_grouped_gemm_w4a8_bf16s(a_q, a_s, plan, w_packed, w_scales, epilogue: int = EPI_NONE,
                                out_dtype=torch.bfloat16, out=None) -> torch.Tensor:
    """moe_grouped_gemm_w4a8 with bfloat16 group scales w_scales [E, N, K/128]."""
    _req(w_scales, "w_scales", torch.bfloat16, 3)
    return moe_grouped_gemm_w4a8(a_q, a_s, plan, w_packed, w_scales, epilogue, out_dtype, out)


def moe_grouped_gemm_nvfp4(a_q: torch.Tensor, a_s: torch.Tensor, plan: torch.Tensor,
                           w_fp4: torch.Tensor, w_block_scale: torch.Tensor,
                           w_scale2: torch.Tensor, epilogue: int = EPI_NONE,
                           out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
                           slab_of: Optional[torch.Tensor] = None, E: Optional[int] = None
                           ) -> torch.Tensor:
    """w_fp4 [S, N, K/2] uint8 (E2M1 pairs), w_block_scale [S, N, K/16] uint8 (E4M3),
    w_scale2 [S] fp32; slab_of [E] int32 (-1: expert not NVFP4; rows left as they are)
    or None (slab e = expert e, E = S).  slab_of values outside [0, S) mark experts of
    another format."""
    _req(a_q, "a_q", torch.uint8, 2)
    _req(a_s, "a_s", torch.float32, 1)
    _req(w_fp4, "w_fp4", torch.uint8, 3)
    _req(w_block_scale, "w_block_scale", torch.uint8, 3)
    _req(w_scale2, "w_scale2", torch.float32, 1)
    S, N, K2 = w_fp4.shape
    K = 2 * K2
    if tuple(w_block_scale.shape) != (S, N, K // 16) or tuple(w_scale2.shape) != (S,):
        raise ValueError("w_block_scale / w_scale2 shapes do not match w_fp4")
    if slab_of is not None:
        _req(slab_of, "slab_of", torch.int32, 1)
        E = slab_of.shape[0]
    elif E is None:
        E = S
    R = a_q.shape[0]
    _check_plan(plan, E, R)
    if a_q.shape[1] != K:
        raise ValueError("a_q has the wrong K")
    n_out = N // 2 if epilogue == EPI_SILU_MUL else N
    if out is None:
        out = torch.empty(R, n_out, dtype=out_dtype, device=a_q.device)
    odt = MOEQ_BF16 if out.dtype == torch.bfloat16 else MOEQ_F32
    _check("moe_grouped_gemm_nvfp4", lib.moe_grouped_gemm_nvfp4(
        _ptr(a_q), _ptr(a_s), _ptr(plan), plan.numel() * 4, E, R, _ptr(slab_of), S, _ptr(w_fp4),
        _ptr(w_block_scale), _ptr(w_scale2), N, K, epilogue, _ptr(out), odt, _stream(a_q.device)))
    return out


def moe_grouped_gemm_aqlm(a_q: torch.Tensor, a_s: torch.Tensor, plan: torch.Tensor,
                          codes: list, codebooks: list, row_scale: torch.Tensor,
                          epilogue: int = EPI_NONE, out_dtype=torch.bfloat16,
                          out: Optional[torch.Tensor] = None,
                          slab_of: Optional[torch.Tensor] = None,
                          E: Optional[int] = None) -> torch.Tensor:
    """codes: list (1 or 2) of [S, N, K/8] uint8 (book of <= 256 entries) or int16;
    codebooks: list of fp16 [entries, 8]; row_scale [S, N] fp16; slab_of as for
    moe_grouped_gemm_nvfp4."""
    _req(a_q, "a_q", torch.uint8, 2)
    _req(a_s, "a_s", torch.float32, 1)
    _req(row_scale, "row_scale", torch.float16, 2)
    nb = len(codes)
    if nb != len(codebooks) or nb not in (1, 2):
        raise ValueError("one or two books, with one code tensor each")
    S, N = row_scale.shape
    R, K = a_q.shape
    for c, bk in zip(codes, codebooks):
        _req(bk, "codebook", torch.float16, 2)
        _req(c, "codes", torch.int16 if bk.shape[0] > 256 else torch.uint8, 3)
        if tuple(c.shape) != (S, N, K // 8) or bk.shape[1] != 8:
            raise ValueError("codes must be [S, N, K/8] and codebooks [entries, 8]")
    if slab_of is not None:
        _req(slab_of, "slab_of", torch.int32, 1)
        E = slab_of.shape[0]
    elif E is None:
        E = S
    _check_plan(plan, E, R)
    n_out = N // 2 if epilogue == EPI_SILU_MUL else N
    if out is None:
        out = torch.empty(R, n_out, dtype=out_dtype, device=a_q.device)
    odt = MOEQ_BF16 if out.dtype == torch.bfloat16 else MOEQ_F32
    cptr = (ctypes.c_void_p * nb)(*[c.data_ptr() for c in codes])
    bptr = (ctypes.c_void_p * nb)(*[b.data_ptr() for b in codebooks])
    ents = (ctypes.c_int * nb)(*[b.shape[0] for b in codebooks])
    _check("moe_grouped_gemm_aqlm", lib.moe_grouped_gemm_aqlm(
        _ptr(a_q), _ptr(a_s), _ptr(plan), plan.numel() * 4, E, R, _ptr(slab_of), S, nb, cptr,
        ents, bptr, _ptr(row_scale), N, K, epilogue, _ptr(out), odt, _stream(a_q.device)))
    return out


def moe_grouped_gemm_fp8row(a_q: torch.Tensor, a_s: torch.Tensor, plan: torch.Tensor,
                            w_fp8: torch.Tensor, w_row_scale: torch.Tensor,
                            epilogue: int = EPI_NONE, out_dtype=torch.bfloat16,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w_fp8 [E, N, K] uint8 (E4M3 bytes), w_row_scale [E, N] fp32."""
    _req(w_fp8, "w_fp8", torch.uint8, 3)
    _req(w_row_scale, "w_row_scale", torch.float32, 2)
    E, N, K = w_fp8.shape
    if tuple(w_row_scale.shape) != (E, N):
        raise ValueError("w_row_scale shape does not match w_fp8")
    return _gemm("moe_grouped_gemm_fp8row", a_q, a_s, plan, E, w_fp8, w_row_scale, N, K,
                 epilogue, out_dtype, out)


def _expert_mlp(fn_name: str, xp_q, xp_s, plan, E, w13, s13, w2, s2, H, I, out):
    _req(xp_q, "xp_q", torch.uint8, 2)
    _req(xp_s, "xp_s", torch.float32, 1)
    R = xp_q.shape[0]
    _check_plan(plan, E, R)
    if xp_q.shape[1] != H:
        raise ValueError("xp_q has the wrong H")
    dev = xp_q.device
    o = dict(out) if out is not None else {}
    _out(o, "h", (R, I), torch.bfloat16, dev)
    _out(o, "h_q", (R, I), torch.uint8, dev)
    _out(o, "h_s", (R,), torch.float32, dev)
    _out(o, "o", (R, H), torch.bfloat16, dev)
    fn = getattr(lib, fn_name)
    _check(fn_name, fn(_ptr(xp_q), _ptr(xp_s), _ptr(plan), plan.numel() * 4, E, R, _ptr(w13),
                       _ptr(s13), _ptr(w2), _ptr(s2), H, I, _ptr(o["h"]), _ptr(o["h_q"]),
                       _ptr(o["h_s"]), _ptr(o["o"]), _stream(dev)))
    return o


def _w4_mlp_shapes(w13, w13_scales, w2, w2_scales, scale_dtype=None) -> Tuple[int, int, int]:
    """(E, H, I) of tiled INT4 w13 [2I x H] and w2 [H x I] with their group scales."""
    E, N13, H = _tiled_int4(w13, "w13")
    E2, H2, I = _tiled_int4(w2, "w2")
    sdt = scale_dtype or (torch.bfloat16 if w13_scales.dtype == torch.bfloat16 else torch.float32)
    for t, name in ((w13_scales, "w13_scales"), (w2_scales, "w2_scales")):
        _req(t, name, sdt, 3)
    if (E2, H2, N13) != (E, H, 2 * I) or tuple(w13_scales.shape) != (E, N13, H // 128) or \
            tuple(w2_scales.shape) != (E, H, I // 128):
        raise ValueError("w13 / w2 / scale shapes do not match")
    return E, H, I


def moe_expert_mlp_w4a8(xp_q: torch.Tensor, xp_s: torch.Tensor, plan: torch.Tensor,
                        w13: torch.Tensor, w13_scales: torch.Tensor, w2: torch.Tensor,
                        w2_scales: torch.Tensor, out: Optional[dict] = None) -> dict:
    """gate/up GEMM + SiLU, FP8 quantization of h, down GEMM (two launches for R <= 192
    and I <= 2048, else three).
    w13 (2I x H) and w2 (H x I) INT4 weights in the tiled order (tile_int4_weights),
    w13_scales [E, 2I, H/128], w2_scales [E, H, I/128]; scales fp32, or both
    bfloat16 (then moe_expert_mlp_w4a8_bf16s).
    Returns a dict with h, h_q, h_s, o (reusing `out`'s tensors)."""
    E, H, I = _w4_mlp_shapes(w13, w13_scales, w2, w2_scales)
    sdt = w13_scales.dtype
    name = "moe_expert_mlp_w4a8_bf16s" if sdt == torch.bfloat16 else "moe_expert_mlp_w4a8"
    return _expert_mlp(name, xp_q, xp_s, plan, E, w13, w13_scales, w2, w2_scales, H, I, out)


def moe_expert_mlp_w4a8_noalloc(xp_q: torch.Tensor, xp_s: torch.Tensor, plan: torch.Tensor,
                                w13: torch.Tensor, w13_scales: torch.Tensor, w2: torch.Tensor,
                                w2_scales: torch.Tensor,
                                o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_expert_mlp_w4a8 (fp32 group scales) with h, h_q, h_s in the library's own
    per-GPU scratch array: the C call allocates nothing.  Returns o [R, H] bf16 (a
    new tensor unless `o` is given).  Calls overlapping on one GPU race on the array."""
    E, H, I = _w4_mlp_shapes(w13, w13_scales, w2, w2_scales, torch.float32)
    _req(xp_q, "xp_q", torch.uint8, 2)
    _req(xp_s, "xp_s", torch.float32, 1)
    R = xp_q.shape[0]
    _check_plan(plan, E, R)
    if xp_q.shape[1] != H:
        raise ValueError("xp_q has the wrong H")
    if o is None:
        o = torch.empty(R, H, dtype=torch.bfloat16, device=xp_q.device)
    _req(o, "o", torch.bfloat16, 2)
    _check("moe_expert_mlp_w4a8_noalloc", lib.moe_expert_mlp_w4a8_noalloc(
        _ptr(xp_q), _ptr(xp_s), _ptr(plan), plan.numel() * 4, E, R, _ptr(w13), _ptr(w13_scales),
        _ptr(w2), _ptr(w2_scales), H, I, _ptr(o), _stream(xp_q.device)))
    return o


def moe_expert_mlp_w4a8_bf16s(xp_q, xp_s, plan, w13, w13_scales, w2, w2_scales, out=None) -> dict:
    """moe_expert_mlp_w4a8 with bfloat16 group scales."""
    _req(w13_scales, "w13_scales", torch.bfloat16, 3)
    return moe_expert_mlp_w4a8(xp_q, xp_s, plan, w13, w13_scales, w2, w2_scales, out)


def moe_expert_mlp_fp8row(xp_q: torch.Tensor, xp_s: torch.Tensor, plan: torch.Tensor,
                          w13: torch.Tensor, w13_scales: torch.Tensor, w2: torch.Tensor,
                          w2_scales: torch.Tensor, out: Optional[dict] = None) -> dict:
    """moe_expert_mlp_w4a8 with E4M3 weights: w13 [E, 2I, H], w13_scales [E, 2I],
    w2 [E, H, I], w2_scales [E, H]."""
    for t, name in ((w13, "w13"), (w2, "w2")):
        _req(t, name, torch.uint8, 3)
    for t, name in ((w13_scales, "w13_scales"), (w2_scales, "w2_scales")):
        _req(t, name, torch.float32, 2)
    E, N13, H = w13.shape
    I = N13 // 2
    if tuple(w2.shape) != (E, H, I) or tuple(w13_scales.shape) != (E, N13) or \
            tuple(w2_scales.shape) != (E, H):
        raise ValueError("w13 / w2 / scale shapes do not match")
    return _expert_mlp("moe_expert_mlp_fp8row", xp_q, xp_s, plan, E, w13, w13_scales, w2,
                       w2_scales, H, I, out)


def moe_combine(o: torch.Tensor, plan: torch.Tensor, topk_w: torch.Tensor,
                shared: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                E: Optional[int] = None):
    """y [T, H] bf16 = sum_j topk_w[t, j] * o[row_pos[t*k + j]] (+ shared).  The plan was
    built for E experts and R = T*k rows; E=None takes it from a plan this binding built."""
    _req(o, "o", torch.bfloat16, 2)
    _req(topk_w, "topk_w", torch.float32, 2)
    T, k = topk_w.shape
    if E is None:
        built = getattr(plan, "_moeq_shape", None)
        if built is None:
            raise ValueError("moe_combine needs E for a plan not built by this binding")
        E = built[0]
    _check_plan(plan, E, T * k)
    if o.shape[0] != T * k:
        raise ValueError("o must have T*k rows")
    H = o.shape[1]
    if shared is not None:
        _req(shared, "shared", torch.bfloat16, 2)
    if y is None:
        y = torch.empty(T, H, dtype=torch.bfloat16, device=o.device)
    _check("moe_combine", lib.moe_combine(_ptr(o), _ptr(plan), plan.numel() * 4, E, _ptr(topk_w),
                                          _ptr(shared), T, k, H, _ptr(y), _stream(o.device)))
    return y


def moe_shared_gemm_bf16(a: torch.Tensor, w: torch.Tensor, epilogue: int = EPI_NONE,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _req(a, "a", torch.bfloat16, 2)
    _req(w, "w", torch.bfloat16, 2)
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("K mismatch")
    if out is None:
        out = torch.empty(M, N // 2 if epilogue == EPI_SILU_MUL else N, dtype=torch.bfloat16,
                          device=a.device)
    _check("moe_shared_gemm_bf16", lib.moe_shared_gemm_bf16(_ptr(a), _ptr(w), M, N, K, epilogue,
                                                            _ptr(out), _stream(a.device)))
    return out


from .layer import HybridMoELayer, MoELayer  # noqa: E402,F401  (composition of the calls above)
