"""Python binding of the MI355X MXFP4 sparse-MoE library (libmoe_mi355x.so).

Argument marshalling only: every step of the layer runs in the HIP kernels behind
the C ABI declared in include/moe.h. torch provides device memory and the
current stream; no torch operator computes any part of the layer here, and there
is no fallback: if the library is missing or a call fails, an exception says so.

The names follow the C ABI: route, permute, expert_ffn_mxfp4, combine (plus
rmsnorm, residual_add and the fused block glue for a pre-norm stack, and
workspace_bytes).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch  # imported before the library so that it binds to torch's HIP runtime

__all__ = [
    "MoeError", "Dims", "MXFP4", "library_path", "lib", "workspace_bytes", "route",
    "permute", "expert_ffn_mxfp4", "combine", "rmsnorm", "residual_add", "residual_rmsnorm", "forward",
    "ExpertWeights", "EXPORTED", "pack_mxfp4", "packed_bytes", "load_expert_weights",
    "forward_calls", "expert_ffn_mxfp4_stage", "forward_noalloc", "Fp8Weights",
    "convert_mxfp4_to_fp8", "pack_fp8", "load_fp8_weights", "fp8_from_mxfp4", "expert_ffn_fp8",
    "round_weights_bf16", "AttnDims", "attention_workspace_bytes", "attention_sink",
    "combine_residual_rmsnorm", "forward_residual_rmsnorm",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoe_mi355x.so"
EXPORTED = (
    "moe_workspace_bytes", "moe_route", "moe_permute", "moe_expert_ffn_mxfp4", "moe_combine",
    "moe_rmsnorm", "moe_residual_add", "moe_status_string", "moe_last_error",
    "moe_mxfp4_packed_bytes", "moe_pack_mxfp4", "moe_forward", "moe_expert_ffn_mxfp4_stage",
    "moe_forward_noalloc", "moe_forward_noalloc_max_bytes",
    "moe_convert_mxfp4_to_fp8", "moe_fp8_packed_bytes", "moe_pack_fp8", "moe_expert_ffn_fp8",
    "moe_round_weights_bf16", "moe_attention_workspace_bytes", "moe_attention_sink",
    "moe_residual_rmsnorm", "moe_combine_residual_rmsnorm", "moe_forward_residual_rmsnorm",
)


class MoeError(RuntimeError):
    pass


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("F", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32)]


class AttnDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Tq", ctypes.c_int32), ("S", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("window", ctypes.c_int32)]


class MXFP4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


def library_path() -> str:
    return os.environ.get("MOE_MI355X_LIB", os.path.join(_HERE, _LIB_NAME))


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise MoeError(f"{path} not found: build it with "
                       f"`python -m sparse_moe_transformer_gemm_amd.build`")
    L = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    L.moe_workspace_bytes.argtypes = [Dims]
    L.moe_workspace_bytes.restype = sz
    L.moe_route.argtypes = [Dims, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_permute.argtypes = [Dims, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn_mxfp4.argtypes = [Dims, vp, vp, vp, MXFP4, MXFP4, MXFP4, vp, vp, vp, vp,
                                       vp, sz, vp]
    L.moe_expert_ffn_mxfp4_stage.argtypes = [Dims, vp, vp, vp, MXFP4, MXFP4, MXFP4, vp, vp, vp, vp,
                                             i32, vp, sz, vp]
    L.moe_combine.argtypes = [Dims, vp, vp, vp, vp, vp]
    L.moe_forward.argtypes = [Dims, vp, vp, vp, MXFP4, MXFP4, MXFP4, vp, vp, vp, vp, vp, vp, vp,
                              vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward_noalloc.argtypes = [Dims, vp, vp, vp, MXFP4, MXFP4, MXFP4, vp, vp, vp, vp, vp,
                                      vp, vp, vp, vp, vp, vp, vp]
    L.moe_forward_noalloc_max_bytes.argtypes = []
    L.moe_forward_noalloc_max_bytes.restype = sz
    L.moe_convert_mxfp4_to_fp8.argtypes = [i32, i32, i32, MXFP4, vp, vp, vp]
    L.moe_fp8_packed_bytes.argtypes = [i32, i32, i32]
    L.moe_fp8_packed_bytes.restype = sz
    L.moe_pack_fp8.argtypes = [i32, i32, i32, vp, vp, vp]
    L.moe_expert_ffn_fp8.argtypes = [Dims, vp, vp, vp, MXFP4, MXFP4, MXFP4, vp, vp, vp, vp, vp, sz, vp]
    L.moe_round_weights_bf16.argtypes = [i32, i32, vp, vp]
    L.moe_attention_workspace_bytes.argtypes = [AttnDims]
    L.moe_attention_workspace_bytes.restype = sz
    L.moe_attention_sink.argtypes = [AttnDims, vp, vp, vp, vp, ctypes.c_float, vp, vp, sz, vp]
    L.moe_mxfp4_packed_bytes.argtypes = [i32, i32, i32, i32]
    L.moe_mxfp4_packed_bytes.restype = sz
    L.moe_pack_mxfp4.argtypes = [i32, i32, i32, MXFP4, vp, vp, vp]
    L.moe_rmsnorm.argtypes = [i32, i32, vp, vp, ctypes.c_float, vp, vp]
    L.moe_residual_add.argtypes = [i32, i32, vp, vp, vp, vp]
    L.moe_residual_rmsnorm.argtypes = [i32, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    L.moe_combine_residual_rmsnorm.argtypes = [Dims, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                               vp]
    L.moe_forward_residual_rmsnorm.argtypes = [Dims, vp, vp, vp, MXFP4, MXFP4, MXFP4, vp, vp, vp, vp,
                                               vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                               vp, vp, vp, sz, vp]
    for f in ("moe_route", "moe_permute", "moe_expert_ffn_mxfp4", "moe_expert_ffn_mxfp4_stage",
              "moe_combine", "moe_rmsnorm",
              "moe_residual_add", "moe_pack_mxfp4", "moe_forward", "moe_forward_noalloc",
              "moe_convert_mxfp4_to_fp8", "moe_pack_fp8", "moe_expert_ffn_fp8", "moe_round_weights_bf16",
              "moe_attention_sink", "moe_residual_rmsnorm", "moe_combine_residual_rmsnorm",
              "moe_forward_residual_rmsnorm"):
        getattr(L, f).restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise MoeError(f"{what}: {L.moe_status_string(status).decode()} "
                       f"({status}): {L.moe_last_error().decode()}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype, shape, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


@dataclass
class ExpertWeights:
    """Device tensors of one MoE layer: the fp32 router, the three MXFP4 expert
    tensors in the packed layout of moe_pack_mxfp4 (flat uint8), the bf16 biases."""
    d: int
    F: int
    E: int
    w_router: torch.Tensor            # fp32 [d][E]
    b_router: Optional[torch.Tensor]  # fp32 [E] or None
    gate_codes: torch.Tensor          # packed, from codes [E][F][d/2]
    gate_scales: torch.Tensor         # packed, from scales [E][F][d/32]
    up_codes: torch.Tensor
    up_scales: torch.Tensor
    down_codes: torch.Tensor          # packed, from codes [E][d][F/2]
    down_scales: torch.Tensor
    b_gate: torch.Tensor              # bf16 [E][F]
    b_up: torch.Tensor                # bf16 [E][F]
    b_down: torch.Tensor              # bf16 [E][d]

    @property
    def dims(self):
        return self.d, self.F, self.E


def packed_bytes(E: int, N: int, K: int) -> tuple:
    """(code bytes, scale bytes) of the packed form of an [E][N][K] MXFP4 tensor."""
    L = lib()
    c, s = L.moe_mxfp4_packed_bytes(E, N, K, 0), L.moe_mxfp4_packed_bytes(E, N, K, 1)
    if c == 0 or s == 0:
        raise MoeError(f"unsupported MXFP4 tensor shape E={E} N={N} K={K}")
    return c, s


def pack_mxfp4(codes: torch.Tensor, scales: torch.Tensor):
    """Repack an MXFP4 tensor (codes uint8 [E][N][K/2], scales uint8 [E][N][K/32],
    OCP layout) into the packed layout; returns two new flat uint8 device tensors."""
    E, N, Kh = codes.shape
    K = 2 * Kh
    c_bytes, s_bytes = packed_bytes(E, N, K)
    pc = torch.empty(c_bytes, dtype=torch.uint8, device=codes.device)
    ps = torch.empty(s_bytes, dtype=torch.uint8, device=codes.device)
    src = MXFP4(_dev(codes, torch.uint8, (E, N, K // 2), "codes"),
                _dev(scales, torch.uint8, (E, N, K // 32), "scales"))
    _check(lib().moe_pack_mxfp4(E, N, K, src, pc.data_ptr(), ps.data_ptr(), _stream()),
           "moe_pack_mxfp4")
    return pc, ps


def load_expert_weights(w_router, b_router, gate_codes, gate_scales, up_codes, up_scales,
                        down_codes, down_scales, b_gate, b_up, b_down) -> ExpertWeights:
    """ExpertWeights from device tensors in the OCP layout (include/moe.h): the
    expert tensors are packed once here; the raw ones may be freed afterwards."""
    d, E = w_router.shape
    F = gate_codes.shape[1]
    gc, gs = pack_mxfp4(gate_codes, gate_scales)
    uc, us = pack_mxfp4(up_codes, up_scales)
    dc, ds = pack_mxfp4(down_codes, down_scales)
    return ExpertWeights(d=int(d), F=int(F), E=int(E), w_router=w_router, b_router=b_router,
                         gate_codes=gc, gate_scales=gs, up_codes=uc, up_scales=us,
                         down_codes=dc, down_scales=ds, b_gate=b_gate, b_up=b_up, b_down=b_down)


def _dims(T, d, F, E, k) -> Dims:
    return Dims(int(T), int(d), int(F), int(E), int(k))


def workspace_bytes(T: int, d: int, F: int, E: int, k: int) -> int:
    n = lib().moe_workspace_bytes(_dims(T, d, F, E, k))
    if n == 0:
        raise MoeError(f"unsupported dims T={T} d={d} F={F} E={E} k={k}")
    return n


def route(x, w_router, b_router, k: int, ws, topk_idx=None, topk_w=None):
    T, d = x.shape
    E = w_router.shape[1]
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    dims = _dims(T, d, 64, E, k)
    b = None if b_router is None else _dev(b_router, torch.float32, (E,), "b_router")
    _check(lib().moe_route(dims, _dev(x, torch.bfloat16, (T, d), "x"),
                           _dev(w_router, torch.float32, (d, E), "w_router"), b,
                           _dev(topk_idx, torch.int32, (T, k), "topk_idx"),
                           _dev(topk_w, torch.float32, (T, k), "topk_w"),
                           ws.data_ptr(), ws.numel() * ws.element_size(), _stream()), "moe_route")
    return topk_idx, topk_w


def permute(topk_idx, E: int, ws, out=None):
    T, k = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev))
    counts, offsets, sorted_pair, pair_row = out
    _check(lib().moe_permute(_dims(T, 64, 64, E, k), _dev(topk_idx, torch.int32, (T, k), "topk_idx"),
                             _dev(counts, torch.int32, (E,), "counts"),
                             _dev(offsets, torch.int32, (E + 1,), "offsets"),
                             _dev(sorted_pair, torch.int32, (T * k,), "sorted_pair"),
                             _dev(pair_row, torch.int32, (T * k,), "pair_row"),
                             ws.data_ptr(), ws.numel() * ws.element_size(), _stream()),
           "moe_permute")
    return counts, offsets, sorted_pair, pair_row


def _packed_args(w: ExpertWeights):
    d, F, E = w.dims
    u8 = torch.uint8
    gb, ub = packed_bytes(E, F, d), packed_bytes(E, d, F)
    mg = MXFP4(_dev(w.gate_codes, u8, (gb[0],), "gate_codes"),
               _dev(w.gate_scales, u8, (gb[1],), "gate_scales"))
    mu = MXFP4(_dev(w.up_codes, u8, (gb[0],), "up_codes"),
               _dev(w.up_scales, u8, (gb[1],), "up_scales"))
    md = MXFP4(_dev(w.down_codes, u8, (ub[0],), "down_codes"),
               _dev(w.down_scales, u8, (ub[1],), "down_scales"))
    return mg, mu, md


def expert_ffn_mxfp4(x, sorted_pair, offsets, w: ExpertWeights, k: int, ws, y_sorted=None):
    T, d = x.shape
    dw, F, E = w.dims
    if dw != d:
        raise ValueError("x width does not match the router weight")
    P = T * k
    if y_sorted is None:
        y_sorted = torch.empty((P, d), dtype=torch.float32, device=x.device)
    mg, mu, md = _packed_args(w)
    _check(lib().moe_expert_ffn_mxfp4(
        _dims(T, d, F, E, k), _dev(x, torch.bfloat16, (T, d), "x"),
        _dev(sorted_pair, torch.int32, (P,), "sorted_pair"),
        _dev(offsets, torch.int32, (E + 1,), "offsets"), mg, mu, md,
        _dev(w.b_gate, torch.bfloat16, (E, F), "b_gate"),
        _dev(w.b_up, torch.bfloat16, (E, F), "b_up"),
        _dev(w.b_down, torch.bfloat16, (E, d), "b_down"),
        _dev(y_sorted, torch.float32, (P, d), "y_sorted"),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream()), "moe_expert_ffn_mxfp4")
    return y_sorted


def expert_ffn_mxfp4_stage(x, sorted_pair, offsets, w: ExpertWeights, k: int, ws, y_sorted, stage: int):
    """One stage of expert_ffn_mxfp4 (0: encode x and build the tile tables,
    1: gate/up GEMM + SwiGLU, 2: down GEMM into y_sorted); the three in order
    with the same arguments are expert_ffn_mxfp4."""
    T, d = x.shape
    dw, F, E = w.dims
    if dw != d:
        raise ValueError("x width does not match the router weight")
    P = T * k
    mg, mu, md = _packed_args(w)
    _check(lib().moe_expert_ffn_mxfp4_stage(
        _dims(T, d, F, E, k), _dev(x, torch.bfloat16, (T, d), "x"),
        _dev(sorted_pair, torch.int32, (P,), "sorted_pair"),
        _dev(offsets, torch.int32, (E + 1,), "offsets"), mg, mu, md,
        _dev(w.b_gate, torch.bfloat16, (E, F), "b_gate"),
        _dev(w.b_up, torch.bfloat16, (E, F), "b_up"),
        _dev(w.b_down, torch.bfloat16, (E, d), "b_down"),
        _dev(y_sorted, torch.float32, (P, d), "y_sorted"), int(stage),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream()), "moe_expert_ffn_mxfp4_stage")
    return y_sorted


# --------------------------------------------------------------------------- FP8 weights
# moe_fp8 has the same two pointers as moe_mxfp4 (codes, then float32 scales),
# so the MXFP4 ctypes structure carries it.

@dataclass
class Fp8Weights:
    """Device tensors of one MoE layer with FP8-E4M3 expert weights: the three
    expert tensors as packed codes (moe_pack_fp8, flat uint8) and float32
    128x128 block scales, the bf16 biases, and the fp32 router."""
    d: int
    F: int
    E: int
    w_router: torch.Tensor
    b_router: Optional[torch.Tensor]
    gate_codes: torch.Tensor          # packed, from codes [E][F][d]
    gate_scales: torch.Tensor         # float32 [E][ceil(F/128)][ceil(d/128)]
    up_codes: torch.Tensor
    up_scales: torch.Tensor
    down_codes: torch.Tensor          # packed, from codes [E][d][F]
    down_scales: torch.Tensor         # float32 [E][ceil(d/128)][ceil(F/128)]
    b_gate: torch.Tensor
    b_up: torch.Tensor
    b_down: torch.Tensor

    @property
    def dims(self):
        return self.d, self.F, self.E


def _nb(n: int) -> int:
    return (n + 127) // 128


def convert_mxfp4_to_fp8(codes: torch.Tensor, scales: torch.Tensor):
    """MXFP4 tensor (OCP layout: codes uint8 [E][N][K/2], scales uint8 [E][N][K/32])
    -> FP8 codes uint8 [E][N][K] and float32 block scales [E][ceil(N/128)][ceil(K/128)]."""
    E, N, Kh = codes.shape
    K = 2 * Kh
    c8 = torch.empty((E, N, K), dtype=torch.uint8, device=codes.device)
    s8 = torch.empty((E, _nb(N), _nb(K)), dtype=torch.float32, device=codes.device)
    src = MXFP4(_dev(codes, torch.uint8, (E, N, K // 2), "codes"),
                _dev(scales, torch.uint8, (E, N, K // 32), "scales"))
    _check(lib().moe_convert_mxfp4_to_fp8(E, N, K, src, c8.data_ptr(), s8.data_ptr(), _stream()),
           "moe_convert_mxfp4_to_fp8")
    return c8, s8


def pack_fp8(codes: torch.Tensor) -> torch.Tensor:
    """Repack FP8 codes uint8 [E][N][K] into the layout moe_expert_ffn_fp8 streams."""
    E, N, K = codes.shape
    n = lib().moe_fp8_packed_bytes(E, N, K)
    if n == 0:
        raise MoeError(f"unsupported FP8 tensor shape E={E} N={N} K={K}")
    out = torch.empty(n, dtype=torch.uint8, device=codes.device)
    _check(lib().moe_pack_fp8(E, N, K, _dev(codes, torch.uint8, (E, N, K), "codes"), out.data_ptr(),
                              _stream()), "moe_pack_fp8")
    return out


def load_fp8_weights(w_router, b_router, gate, up, down, b_gate, b_up, b_down) -> Fp8Weights:
    """Fp8Weights from device tensors: gate, up, down are (codes uint8 [E][N][K],
    scales float32 [E][ceil(N/128)][ceil(K/128)]); the codes are packed here."""
    d, E = w_router.shape
    F = gate[0].shape[1]
    return Fp8Weights(d=int(d), F=int(F), E=int(E), w_router=w_router, b_router=b_router,
                      gate_codes=pack_fp8(gate[0]), gate_scales=gate[1],
                      up_codes=pack_fp8(up[0]), up_scales=up[1],
                      down_codes=pack_fp8(down[0]), down_scales=down[1],
                      b_gate=b_gate, b_up=b_up, b_down=b_down)


def fp8_from_mxfp4(w_router, b_router, gate_codes, gate_scales, up_codes, up_scales, down_codes,
                   down_scales, b_gate, b_up, b_down) -> Fp8Weights:
    """The same layer as load_expert_weights, converted once to FP8 with 128x128
    block scales (moe_convert_mxfp4_to_fp8) and packed."""
    return load_fp8_weights(w_router, b_router, convert_mxfp4_to_fp8(gate_codes, gate_scales),
                            convert_mxfp4_to_fp8(up_codes, up_scales),
                            convert_mxfp4_to_fp8(down_codes, down_scales), b_gate, b_up, b_down)


def expert_ffn_fp8(x, sorted_pair, offsets, w: Fp8Weights, k: int, ws, y_sorted=None):
    T, d = x.shape
    dw, F, E = w.dims
    if dw != d:
        raise ValueError("x width does not match the router weight")
    P = T * k
    if y_sorted is None:
        y_sorted = torch.empty((P, d), dtype=torch.float32, device=x.device)
    u8, f32 = torch.uint8, torch.float32
    gb, db = lib().moe_fp8_packed_bytes(E, F, d), lib().moe_fp8_packed_bytes(E, d, F)
    mg = MXFP4(_dev(w.gate_codes, u8, (gb,), "gate_codes"),
               _dev(w.gate_scales, f32, (E, _nb(F), _nb(d)), "gate_scales"))
    mu = MXFP4(_dev(w.up_codes, u8, (gb,), "up_codes"),
               _dev(w.up_scales, f32, (E, _nb(F), _nb(d)), "up_scales"))
    md = MXFP4(_dev(w.down_codes, u8, (db,), "down_codes"),
               _dev(w.down_scales, f32, (E, _nb(d), _nb(F)), "down_scales"))
    _check(lib().moe_expert_ffn_fp8(
        _dims(T, d, F, E, k), _dev(x, torch.bfloat16, (T, d), "x"),
        _dev(sorted_pair, torch.int32, (P,), "sorted_pair"),
        _dev(offsets, torch.int32, (E + 1,), "offsets"), mg, mu, md,
        _dev(w.b_gate, torch.bfloat16, (E, F), "b_gate"),
        _dev(w.b_up, torch.bfloat16, (E, F), "b_up"),
        _dev(w.b_down, torch.bfloat16, (E, d), "b_down"),
        _dev(y_sorted, torch.float32, (P, d), "y_sorted"),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream()), "moe_expert_ffn_fp8")
    return y_sorted


def round_weights_bf16(topk_w):
    """moe_round_weights_bf16: the routing weights rounded to bf16 in place."""
    T, k = topk_w.shape
    _check(lib().moe_round_weights_bf16(T, k, _dev(topk_w, torch.float32, (T, k), "topk_w"), _stream()),
           "moe_round_weights_bf16")
    return topk_w


# --------------------------------------------------------------------------- attention

def attention_workspace_bytes(B, Tq, S, Hq, Hkv, D=64, window=0) -> int:
    return lib().moe_attention_workspace_bytes(AttnDims(B, Tq, S, Hq, Hkv, D, window))


def attention_sink(q, k, v, sinks, scale: float, window: int = 0, out=None, ws=None):
    """moe_attention_sink: q [B][Tq][Hq][D], k and v [B][S][Hkv][D] (bf16), sinks
    [Hq] (fp32) -> out [B][Tq][Hq][D] bf16."""
    B, Tq, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    dims = AttnDims(B, Tq, S, Hq, Hkv, D, window)
    if out is None:
        out = torch.empty_like(q)
    n = lib().moe_attention_workspace_bytes(dims)
    if ws is None and n:
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(lib().moe_attention_sink(
        dims, _dev(q, torch.bfloat16, (B, Tq, Hq, D), "q"), _dev(k, torch.bfloat16, (B, S, Hkv, D), "k"),
        _dev(v, torch.bfloat16, (B, S, Hkv, D), "v"), _dev(sinks, torch.float32, (Hq,), "sinks"),
        float(scale), _dev(out, torch.bfloat16, (B, Tq, Hq, D), "out"),
        None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream()), "moe_attention_sink")
    return out


def combine(y_sorted, pair_row, topk_w, out=None):
    T, k = topk_w.shape
    P, d = y_sorted.shape
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=y_sorted.device)
    _check(lib().moe_combine(_dims(T, d, 64, max(k, 1), k),
                             _dev(y_sorted, torch.float32, (T * k, d), "y_sorted"),
                             _dev(pair_row, torch.int32, (T * k,), "pair_row"),
                             _dev(topk_w, torch.float32, (T, k), "topk_w"),
                             _dev(out, torch.bfloat16, (T, d), "out"), _stream()), "moe_combine")
    return out


def rmsnorm(x, gain, eps: float = 1e-5, out=None):
    T, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib().moe_rmsnorm(T, d, _dev(x, torch.bfloat16, (T, d), "x"),
                             _dev(gain, torch.bfloat16, (d,), "gain"), float(eps),
                             _dev(out, torch.bfloat16, (T, d), "out"), _stream()), "moe_rmsnorm")
    return out


def residual_add(x, m, out=None):
    T, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib().moe_residual_add(T, d, _dev(x, torch.bfloat16, (T, d), "x"),
                                  _dev(m, torch.bfloat16, (T, d), "m"),
                                  _dev(out, torch.bfloat16, (T, d), "out"), _stream()),
           "moe_residual_add")
    return out


def residual_rmsnorm(x, m, gain, eps: float = 1e-5, x_out=None, n_out=None):
    """x_out = x + m (bf16), n_out = rmsnorm(x_out): moe_residual_rmsnorm.
    Returns (x_out, n_out); x_out may be x itself (in place)."""
    T, d = x.shape
    if x_out is None:
        x_out = torch.empty_like(x)
    if n_out is None:
        n_out = torch.empty_like(x)
    _check(lib().moe_residual_rmsnorm(T, d, _dev(x, torch.bfloat16, (T, d), "x"),
                                      _dev(m, torch.bfloat16, (T, d), "m"),
                                      _dev(gain, torch.bfloat16, (d,), "gain"), float(eps),
                                      _dev(x_out, torch.bfloat16, (T, d), "x_out"),
                                      _dev(n_out, torch.bfloat16, (T, d), "n_out"), _stream()),
           "moe_residual_rmsnorm")
    return x_out, n_out


def combine_residual_rmsnorm(y_sorted, pair_row, topk_w, resid, gain, eps: float = 1e-5,
                             resid_out=None, n_out=None, m_out=None):
    """m = combine(y), resid_out = resid + m, n_out = rmsnorm(resid_out) in one pass
    (moe_combine_residual_rmsnorm). gain None: no norm (n_out None). m_out, if
    given, receives m. Returns (resid_out, n_out); resid_out may be resid."""
    T, k = topk_w.shape
    P, d = y_sorted.shape
    if resid_out is None:
        resid_out = torch.empty_like(resid)
    if gain is not None and n_out is None:
        n_out = torch.empty_like(resid)
    _check(lib().moe_combine_residual_rmsnorm(
        _dims(T, d, 64, max(k, 1), k), _dev(y_sorted, torch.float32, (T * k, d), "y_sorted"),
        _dev(pair_row, torch.int32, (T * k,), "pair_row"), _dev(topk_w, torch.float32, (T, k), "topk_w"),
        _dev(resid, torch.bfloat16, (T, d), "resid"),
        None if gain is None else _dev(gain, torch.bfloat16, (d,), "gain"), float(eps),
        None if m_out is None else _dev(m_out, torch.bfloat16, (T, d), "m_out"),
        _dev(resid_out, torch.bfloat16, (T, d), "resid_out"),
        None if n_out is None else _dev(n_out, torch.bfloat16, (T, d), "n_out"), _stream()),
        "moe_combine_residual_rmsnorm")
    return resid_out, n_out


def _outputs(T, d, E, k, dev, bufs: Optional[dict], store_out: bool = True) -> dict:
    b = dict(bufs or {})
    P = T * k
    if b.get("topk_idx") is None:
        b["topk_idx"] = torch.empty((T, k), dtype=torch.int32, device=dev)
    if b.get("topk_w") is None:
        b["topk_w"] = torch.empty((T, k), dtype=torch.float32, device=dev)
    if b.get("perm") is None:
        b["perm"] = (torch.empty(E, dtype=torch.int32, device=dev),
                     torch.empty(E + 1, dtype=torch.int32, device=dev),
                     torch.empty(P, dtype=torch.int32, device=dev),
                     torch.empty(P, dtype=torch.int32, device=dev))
    if b.get("y_sorted") is None:
        b["y_sorted"] = torch.empty((P, d), dtype=torch.float32, device=dev)
    if b.get("out") is None and store_out:
        b["out"] = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    b.setdefault("out", None)
    return b


def forward(x, w: ExpertWeights, k: int, ws, bufs: Optional[dict] = None) -> dict:
    """The whole block in one call (moe_forward) on the current stream. `bufs`, if
    given, supplies preallocated outputs (keys as in the returned dict)."""
    return _forward(x, w, k, ws, bufs)


def forward_noalloc(x, w: ExpertWeights, k: int, bufs: Optional[dict] = None) -> dict:
    """moe_forward_noalloc: the whole block with the library's own scratch array
    instead of a workspace (the outputs are still the caller's: pass them in
    `bufs` to allocate nothing at all)."""
    return _forward(x, w, k, None, bufs)


def forward_residual_rmsnorm(x, w: ExpertWeights, k: int, ws, resid, gain, eps: float = 1e-5,
                             resid_out=None, n_out=None, bufs: Optional[dict] = None,
                             store_out: bool = False) -> dict:
    """One block of a pre-norm stack after its norm (moe_forward_residual_rmsnorm):
    the whole block on the normalised input x, then resid_out = resid + MoE(x) and
    n_out = rmsnorm(resid_out, gain) (no norm when gain is None). The block output
    itself is stored only with store_out (key "out"). Returns the dict of
    `forward` plus resid_out and n_out."""
    T, d = x.shape
    if resid_out is None:
        resid_out = torch.empty_like(resid)
    if gain is not None and n_out is None:
        n_out = torch.empty_like(resid)
    rn = (_dev(resid, torch.bfloat16, (T, d), "resid"),
          None if gain is None else _dev(gain, torch.bfloat16, (d,), "gain"), float(eps),
          _dev(resid_out, torch.bfloat16, (T, d), "resid_out"),
          None if n_out is None else _dev(n_out, torch.bfloat16, (T, d), "n_out"))
    r = _forward(x, w, k, ws, bufs, resid_norm=rn, store_out=store_out)
    r["resid_out"], r["n_out"] = resid_out, n_out
    return r


def _forward(x, w: ExpertWeights, k: int, ws, bufs: Optional[dict], resid_norm=None,
             store_out: bool = True) -> dict:
    T, d = x.shape
    dw, F, E = w.dims
    if dw != d:
        raise ValueError("x width does not match the router weight")
    P = T * k
    b = _outputs(T, d, E, k, x.device, bufs, store_out)
    counts, offsets, sorted_pair, pair_row = b["perm"]
    mg, mu, md = _packed_args(w)
    br = None if w.b_router is None else _dev(w.b_router, torch.float32, (E,), "b_router")
    args = [
        _dims(T, d, F, E, k), _dev(x, torch.bfloat16, (T, d), "x"),
        _dev(w.w_router, torch.float32, (d, E), "w_router"), br, mg, mu, md,
        _dev(w.b_gate, torch.bfloat16, (E, F), "b_gate"),
        _dev(w.b_up, torch.bfloat16, (E, F), "b_up"),
        _dev(w.b_down, torch.bfloat16, (E, d), "b_down"),
        _dev(b["topk_idx"], torch.int32, (T, k), "topk_idx"),
        _dev(b["topk_w"], torch.float32, (T, k), "topk_w"),
        _dev(counts, torch.int32, (E,), "counts"),
        _dev(offsets, torch.int32, (E + 1,), "offsets"),
        _dev(sorted_pair, torch.int32, (P,), "sorted_pair"),
        _dev(pair_row, torch.int32, (P,), "pair_row"),
        _dev(b["y_sorted"], torch.float32, (P, d), "y_sorted"),
        None if b["out"] is None else _dev(b["out"], torch.bfloat16, (T, d), "out")]
    if resid_norm is not None:
        _check(lib().moe_forward_residual_rmsnorm(*args, *resid_norm, ws.data_ptr(),
                                                  ws.numel() * ws.element_size(), _stream()),
               "moe_forward_residual_rmsnorm")
    elif ws is None:
        _check(lib().moe_forward_noalloc(*args, _stream()), "moe_forward_noalloc")
    else:
        _check(lib().moe_forward(*args, ws.data_ptr(), ws.numel() * ws.element_size(), _stream()),
               "moe_forward")
    return dict(topk_idx=b["topk_idx"], topk_w=b["topk_w"], perm=b["perm"],
                y_sorted=b["y_sorted"], out=b["out"])


def forward_calls(x, w: ExpertWeights, k: int, ws, bufs: Optional[dict] = None) -> dict:
    """The whole block as the four separate calls in order on the current stream."""
    T, d = x.shape
    _, F, E = w.dims
    b = bufs or {}
    idx, tw = route(x, w.w_router, w.b_router, k, ws, b.get("topk_idx"), b.get("topk_w"))
    perm = permute(idx, E, ws, b.get("perm"))
    y = expert_ffn_mxfp4(x, perm[2], perm[1], w, k, ws, b.get("y_sorted"))
    out = combine(y, perm[3], tw, b.get("out"))
    return dict(topk_idx=idx, topk_w=tw, perm=perm, y_sorted=y, out=out)
