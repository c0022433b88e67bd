"""Python binding of the MoE FFN layer's C ABI (include/moe_ffn.h).

Argument marshalling only: every function passes device pointers of torch
tensors and the current HIP stream to the library; all computation happens in
the HIP kernels.  bf16 tensors may be torch.bfloat16 or torch.int16/uint16
views of the same bits.  Output tensors are allocated with torch (device
memory is torch's; the library never allocates).
"""
import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import MoeDims, MOE_FLAG_IDS_IN

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def dims(N: int, M: int, E: int, k: int, H: int = 64, S: int = 0, Hs: int = 0) -> MoeDims:
    return MoeDims(N, M, E, k, H, S, Hs)


def _ptr(t: Optional[torch.Tensor], dtypes=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"dtype {t.dtype} not in {dtypes}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def moe_layer_workspace_bytes(d: MoeDims, flags: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().moe_layer_workspace_bytes(ctypes.byref(d), flags, ctypes.byref(n)))
    return n.value


def moe_layer_single_launch(d: MoeDims, flags: int = 0, fp8: bool = False) -> bool:
    """Whether moe_layer (or moe_layer_fp8) runs these dims as one launch."""
    v = ctypes.c_int(0)
    _lib.check(_lib.load().moe_layer_single_launch(ctypes.byref(d), flags, int(fp8), ctypes.byref(v)))
    return bool(v.value)


def moe_route_workspace_bytes(d: MoeDims) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().moe_route_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def moe_permute_workspace_bytes(d: MoeDims) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().moe_permute_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def moe_grouped_ffn_workspace_bytes(d: MoeDims) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().moe_grouped_ffn_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def moe_route(d: MoeDims, x, w_router, router_bias=None, topk_ids=None, topk_weights=None, ws=None,
              stream=None):
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((d.n_tokens, d.top_k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((d.n_tokens, d.top_k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(moe_route_workspace_bytes(d), dev)
    _lib.check(_lib.load().moe_route(ctypes.byref(d), _ptr(x, _BF16_LIKE), _ptr(w_router, _BF16_LIKE),
                                     _ptr(router_bias, (torch.float32,)), _ptr(topk_ids, (torch.int32,)),
                                     _ptr(topk_weights, (torch.float32,)), _ptr(ws), ws.numel(),
                                     _stream(stream)))
    return topk_ids, topk_weights


def moe_permute(d: MoeDims, topk_ids, x=None, want_x_sorted: bool = False, ws=None, stream=None):
    dev = topk_ids.device
    A = d.n_tokens * d.top_k
    counts = torch.empty(d.n_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(d.n_experts + 1, dtype=torch.int32, device=dev)
    s2a = torch.empty(max(A, 1), dtype=torch.int32, device=dev)[:A]
    a2s = torch.empty(max(A, 1), dtype=torch.int32, device=dev)[:A]
    xs = torch.empty((A, d.hidden), dtype=x.dtype, device=dev) if want_x_sorted else None
    if ws is None:
        ws = workspace(moe_permute_workspace_bytes(d), dev)
    _lib.check(_lib.load().moe_permute(ctypes.byref(d), _ptr(topk_ids, (torch.int32,)),
                                       _ptr(x, _BF16_LIKE) if want_x_sorted else None,
                                       _ptr(counts), _ptr(offsets), _ptr(s2a), _ptr(a2s),
                                       _ptr(xs), _ptr(ws), ws.numel(), _stream(stream)))
    return {"expert_counts": counts, "expert_offsets": offsets, "sorted_to_assign": s2a,
            "assign_to_sorted": a2s, "x_sorted": xs}


def moe_grouped_ffn(d: MoeDims, x_sorted, expert_offsets, w_gate, w_up, w_down, row_scale=None,
                    y_sorted=None, ws=None, stream=None):
    dev = x_sorted.device
    A = d.n_tokens * d.top_k
    if y_sorted is None:
        y_sorted = torch.empty((A, d.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(moe_grouped_ffn_workspace_bytes(d), dev)
    _lib.check(_lib.load().moe_grouped_ffn(ctypes.byref(d), _ptr(x_sorted, _BF16_LIKE),
                                           _ptr(expert_offsets, (torch.int32,)), _ptr(w_gate, _BF16_LIKE),
                                           _ptr(w_up, _BF16_LIKE), _ptr(w_down, _BF16_LIKE),
                                           _ptr(row_scale, (torch.float32,)), _ptr(y_sorted, _BF16_LIKE),
                                           _ptr(ws), ws.numel(), _stream(stream)))
    return y_sorted


def moe_combine(d: MoeDims, y_sorted, assign_to_sorted, topk_weights=None, shared_out=None, out=None,
                stream=None):
    if out is None:
        out = torch.empty((d.n_tokens, d.hidden), dtype=torch.bfloat16, device=y_sorted.device)
    _lib.check(_lib.load().moe_combine(ctypes.byref(d), _ptr(y_sorted, _BF16_LIKE),
                                       _ptr(assign_to_sorted, (torch.int32,)),
                                       _ptr(topk_weights, (torch.float32,)), _ptr(shared_out, _BF16_LIKE),
                                       _ptr(out, _BF16_LIKE), _stream(stream)))
    return out


def moe_layer(d: MoeDims, x, w_gate, w_up, w_down, w_router=None, router_bias=None, ws_gate=None,
              ws_up=None, ws_down=None, topk_ids=None, topk_weights=None, ids_in: bool = False, out=None,
              ws=None, stream=None):
    dev = x.device
    flags = MOE_FLAG_IDS_IN if ids_in else 0
    if out is None:
        out = torch.empty((d.n_tokens, d.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(moe_layer_workspace_bytes(d, flags), dev)
    _lib.check(_lib.load().moe_layer(
        ctypes.byref(d), flags, _ptr(x, _BF16_LIKE), _ptr(w_router, _BF16_LIKE),
        _ptr(router_bias, (torch.float32,)), _ptr(w_gate, _BF16_LIKE), _ptr(w_up, _BF16_LIKE),
        _ptr(w_down, _BF16_LIKE), _ptr(ws_gate, _BF16_LIKE), _ptr(ws_up, _BF16_LIKE),
        _ptr(ws_down, _BF16_LIKE), _ptr(topk_ids, (torch.int32,)), _ptr(topk_weights, (torch.float32,)),
        _ptr(out, _BF16_LIKE), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_layer_noalloc(d: MoeDims, x, w_gate, w_up, w_down, w_router=None, router_bias=None, ws_gate=None,
                      ws_up=None, ws_down=None, topk_ids=None, topk_weights=None, ids_in: bool = False, out=None,
                      stream=None):
    """moe_layer with the library's own workspace array: nothing is
    allocated for the call except `out` when the caller passes none."""
    dev = x.device
    flags = MOE_FLAG_IDS_IN if ids_in else 0
    if out is None:
        out = torch.empty((d.n_tokens, d.hidden), dtype=torch.bfloat16, device=dev)
    _lib.check(_lib.load().moe_layer_noalloc(
        ctypes.byref(d), flags, _ptr(x, _BF16_LIKE), _ptr(w_router, _BF16_LIKE),
        _ptr(router_bias, (torch.float32,)), _ptr(w_gate, _BF16_LIKE), _ptr(w_up, _BF16_LIKE),
        _ptr(w_down, _BF16_LIKE), _ptr(ws_gate, _BF16_LIKE), _ptr(ws_up, _BF16_LIKE),
        _ptr(ws_down, _BF16_LIKE), _ptr(topk_ids, (torch.int32,)), _ptr(topk_weights, (torch.float32,)),
        _ptr(out, _BF16_LIKE), _stream(stream)))
    return out


class Fp8Weights:
    """FP8 (OCP E4M3) expert weights with one float32 scale per output channel:
    codes `gate`/`up` [E][H][M] and `down` [E][M][H] (torch.uint8), scales
    `gate_scale`/`up_scale` [E][H] and `down_scale` [E][M] (torch.float32)."""

    FIELDS = ("gate", "up", "down", "gate_scale", "up_scale", "down_scale")

    def __init__(self, gate, up, down, gate_scale, up_scale, down_scale):
        self.gate, self.up, self.down = gate, up, down
        self.gate_scale, self.up_scale, self.down_scale = gate_scale, up_scale, down_scale

    def c_struct(self) -> _lib.MoeFp8Ffn:
        codes = [_ptr(getattr(self, n), (torch.uint8,)) for n in self.FIELDS[:3]]
        scales = [_ptr(getattr(self, n), (torch.float32,)) for n in self.FIELDS[3:]]
        return _lib.MoeFp8Ffn(*codes, *scales)


def moe_quantize_fp8(w, q=None, scale=None, stream=None):
    """Per-output-channel E4M3 quantisation of a bf16 matrix [..., cols]
    (every leading index is one output channel).  Returns (codes, scales)."""
    rows = w.numel() // w.shape[-1]
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scale is None:
        scale = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    _lib.check(_lib.load().moe_quantize_fp8(_ptr(w, _BF16_LIKE), rows, w.shape[-1], _ptr(q, (torch.uint8,)),
                                            _ptr(scale, (torch.float32,)), _stream(stream)))
    return q, scale


def quantize_ffn_fp8(w_gate, w_up, w_down, stream=None) -> Fp8Weights:
    """FP8 copies of one set of expert weights (three moe_quantize_fp8 calls)."""
    g, sg = moe_quantize_fp8(w_gate, stream=stream)
    u, su = moe_quantize_fp8(w_up, stream=stream)
    d, sd = moe_quantize_fp8(w_down, stream=stream)
    return Fp8Weights(g, u, d, sg, su, sd)


def moe_grouped_ffn_fp8(d: MoeDims, x_sorted, expert_offsets, experts: Fp8Weights, row_scale=None,
                        y_sorted=None, ws=None, stream=None):
    dev = x_sorted.device
    A = d.n_tokens * d.top_k
    if y_sorted is None:
        y_sorted = torch.empty((A, d.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(moe_grouped_ffn_workspace_bytes(d), dev)
    st = experts.c_struct()
    _lib.check(_lib.load().moe_grouped_ffn_fp8(ctypes.byref(d), _ptr(x_sorted, _BF16_LIKE),
                                               _ptr(expert_offsets, (torch.int32,)), ctypes.byref(st),
                                               _ptr(row_scale, (torch.float32,)), _ptr(y_sorted, _BF16_LIKE),
                                               _ptr(ws), ws.numel(), _stream(stream)))
    return y_sorted


def moe_layer_fp8(d: MoeDims, x, experts: Fp8Weights, shared: Optional[Fp8Weights] = None, w_router=None,
                  router_bias=None, topk_ids=None, topk_weights=None, ids_in: bool = False, out=None, ws=None,
                  stream=None):
    dev = x.device
    flags = MOE_FLAG_IDS_IN if ids_in else 0
    if out is None:
        out = torch.empty((d.n_tokens, d.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(moe_layer_workspace_bytes(d, flags), dev)
    ex = experts.c_struct()
    sh = shared.c_struct() if shared is not None else None
    _lib.check(_lib.load().moe_layer_fp8(
        ctypes.byref(d), flags, _ptr(x, _BF16_LIKE), _ptr(w_router, _BF16_LIKE),
        _ptr(router_bias, (torch.float32,)), ctypes.byref(ex), ctypes.byref(sh) if sh is not None else None,
        _ptr(topk_ids, (torch.int32,)), _ptr(topk_weights, (torch.float32,)), _ptr(out, _BF16_LIKE),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_layer_pipelined_workspace_bytes(d: MoeDims, n_micro: int, flags: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().moe_layer_pipelined_workspace_bytes(ctypes.byref(d), flags, n_micro, ctypes.byref(n)))
    return n.value


def moe_layer_pipelined(d: MoeDims, n_micro: int, x, w_gate, w_up, w_down, w_router=None, router_bias=None,
                        ws_gate=None, ws_up=None, ws_down=None, topk_ids=None, topk_weights=None,
                        ids_in: bool = False, out=None, ws=None, stream=None):
    dev = x.device
    flags = MOE_FLAG_IDS_IN if ids_in else 0
    if out is None:
        out = torch.empty((d.n_tokens, d.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(moe_layer_pipelined_workspace_bytes(d, n_micro, flags), dev)
    _lib.check(_lib.load().moe_layer_pipelined(
        ctypes.byref(d), flags, n_micro, _ptr(x, _BF16_LIKE), _ptr(w_router, _BF16_LIKE),
        _ptr(router_bias, (torch.float32,)), _ptr(w_gate, _BF16_LIKE), _ptr(w_up, _BF16_LIKE),
        _ptr(w_down, _BF16_LIKE), _ptr(ws_gate, _BF16_LIKE), _ptr(ws_up, _BF16_LIKE),
        _ptr(ws_down, _BF16_LIKE), _ptr(topk_ids, (torch.int32,)), _ptr(topk_weights, (torch.float32,)),
        _ptr(out, _BF16_LIKE), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def moe_set_stage_events(events) -> None:
    """Record the given MOE_STAGE_EVENTS torch.cuda.Event objects at the stage
    boundaries of the next moe_layer call on this thread (None clears).  The
    events must have been recorded once (torch creates them lazily)."""
    lib = _lib.load()
    if events is None:
        _lib.check(lib.moe_set_stage_events(None, 0))
        return
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _lib.check(lib.moe_set_stage_events(arr, len(events)))
