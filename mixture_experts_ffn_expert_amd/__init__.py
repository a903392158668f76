"""Python binding of libmoe.so, the MI355X (gfx950) BF16 MoE expert path.

Argument marshalling only: every step of the path runs in the HIP kernels of
libmoe.so (C ABI in include/moe.h). torch supplies device memory and the
current stream. The binding raises ``MoeError`` with the library's message
when a call is refused, and ``RuntimeError`` when the library is not built:
there is no fallback path.

Functions (same names as the C ABI):
  moe_router_logits(x, w, bias=None, out=None)                -> f32 [T, N]
  moe_route(logits, K, ...)                                   -> ids, w, offsets, sorted_pairs
  moe_route_scored(logits, K, score, selection_bias, n_group, topk_group, group_score,
                   renormalize, ...)                          -> ids, w, offsets, sorted_pairs
  moe_grouped_gemm_gateup_silu(x, w_gu, sorted_pairs, expert_offsets, K, act=None)
  moe_grouped_gemm_down(act, w_d, sorted_pairs, expert_offsets, pair_w, expert_out=None)
  moe_combine_gate(expert_out, T, K, topk_w=None, routed_scale=1.0, shared=None,
                   gate_logit=None, out=None, out_dtype=torch.bfloat16)
plus ``moe_layer`` which enqueues one whole layer, and the measurement-only
  moe_time_next_gemm(start, stop)   (torch.cuda.Event pair, or None, None)
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MoeError", "load", "lib_path", "moe_init", "PackedWeights", "moe_pack_weights",
    "moe_packed_weight_bytes", "Q8KBuffer", "QBuffer", "moe_q8k_bytes", "moe_quantize_q8k",
    "moe_q8_0_bytes", "moe_quantize_q8_0", "moe_quantize_act",
    "moe_fused_expert_ffn_workspace_bytes", "moe_fused_expert_ffn", "fused_ffn_status",
    "moe_grouped_qgemm_gateup_silu", "moe_grouped_qgemm_down", "MOE_Q4_K", "MOE_Q5_K",
    "MOE_Q6_K", "MOE_Q8_0", "MOE_QTYPE", "KQ_BLOCK", "moe_router_logits", "moe_route",
    "moe_route_workspace_bytes", "moe_route_noalloc", "moe_route_scored", "moe_grouped_gemm_gateup_silu", "moe_grouped_gemm_down",
    "moe_combine_gate", "moe_layer", "moe_time_next_gemm", "moe_probe_out_values",
    "moe_probe_hbm_read", "moe_probe_mfma_bf16", "moe_probe_mfma_flops", "MOE_F32", "MOE_BF16", "MOE_F16", "SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmoe.so")
_lib = None

MOE_F32, MOE_BF16, MOE_F16 = 0, 1, 2
STATUS = {0: "MOE_OK", 1: "MOE_E_INVALID", 2: "MOE_E_DTYPE", 3: "MOE_E_SHAPE",
          4: "MOE_E_WORKSPACE", 5: "MOE_E_HIP"}

_p = ctypes.c_void_p
_i = ctypes.c_int
_st = ctypes.c_int

MOE_WEIGHTS_PACKED_V1 = 0x4D4F4531


class MoeWeights(ctypes.Structure):
    """The C ABI's moe_weights: host descriptor of a packed expert weight set,
    filled by moe_pack_weights / moe_weights_slice."""
    _fields_ = [("layout", ctypes.c_uint32), ("kind", ctypes.c_int32), ("E", ctypes.c_int32),
                ("R", ctypes.c_int32), ("K", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("data", ctypes.c_void_p), ("expert_bytes", ctypes.c_uint64)]


_wp = ctypes.POINTER(MoeWeights)
SYMBOLS = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_init": (_st, []),
    "moe_packed_weight_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "moe_q8k_bytes": (ctypes.c_size_t, [_i, _i]),
    "moe_quantize_q8k": (_st, [_p, _i, _i, _p, _p]),
    "moe_q8_0_bytes": (ctypes.c_size_t, [_i, _i]),
    "moe_fused_expert_ffn_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "moe_fused_expert_ffn": (_st, [_p, _i, _i, _wp, _wp, _i, _i, _p, _p, _i, _p, _p, _p, _p,
                                   ctypes.c_size_t, _p]),
    "moe_quantize_q8_0": (_st, [_p, _i, _i, _p, _p]),
    "moe_grouped_qgemm_gateup_silu": (_st, [_p, _i, _i, _p, _i, _i, _i, _p, _p, _i, _p, _p]),
    "moe_grouped_qgemm_down": (_st, [_p, _i, _i, _p, _i, _i, _i, _p, _p, _p, _p, _p]),
    "moe_pack_weights": (_st, [_p, _i, _i, _i, _i, _p, _wp, _p]),
    "moe_weights_slice": (_st, [_wp, _i, _i, _wp]),
    "moe_time_next_gemm": (_st, [_p, _p]),
    "moe_router_logits": (_st, [_p, _i, _i, _p, _i, _p, _p, _p]),
    "moe_route_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i]),
    "moe_route": (_st, [_p, _i, _i, _i, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    "moe_route_noalloc": (_st, [_p, _i, _i, _i, _p, _p, _p, _p, _p]),
    "moe_route_scored": (_st, [_p, _i, _i, _i, _i, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p,
                               ctypes.c_size_t, _p]),
    "moe_grouped_gemm_gateup_silu": (_st, [_p, _i, _i, _wp, _i, _i, _p, _p, _i, _p, _p]),
    "moe_grouped_gemm_down": (_st, [_p, _i, _i, _wp, _i, _i, _p, _p, _p, _p, _p]),
    "moe_combine_gate": (_st, [_p, _i, _i, _i, _i, _p, ctypes.c_float, _p, _i, _p, _p, _i, _p]),
    "moe_probe_out_values": (ctypes.c_size_t, []),
    "moe_probe_hbm_read": (_st, [_p, ctypes.c_size_t, _p, _p]),
    "moe_probe_mfma_bf16": (_st, [_p, ctypes.c_size_t, _i, _p, _p]),
    "moe_probe_mfma_flops": (ctypes.c_double, [_i]),
}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libmoe.so (built by ``__graft_entry__.build()``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python mixture_experts_ffn_expert_amd/build.py` first")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in SYMBOLS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise MoeError(status, load().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, ndim=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise MoeError(2, f"{name} dtype {t.dtype} unsupported (expected {dtype})")
    if not t.is_cuda:
        raise MoeError(1, f"{name} must be a device (cuda/hip) tensor")
    if not t.is_contiguous():
        raise MoeError(1, f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise MoeError(3, f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoeError(3, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _dt_code(dtype):
    import torch
    if dtype == torch.float32:
        return MOE_F32
    if dtype == torch.bfloat16:
        return MOE_BF16
    if dtype == torch.float16:
        return MOE_F16
    raise MoeError(2, f"dtype {dtype} unsupported (f32 or bf16)")


def moe_init():
    _check(load().moe_init())


def moe_time_next_gemm(start=None, stop=None):
    """Measurement only: the next GEMM call made by this thread records its
    kernel's own start and end into ``start`` and ``stop``
    (``torch.cuda.Event(enable_timing=True)``, each recorded once beforehand
    so that the HIP event exists). ``None, None`` disarms."""
    def handle(ev, name):
        if ev is None:
            return None
        h = int(ev.cuda_event)
        if h == 0:
            raise MoeError(1, f"moe_time_next_gemm: {name} event was never recorded, so it does "
                              f"not exist yet")
        return ctypes.c_void_p(h)
    _check(load().moe_time_next_gemm(handle(start, "start"), handle(stop, "stop")))


def moe_probe_out_values():
    return int(load().moe_probe_out_values())


def moe_probe_hbm_read(buf, out=None, stream=None):
    """Measurement only: streaming read of the uint8 device buffer ``buf``
    (its size a multiple of 16). Returns the per-thread XORs (int32 view of
    the uint32 values; their XOR is the XOR of every dword of ``buf``)."""
    import torch
    _need(buf, "buf", torch.uint8, 1)
    if out is None:
        out = torch.empty((moe_probe_out_values(),), dtype=torch.int32, device=buf.device)
    _need(out, "out", torch.int32, shape=(moe_probe_out_values(),))
    _check(load().moe_probe_hbm_read(_ptr(buf), buf.numel(), _ptr(out), _stream(stream)))
    return out


def moe_probe_mfma_bf16(ops, iters, out=None, stream=None):
    """Measurement only: register-only bf16 MFMA loop on operands from
    ``ops`` (bf16, a multiple of 8 values); moe_probe_mfma_flops(iters)
    flops per launch. Returns the per-thread accumulator sums (f32)."""
    import torch
    _need(ops, "ops", torch.bfloat16, 1)
    if ops.numel() % 8:
        raise MoeError(1, "ops must hold a multiple of 8 values")
    if out is None:
        out = torch.empty((moe_probe_out_values(),), dtype=torch.float32, device=ops.device)
    _need(out, "out", torch.float32, shape=(moe_probe_out_values(),))
    _check(load().moe_probe_mfma_bf16(_ptr(ops), ops.numel() // 8, int(iters), _ptr(out),
                                      _stream(stream)))
    return out


def moe_probe_mfma_flops(iters):
    return float(load().moe_probe_mfma_flops(int(iters)))


def moe_router_logits(x, w, bias=None, out=None, stream=None):
    import torch
    _need(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    _need(w, "w", torch.bfloat16, 2)
    N = w.shape[0]
    if w.shape[1] != H:
        raise MoeError(3, f"w must be [N, {H}], got {tuple(w.shape)}")
    if bias is not None:
        _need(bias, "bias", torch.float32, shape=(N,))
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, shape=(T, N))
    _check(load().moe_router_logits(_ptr(x), T, H, _ptr(w), N, _ptr(bias), _ptr(out), _stream(stream)))
    return out


def moe_route_workspace_bytes(T, E, K):
    return int(load().moe_route_workspace_bytes(T, E, K))


def moe_route(logits, K, topk_ids=None, topk_w=None, expert_offsets=None, sorted_pairs=None,
              workspace=None, stream=None):
    import torch
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    if expert_offsets is None:
        expert_offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    if sorted_pairs is None:
        sorted_pairs = torch.empty((T * K,), dtype=torch.int32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32, shape=(T, K))
    _need(topk_w, "topk_w", torch.float32, shape=(T, K))
    _need(expert_offsets, "expert_offsets", torch.int32, shape=(E + 1,))
    _need(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * K,))
    need = moe_route_workspace_bytes(T, E, K)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().moe_route(_ptr(logits), T, E, K, _ptr(topk_ids), _ptr(topk_w),
                            _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(workspace), ws_bytes,
                            _stream(stream)))
    return topk_ids, topk_w, expert_offsets, sorted_pairs


def moe_route_noalloc(logits, K, topk_ids, topk_w, expert_offsets, sorted_pairs, stream=None):
    """moe_route with the library's own grouping scratch: the caller passes
    every output and nothing is allocated (for code under graph capture or
    loops that must not allocate). Calls that overlap on one GPU race."""
    import torch
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    _need(topk_ids, "topk_ids", torch.int32, shape=(T, K))
    _need(topk_w, "topk_w", torch.float32, shape=(T, K))
    _need(expert_offsets, "expert_offsets", torch.int32, shape=(E + 1,))
    _need(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * K,))
    _check(load().moe_route_noalloc(_ptr(logits), T, E, K, _ptr(topk_ids), _ptr(topk_w),
                                    _ptr(expert_offsets), _ptr(sorted_pairs), _stream(stream)))
    return topk_ids, topk_w, expert_offsets, sorted_pairs


MOE_SCORE = {"softmax": 0, "sigmoid": 1}
MOE_GROUP_SCORE = {"max": 0, "top2": 1}


def moe_route_scored(logits, K, score="softmax", selection_bias=None, n_group=1, topk_group=1,
                     group_score="max", renormalize=True, topk_ids=None, topk_w=None,
                     expert_offsets=None, sorted_pairs=None, workspace=None, stream=None):
    """General router (sigmoid / full-softmax scores, selection bias,
    group-limited selection); outputs as ``moe_route``."""
    import torch
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    if score not in MOE_SCORE:
        raise MoeError(1, f"score must be one of {sorted(MOE_SCORE)}, got {score!r}")
    if group_score not in MOE_GROUP_SCORE:
        raise MoeError(1, f"group_score must be one of {sorted(MOE_GROUP_SCORE)}, "
                          f"got {group_score!r}")
    if selection_bias is not None:
        _need(selection_bias, "selection_bias", torch.float32, shape=(E,))
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    if expert_offsets is None:
        expert_offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    if sorted_pairs is None:
        sorted_pairs = torch.empty((T * K,), dtype=torch.int32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32, shape=(T, K))
    _need(topk_w, "topk_w", torch.float32, shape=(T, K))
    _need(expert_offsets, "expert_offsets", torch.int32, shape=(E + 1,))
    _need(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * K,))
    need = moe_route_workspace_bytes(T, E, K)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().moe_route_scored(
        _ptr(logits), T, E, K, MOE_SCORE[score], _ptr(selection_bias), int(n_group),
        int(topk_group), MOE_GROUP_SCORE[group_score], 1 if renormalize else 0, _ptr(topk_ids),
        _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(workspace), ws_bytes,
        _stream(stream)))
    return topk_ids, topk_w, expert_offsets, sorted_pairs


MOE_PACK = {"plain": 0, "gateup": 1}


class PackedWeights:
    """Expert weights in the library's packed layout (``moe_pack_weights``):
    ``data`` is the device buffer (uint8), ``E`` experts of a matrix [R, K]
    packed as ``kind`` ("gateup": R = 2I gate and up rows; "plain");
    ``desc`` is the library's descriptor of them, which the GEMM calls take."""

    def __init__(self, data, desc):
        self.data, self.desc = data, desc
        self.E, self.R, self.K = desc.E, desc.R, desc.K
        self.kind = {v: k for k, v in MOE_PACK.items()}[desc.kind]

    def __repr__(self):
        return f"PackedWeights(E={self.E}, R={self.R}, K={self.K}, kind={self.kind!r})"

    def experts(self, e0, e1):
        """Experts [e0, e1) as PackedWeights viewing the same memory (each
        expert's packed matrix is contiguous): the block of experts that one
        rank owns when experts are split across GPUs."""
        sub = MoeWeights()
        _check(load().moe_weights_slice(ctypes.byref(self.desc), e0, e1, ctypes.byref(sub)))
        per = int(self.desc.expert_bytes)
        return PackedWeights(self.data[e0 * per:e1 * per], sub)


def moe_packed_weight_bytes(E, R, K, kind):
    return int(load().moe_packed_weight_bytes(E, R, K, MOE_PACK[kind]))


def moe_pack_weights(w, kind, out=None, stream=None):
    """Pack bf16 expert weights [E, R, K] (or [R, K], one expert) into the
    layout the grouped GEMMs read: kind "gateup" for W_gu [E, 2I, H], "plain"
    for W_d [E, H, I]. Done once when weights are loaded."""
    import torch
    if kind not in MOE_PACK:
        raise MoeError(1, f"kind must be one of {sorted(MOE_PACK)}, got {kind!r}")
    if w.dim() == 2:
        w = w.unsqueeze(0)
    _need(w, "w", torch.bfloat16, 3)
    E, R, K = w.shape
    nbytes = moe_packed_weight_bytes(E, R, K, kind)
    if nbytes == 0:
        raise MoeError(3, f"cannot pack a [{E}, {R}, {K}] matrix as {kind!r}")
    if out is None:
        out = torch.empty((nbytes,), dtype=torch.uint8, device=w.device)
    _need(out, "packed", torch.uint8, shape=(nbytes,))
    desc = MoeWeights()
    _check(load().moe_pack_weights(_ptr(w), E, R, K, MOE_PACK[kind], _ptr(out), ctypes.byref(desc),
                                   _stream(stream)))
    return PackedWeights(out, desc)


def _need_packed(pw, name, kind, R=None, K=None):
    if not isinstance(pw, PackedWeights):
        raise MoeError(1, f"{name} must be PackedWeights from moe_pack_weights, got "
                          f"{type(pw).__name__}")
    if pw.kind != kind or (R is not None and pw.R != R) or (K is not None and pw.K != K):
        raise MoeError(3, f"{name} is {pw!r}; expected kind={kind!r}"
                          + (f" R={R}" if R is not None else "") + (f" K={K}" if K is not None else ""))


def moe_grouped_gemm_gateup_silu(x, w_gu, sorted_pairs, expert_offsets, K, act=None, stream=None):
    """w_gu: PackedWeights of W_gu [E, 2I, H] (kind "gateup")."""
    import torch
    _need(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    _need_packed(w_gu, "w_gu", "gateup", K=H)
    E, I = w_gu.E, w_gu.R // 2
    if sorted_pairs is not None:
        _need(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * K,))
    if expert_offsets is not None:
        _need(expert_offsets, "expert_offsets", torch.int32, shape=(E + 1,))
    if act is None:
        act = torch.empty((T * K, I), dtype=torch.bfloat16, device=x.device)
    _need(act, "act", torch.bfloat16, shape=(T * K, I))
    _check(load().moe_grouped_gemm_gateup_silu(_ptr(x), T, H, ctypes.byref(w_gu.desc), E, I,
                                               _ptr(sorted_pairs), _ptr(expert_offsets), K,
                                               _ptr(act), _stream(stream)))
    return act


def moe_grouped_gemm_down(act, w_d, sorted_pairs, expert_offsets, pair_w, expert_out=None,
                          stream=None):
    """w_d: PackedWeights of W_d [E, H, I] (kind "plain")."""
    import torch
    _need(act, "act", torch.bfloat16, 2)
    P, I = act.shape
    _need_packed(w_d, "w_d", "plain", K=I)
    E, H = w_d.E, w_d.R
    if sorted_pairs is not None:
        _need(sorted_pairs, "sorted_pairs", torch.int32, shape=(P,))
    if expert_offsets is not None:
        _need(expert_offsets, "expert_offsets", torch.int32, shape=(E + 1,))
    if pair_w is not None:
        _need(pair_w, "pair_w", torch.float32)
        if pair_w.numel() != P:
            raise MoeError(3, f"pair_w must hold {P} weights, got {pair_w.numel()}")
    if expert_out is None:
        expert_out = torch.empty((P, H), dtype=torch.bfloat16, device=act.device)
    _need(expert_out, "expert_out", torch.bfloat16, shape=(P, H))
    _check(load().moe_grouped_gemm_down(_ptr(act), P, I, ctypes.byref(w_d.desc), E, H,
                                        _ptr(sorted_pairs),
                                        _ptr(expert_offsets), _ptr(pair_w), _ptr(expert_out),
                                        _stream(stream)))
    return expert_out


MOE_Q8_0, MOE_Q4_K, MOE_Q5_K, MOE_Q6_K = 8, 12, 13, 14
MOE_QTYPE = {"q8_0": MOE_Q8_0, "q4_k": MOE_Q4_K, "q5_k": MOE_Q5_K, "q6_k": MOE_Q6_K}
# (bytes, values) per block of each weight format
KQ_BLOCK = {"q8_0": (34, 32), "q4_k": (144, 256), "q5_k": (176, 256), "q6_k": (210, 256)}
Q4K_BLOCK = 144


class QBuffer:
    """Quantized activations: ``data`` (uint8) holding R rows of K values in
    the layout of ``kind`` ("q8_k": moe_quantize_q8k, "q8_0":
    moe_quantize_q8_0)."""

    def __init__(self, data, R, K, kind="q8_k"):
        self.data, self.R, self.K, self.kind = data, R, K, kind


Q8KBuffer = QBuffer


def moe_q8k_bytes(R, K):
    return int(load().moe_q8k_bytes(R, K))


def moe_q8_0_bytes(R, K):
    return int(load().moe_q8_0_bytes(R, K))


def _quantize(fn_name, kind, nbytes_fn, x, out, stream):
    import torch
    _need(x, "x", torch.bfloat16, 2)
    R, K = x.shape
    nbytes = max(nbytes_fn(R, K), 16)
    if out is None:
        out = torch.empty((nbytes,), dtype=torch.uint8, device=x.device)
    _need(out, "xq", torch.uint8)
    if out.numel() < nbytes:
        raise MoeError(3, f"xq holds {out.numel()} bytes, {nbytes} needed")
    _check(getattr(load(), fn_name)(_ptr(x), R, K, _ptr(out), _stream(stream)))
    return QBuffer(out, R, K, kind)


def moe_quantize_q8k(x, out=None, stream=None):
    """Q8_K quantization of bf16 rows x [R, K] (K a multiple of 256)."""
    return _quantize("moe_quantize_q8k", "q8_k", moe_q8k_bytes, x, out, stream)


def moe_quantize_q8_0(x, out=None, stream=None):
    """Q8_0 quantization of bf16 rows x [R, K] (K a multiple of 32)."""
    return _quantize("moe_quantize_q8_0", "q8_0", moe_q8_0_bytes, x, out, stream)


def moe_quantize_act(wtype, x, out=None, stream=None):
    """The activation quantizer paired with weight format wtype."""
    if wtype == "q8_0":
        return moe_quantize_q8_0(x, out, stream)
    return moe_quantize_q8k(x, out, stream)


def _need_kq(w, name, K, wtype):
    import torch
    if wtype not in KQ_BLOCK:
        raise MoeError(2, f"{name}: weight format {wtype!r} unsupported ({', '.join(KQ_BLOCK)})")
    nbytes, nval = KQ_BLOCK[wtype]
    _need(w, name, torch.uint8, 4)
    if w.shape[2] * nval != K or w.shape[3] != nbytes:
        raise MoeError(3, f"{name} must be {wtype} blocks [E, R, {K // nval}, {nbytes}], got "
                          f"{tuple(w.shape)}")


def _need_act_kind(xq, wtype):
    want = "q8_0" if wtype == "q8_0" else "q8_k"
    if getattr(xq, "kind", "q8_k") != want:
        raise MoeError(3, f"{wtype} weights need {want} activations, got {xq.kind}")


def moe_grouped_qgemm_gateup_silu(xq, w_gu, sorted_pairs, expert_offsets, K, act=None,
                                  stream=None, wtype="q4_k"):
    """xq: QBuffer of x [T, H] (the quantizer paired with wtype); w_gu: blocks
    uint8 [E, 2I, H/values, bytes] of format wtype."""
    import torch
    T, H = xq.R, xq.K
    _need_kq(w_gu, "w_gu", H, wtype)
    _need_act_kind(xq, wtype)
    E, I = w_gu.shape[0], w_gu.shape[1] // 2
    if sorted_pairs is not None:
        _need(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * K,))
    if expert_offsets is not None:
        _need(expert_offsets, "expert_offsets", torch.int32, shape=(E + 1,))
    if act is None:
        act = torch.empty((T * K, I), dtype=torch.bfloat16, device=w_gu.device)
    _need(act, "act", torch.bfloat16, shape=(T * K, I))
    _check(load().moe_grouped_qgemm_gateup_silu(
        _ptr(xq.data), T, H, _ptr(w_gu), MOE_QTYPE[wtype], E, I, _ptr(sorted_pairs),
        _ptr(expert_offsets), K, _ptr(act), _stream(stream)))
    return act


def moe_grouped_qgemm_down(actq, w_d, sorted_pairs, expert_offsets, pair_w, expert_out=None,
                           stream=None, wtype="q4_k"):
    """actq: QBuffer of act [P, I]; w_d: blocks uint8 [E, H, I/values, bytes]
    of format wtype."""
    import torch
    P, I = actq.R, actq.K
    _need_kq(w_d, "w_d", I, wtype)
    _need_act_kind(actq, wtype)
    E, H = w_d.shape[0], w_d.shape[1]
    if sorted_pairs is not None:
        _need(sorted_pairs, "sorted_pairs", torch.int32, shape=(P,))
    if expert_offsets is not None:
        _need(expert_offsets, "expert_offsets", torch.int32, shape=(E + 1,))
    if pair_w is not None:
        _need(pair_w, "pair_w", torch.float32)
        if pair_w.numel() != P:
            raise MoeError(3, f"pair_w must hold {P} weights, got {pair_w.numel()}")
    if expert_out is None:
        expert_out = torch.empty((P, H), dtype=torch.bfloat16, device=w_d.device)
    _need(expert_out, "expert_out", torch.bfloat16, shape=(P, H))
    _check(load().moe_grouped_qgemm_down(
        _ptr(actq.data), P, I, _ptr(w_d), MOE_QTYPE[wtype], E, H, _ptr(sorted_pairs),
        _ptr(expert_offsets), _ptr(pair_w), _ptr(expert_out), _stream(stream)))
    return expert_out


def moe_fused_expert_ffn_workspace_bytes(T, E, K, grouped=True):
    return int(load().moe_fused_expert_ffn_workspace_bytes(T, E, K, int(bool(grouped))))


def moe_fused_expert_ffn(x, w_gu, w_d, sorted_pairs, expert_offsets, K, pair_w, workspace,
                         act=None, expert_out=None, stream=None):
    """Gate-up, SiLU-mul and down in one launch (packed w_gu, w_d).
    workspace: int32 tensor of moe_fused_expert_ffn_workspace_bytes bytes,
    zero-filled before its first use. A launch whose status word ends 0
    (fused_ffn_status) leaves the counters zero for the next one; after a
    nonzero status the results are invalid and the whole workspace must be
    zero-filled again before it is reused. Slower than the two GEMM calls at
    the decode shape (see moe.h); kept for callers that want one launch."""
    import torch
    _need(x, "x", torch.bfloat16, 2)
    _need_packed(w_gu, "w_gu", "gateup")
    _need_packed(w_d, "w_d", "plain")
    T, H = x.shape
    E, I = w_gu.E, w_gu.R // 2
    if w_d.E != E or w_d.R != H or w_d.K != I or w_gu.K != H:
        raise MoeError(3, f"w_gu {w_gu.E}x{w_gu.R}x{w_gu.K} and w_d {w_d.E}x{w_d.R}x{w_d.K} do not "
                          f"match x [{T}, {H}]")
    P = T * K
    if sorted_pairs is not None:
        _need(sorted_pairs, "sorted_pairs", torch.int32, shape=(P,))
    if expert_offsets is not None:
        _need(expert_offsets, "expert_offsets", torch.int32, shape=(E + 1,))
    if pair_w is not None:
        _need(pair_w, "pair_w", torch.float32)
        if pair_w.numel() != P:
            raise MoeError(3, f"pair_w must hold {P} weights, got {pair_w.numel()}")
    _need(workspace, "workspace", torch.int32)
    if act is None:
        act = torch.empty((P, I), dtype=torch.bfloat16, device=x.device)
    if expert_out is None:
        expert_out = torch.empty((P, H), dtype=torch.bfloat16, device=x.device)
    _need(act, "act", torch.bfloat16, shape=(P, I))
    _need(expert_out, "expert_out", torch.bfloat16, shape=(P, H))
    _check(load().moe_fused_expert_ffn(
        _ptr(x), T, H, ctypes.byref(w_gu.desc), ctypes.byref(w_d.desc), E, I, _ptr(sorted_pairs),
        _ptr(expert_offsets), K,
        _ptr(pair_w), _ptr(act), _ptr(expert_out), _ptr(workspace),
        workspace.numel() * 4, _stream(stream)))
    return act, expert_out


def fused_ffn_status(workspace):
    """The status word of a fused-FFN workspace (0: every wait ended normally)."""
    return int(workspace.view(-1)[-1].item())


def moe_combine_gate(expert_out, T, K, topk_w=None, routed_scale=1.0, shared=None,
                     gate_logit=None, out=None, out_dtype=None, stream=None):
    import torch
    if not isinstance(expert_out, torch.Tensor):
        raise TypeError("expert_out must be a torch.Tensor")
    eo_dt = _dt_code(expert_out.dtype)
    H = expert_out.numel() // max(1, T * K)
    if T * K * H != expert_out.numel():
        raise MoeError(3, f"expert_out holds {expert_out.numel()} values, not T*K*H")
    _need(expert_out, "expert_out", expert_out.dtype)
    sh_dt = MOE_BF16
    if shared is not None:
        sh_dt = _dt_code(shared.dtype)
        _need(shared, "shared", shared.dtype)
        if shared.numel() != T * H:
            raise MoeError(3, f"shared must hold T*H = {T * H} values")
    if topk_w is not None:
        _need(topk_w, "topk_w", torch.float32)
        if topk_w.numel() != T * K:
            raise MoeError(3, f"topk_w must hold T*K = {T * K} values")
    if gate_logit is not None:
        _need(gate_logit, "gate_logit", torch.float32)
        if gate_logit.numel() != T:
            raise MoeError(3, f"gate_logit must hold T = {T} values")
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype or torch.bfloat16, device=expert_out.device)
    out_dt = _dt_code(out.dtype)
    _need(out, "out", out.dtype)
    _check(load().moe_combine_gate(_ptr(expert_out), eo_dt, T, K, H, _ptr(topk_w),
                                   float(routed_scale), _ptr(shared), sh_dt, _ptr(gate_logit),
                                   _ptr(out), out_dt, _stream(stream)))
    return out


def moe_layer(x, w_r, w_gu, w_d, K, router_bias=None, w_gu_s=None, w_d_s=None, w_g=None,
              bufs=None, stream=None, router=None, selection_bias=None, routed_scale=1.0):
    """Enqueue one MoE layer: logits, route, gate-up, down, (shared), combine.

    ``w_gu``, ``w_d`` (and ``w_gu_s``, ``w_d_s`` for a shared expert) are
    PackedWeights from ``moe_pack_weights``; ``w_r`` and ``w_g`` are bf16
    row-major [E, H] and [1, H].

    ``router`` (dict of ``moe_route_scored`` keyword arguments: score,
    n_group, topk_group, group_score, renormalize) selects the general router
    with ``selection_bias``; None routes with the ungrouped softmax top-k.
    ``bufs`` (dict) may hold preallocated outputs/intermediates under the keys
    logits, ids, w, offsets, sorted, act, expert_out, sd_act, sd, gl, out; the
    dict is filled with everything produced. Returns the bf16 [T, H] output.
    """
    import torch
    T, H = x.shape
    E = w_r.shape[0]
    I = w_gu.R // 2
    b = {} if bufs is None else bufs
    dev = x.device

    def buf(key, shape, dtype):
        if b.get(key) is None:
            b[key] = torch.empty(shape, dtype=dtype, device=dev)
        return b[key]

    logits = moe_router_logits(x, w_r, router_bias, buf("logits", (T, E), torch.float32), stream)
    ws_bytes = moe_route_workspace_bytes(T, E, K)
    ws = buf("route_ws", (ws_bytes,), torch.uint8) if ws_bytes else None
    outs = (buf("ids", (T, K), torch.int32), buf("w", (T, K), torch.float32),
            buf("offsets", (E + 1,), torch.int32), buf("sorted", (T * K,), torch.int32))
    if router is None:
        ids, w, off, sp = moe_route(logits, K, *outs, ws, stream=stream)
    else:
        ids, w, off, sp = moe_route_scored(logits, K, selection_bias=selection_bias, **router,
                                           topk_ids=outs[0], topk_w=outs[1],
                                           expert_offsets=outs[2], sorted_pairs=outs[3],
                                           workspace=ws, stream=stream)
    act = moe_grouped_gemm_gateup_silu(x, w_gu, sp, off, K, buf("act", (T * K, I), torch.bfloat16),
                                       stream)
    eo = moe_grouped_gemm_down(act, w_d, sp, off, w, buf("expert_out", (T * K, H), torch.bfloat16),
                               stream)
    sd = gl = None
    if w_gu_s is not None:
        Is = w_gu_s.R // 2
        sa = moe_grouped_gemm_gateup_silu(x, w_gu_s, None, None, 1,
                                          buf("sd_act", (T, Is), torch.bfloat16), stream)
        sd = moe_grouped_gemm_down(sa, w_d_s, None, None, None,
                                   buf("sd", (T, H), torch.bfloat16), stream)
        gl = moe_router_logits(x, w_g.view(1, H), None, buf("gl", (T, 1), torch.float32), stream)
    return moe_combine_gate(eo, T, K, None, routed_scale, sd, gl,
                            buf("out", (T, H), torch.bfloat16), stream=stream)
