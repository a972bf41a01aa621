"""ctypes binding of libmoe.so (include/moe.h), for torch tensors.

Argument marshalling only: device pointers, sizes and the current HIP
stream go to the C ABI, which runs every step on the GPU. There is no other
implementation behind these functions; a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EALIGN, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4, -5
N_STAGES = 8
STAGES = ("router", "topk", "permute", "pool", "gateup", "down", "combine", "unpool")
VIEWS = dict(logits=0, ids=1, weights=2, offsets=3, sorted=4, latent=5, h=6, rows=7, y=8,
             norm_f32=9, norm_bf16=10, layer_out=11, sync=12, rows_bf16=13)

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


FMT_MXFP4, FMT_NVFP4 = 0, 1  # expert weight formats (MOE_FMT_*)


class MoeDims(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("latent", _i32), ("inter", _i32), ("n_experts", _i32),
                ("top_k", _i32), ("norm_eps", ctypes.c_float), ("gain_per_expert", _i32),
                ("expert_format", _i32), ("expert_split_rows", _i32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router", _vp), ("pooler", _vp), ("w13_codes", _vp), ("w13_scales", _vp),
                ("w2_codes", _vp), ("w2_scales", _vp), ("norm_gain", _vp), ("unpooler", _vp),
                ("w13_global", _vp), ("w2_global", _vp)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().moe_status_string(status).decode()
        if status == MOE_EHIP:
            msg += f" (hip error {lib().moe_last_hip_error()})"
        super().__init__(f"{what}: {msg} [{status}]")


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m latent_mixture_experts_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_workspace_bytes.restype = _sz
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(MoeDims), _i32]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _sz, _vp]
        L.moe_route_validate.restype = ctypes.c_int
        L.moe_route_validate.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _sz]
        L.moe_latent_forward.restype = ctypes.c_int
        L.moe_latent_forward.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp,
                                         ctypes.POINTER(MoeWeights), _vp, _vp, _sz, _vp]
        L.moe_latent_forward_timed.restype = ctypes.c_int
        L.moe_latent_forward_timed.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp,
                                               ctypes.POINTER(MoeWeights), _vp, _vp, _sz, _vp,
                                               ctypes.POINTER(_vp)]
        L.moe_latent_forward_persistent.restype = ctypes.c_int
        L.moe_latent_forward_persistent.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp,
                                                    ctypes.POINTER(MoeWeights), _vp, _vp, _sz, _vp]
        L.moe_latent_forward_noalloc.restype = ctypes.c_int
        L.moe_latent_forward_noalloc.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp,
                                                 ctypes.POINTER(MoeWeights), _vp, _vp]
        L.moe_latent_forward_routed.restype = ctypes.c_int
        L.moe_latent_forward_routed.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp, _vp, _vp,
                                                ctypes.POINTER(MoeWeights), _vp, _vp, _sz, _vp]
        L.moe_latent_forward_routed_validate.restype = ctypes.c_int
        L.moe_latent_forward_routed_validate.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp, _vp,
                                                         _vp, ctypes.POINTER(MoeWeights), _vp,
                                                         _vp, _sz]
        L.moe_block_workspace_bytes.restype = _sz
        L.moe_block_workspace_bytes.argtypes = [ctypes.POINTER(MoeDims), _i32]
        L.moe_block_forward.restype = ctypes.c_int
        L.moe_block_forward.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp, _vp, _vp,
                                        ctypes.c_float, ctypes.POINTER(MoeWeights), _vp, _vp, _sz,
                                        _vp]
        L.moe_block_forward_validate.restype = ctypes.c_int
        L.moe_block_forward_validate.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp, _vp, _vp,
                                                 ctypes.c_float, ctypes.POINTER(MoeWeights), _vp,
                                                 _vp, _sz]
        L.moe_latent_forward_validate.restype = ctypes.c_int
        L.moe_latent_forward_validate.argtypes = [ctypes.POINTER(MoeDims), _i32, _vp,
                                                  ctypes.POINTER(MoeWeights), _vp, _vp, _sz]
        L.moe_workspace_view.restype = ctypes.c_int
        L.moe_workspace_view.argtypes = [ctypes.POINTER(MoeDims), _i32, _i32,
                                         ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_last_hip_error.restype = ctypes.c_int
        L.moe_last_hip_error.argtypes = []
        _lib = L
    return _lib


def make_dims(dims: dict, eps: float = 1e-6, gain_per_expert: int = 0,
              expert_format: int = FMT_MXFP4, expert_split_rows: int = 0) -> MoeDims:
    return MoeDims(dims["hidden"], dims["latent"], dims["inter"], dims["n_experts"],
                   dims["top_k"], eps, int(gain_per_expert), int(expert_format),
                   int(expert_split_rows))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace_bytes(d: MoeDims, max_tokens: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(d), max_tokens))


def alloc_workspace(d: MoeDims, max_tokens: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(d, max_tokens)
    if n == 0 and max_tokens > 0:
        raise MoeError(MOE_EUNSUPPORTED, "moe_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def block_workspace_bytes(d: MoeDims, max_tokens: int) -> int:
    return int(lib().moe_block_workspace_bytes(ctypes.byref(d), max_tokens))


def alloc_block_workspace(d: MoeDims, max_tokens: int, device="cuda") -> torch.Tensor:
    n = block_workspace_bytes(d, max_tokens)
    if n == 0 and max_tokens > 0:
        raise MoeError(MOE_EUNSUPPORTED, "moe_block_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def make_weights(w: dict) -> MoeWeights:
    """Pointers of the weight tensors (w13_global / w2_global: NVFP4 only)."""
    return MoeWeights(*(_ptr(w.get(k)) for k in ("router", "pooler", "w13_codes", "w13_scales",
                                                  "w2_codes", "w2_scales", "norm_gain", "unpooler",
                                                  "w13_global", "w2_global")))


def route(d: MoeDims, x: torch.Tensor, router: torch.Tensor, ws: torch.Tensor,
          want_logits: bool = True, stream=None) -> dict:
    """moe_route on T = x.shape[0] tokens; returns the output tensors."""
    T = x.shape[0]
    E, K = d.n_experts, d.top_k
    dev = x.device
    out = dict(ids=torch.empty((T, K), dtype=torch.int32, device=dev),
               w=torch.empty((T, K), dtype=torch.float32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted=torch.empty(T * K, dtype=torch.int32, device=dev))
    out["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    rc = lib().moe_route(ctypes.byref(d), T, _ptr(x), _ptr(router), _ptr(out["ids"]),
                         _ptr(out["w"]), _ptr(out["offsets"]), _ptr(out["sorted"]),
                         _ptr(out["logits"]), _ptr(ws), ws.numel(), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_route")
    return out


def latent_forward(d: MoeDims, x: torch.Tensor, weights: MoeWeights, out: torch.Tensor,
                   ws: torch.Tensor, stream=None, events=None) -> torch.Tensor:
    """moe_latent_forward, or moe_latent_forward_timed when ``events`` holds
    2 * MOE_N_STAGES hipEvent_t handles (start, stop of each step; None
    entries are skipped)."""
    T = x.shape[0]
    if events is None:
        rc = lib().moe_latent_forward(ctypes.byref(d), T, _ptr(x), ctypes.byref(weights),
                                      _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    else:
        arr = (_vp * len(events))(*[e if e else None for e in events])
        rc = lib().moe_latent_forward_timed(ctypes.byref(d), T, _ptr(x), ctypes.byref(weights),
                                            _ptr(out), _ptr(ws), ws.numel(), _stream(stream), arr)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_latent_forward")
    return out


def latent_forward_routed(d: MoeDims, x: torch.Tensor, ids: torch.Tensor, w: torch.Tensor,
                          weights: MoeWeights, out: torch.Tensor, ws: torch.Tensor,
                          stream=None) -> torch.Tensor:
    """moe_latent_forward_routed: the layer with the routing given (ids
    [T][K] int32, w [T][K] fp32, on the device)."""
    T = x.shape[0]
    rc = lib().moe_latent_forward_routed(ctypes.byref(d), T, _ptr(x), _ptr(ids), _ptr(w),
                                         ctypes.byref(weights), _ptr(out), _ptr(ws), ws.numel(),
                                         _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_latent_forward_routed")
    return out


def latent_forward_persistent(d: MoeDims, x: torch.Tensor, weights: MoeWeights, out: torch.Tensor,
                              ws: torch.Tensor, stream=None) -> torch.Tensor:
    """moe_latent_forward_persistent: the layer for one or two tokens in one launch."""
    T = x.shape[0]
    rc = lib().moe_latent_forward_persistent(ctypes.byref(d), T, _ptr(x), ctypes.byref(weights),
                                             _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_latent_forward_persistent")
    return out


def latent_forward_noalloc(d: MoeDims, x: torch.Tensor, weights: MoeWeights, out: torch.Tensor,
                           stream=None) -> torch.Tensor:
    """moe_latent_forward_noalloc: the layer with the library's own per-GPU
    scratch array as its workspace (no workspace argument)."""
    T = x.shape[0]
    rc = lib().moe_latent_forward_noalloc(ctypes.byref(d), T, _ptr(x), ctypes.byref(weights),
                                          _ptr(out), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_latent_forward_noalloc")
    return out


def block_forward(d: MoeDims, resid: torch.Tensor, pre_gain: torch.Tensor, post_gain: torch.Tensor,
                  block_eps: float, weights: MoeWeights, out: torch.Tensor, ws: torch.Tensor,
                  stream=None) -> torch.Tensor:
    """moe_block_forward: out = resid + post_norm(layer(pre_norm(resid)))."""
    T = resid.shape[0]
    rc = lib().moe_block_forward(ctypes.byref(d), T, _ptr(resid), _ptr(pre_gain), _ptr(post_gain),
                                 block_eps, ctypes.byref(weights), _ptr(out), _ptr(ws), ws.numel(),
                                 _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_block_forward")
    return out


def workspace_view_range(d: MoeDims, T: int, which: str) -> tuple[int, int]:
    """(byte offset, bytes) of an intermediate in the workspace."""
    off, nb = _sz(), _sz()
    rc = lib().moe_workspace_view(ctypes.byref(d), T, VIEWS[which], ctypes.byref(off), ctypes.byref(nb))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_workspace_view")
    return off.value, nb.value


def workspace_view(d: MoeDims, T: int, ws: torch.Tensor, which: str, dtype, shape):
    """An intermediate of the last moe_latent_forward, viewed in the workspace."""
    off, nb = workspace_view_range(d, T, which)
    return ws[off:off + nb].view(dtype).view(shape)


# ---- HIP events (timing of the stages on the stream they run on) ----------
_hip = None


def hip_runtime():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(_vp)]
        _hip.hipEventDestroy.argtypes = [_vp]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        _hip.hipEventSynchronize.argtypes = [_vp]
    return _hip


def create_events(n: int) -> list[int]:
    evs = []
    for _ in range(n):
        e = _vp()
        rc = hip_runtime().hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        evs.append(e.value)
    return evs


def elapsed_ms(e0: int, e1: int) -> float:
    ms = ctypes.c_float()
    rc = hip_runtime().hipEventElapsedTime(ctypes.byref(ms), e0, e1)
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
    return ms.value


def destroy_events(evs) -> None:
    for e in evs:
        hip_runtime().hipEventDestroy(e)
