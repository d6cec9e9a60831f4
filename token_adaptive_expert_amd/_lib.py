"""ctypes binding of ``libace_moe.so`` (include/ace_moe.h): argument marshalling only.

Each function has the name of its C entry point, takes torch tensors (device
memory) or None, passes their data pointers and the stream to the library,
and raises AceMoeError on a non-zero status.  No layer arithmetic happens here.
The library must exist: nothing falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ACE_MOE_LIB") or os.path.join(PKG, "lib", "libace_moe.so")

ACE_OK, ACE_EINVAL, ACE_EUNSUPPORTED, ACE_EWORKSPACE, ACE_EHIP = range(5)
ACE_F32, ACE_BF16 = 0, 1
ACE_PATH_AUTO, ACE_PATH_GROUPED, ACE_PATH_STREAM = 0, 1, 2
ACE_STAGE_GATEUP, ACE_STAGE_DOWN = 0x100, 0x200
FUSION = {"max": 0, "min": 1, "mean": 2, "gsp": 3, "rcr": 4, "score": 5}

STATUS_NAMES = {0: "ACE_OK", 1: "ACE_EINVAL", 2: "ACE_EUNSUPPORTED", 3: "ACE_EWORKSPACE", 4: "ACE_EHIP"}

EXPORTS = ["moe_abi_version", "moe_last_error", "moe_workspace_bytes", "moe_route_skip", "moe_dispatch",
           "moe_expert_forward", "moe_combine", "moe_calibrate_workspace_bytes", "moe_calibrate_thresholds",
           "moe_pack_weights", "moe_router_packed_bytes", "moe_pack_router", "moe_tables_workspace_bytes",
           "moe_build_tables", "moe_forward", "moe_forward_static", "moe_hbm_read_probe", "moe_l2_load_probe", "moe_set_kernel_events"]

ACE_STATIC_SCRATCH_BYTES = 80 << 20


class AceMoeError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("I", ctypes.c_int32),
                ("k", ctypes.c_int32), ("dtype", ctypes.c_int32), ("norm_topk", ctypes.c_int32),
                ("fusion", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("weight_layout", ctypes.c_int32),
                ("router_layout", ctypes.c_int32), ("expert_pool", ctypes.c_int32)]


ACE_LAYOUT_LINEAR, ACE_LAYOUT_PACKED = 0, 1


def make_desc(T, H, E, I, k, dtype, norm_topk=1, fusion="max", rms_eps=1e-6, weight_layout=0,
              router_layout=0, expert_pool=0) -> MoeDesc:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: ACE_F32, torch.bfloat16: ACE_BF16}[dtype]
    elif isinstance(dtype, str):
        dtype = {"f32": ACE_F32, "bf16": ACE_BF16}[dtype]
    if isinstance(fusion, str):
        fusion = FUSION[fusion]
    return MoeDesc(int(T), int(H), int(E), int(I), int(k), int(dtype), int(norm_topk), int(fusion), float(rms_eps),
                   int(weight_layout), int(router_layout), int(expert_pool))


ABI_VERSION = 3  # ACE_MOE_ABI_VERSION of include/ace_moe.h that these bindings follow
_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m token_adaptive_expert_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(MoeDesc)
    lib.moe_abi_version.restype = ctypes.c_int
    lib.moe_abi_version.argtypes = []
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.moe_abi_version()}, these bindings need {ABI_VERSION}: "
                          "rebuild it with `python -m token_adaptive_expert_amd.build`")
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_workspace_bytes.restype = SZ
    lib.moe_workspace_bytes.argtypes = [D]
    lib.moe_route_skip.restype = ctypes.c_int
    lib.moe_route_skip.argtypes = [D, P, P, P, P, P, P, P, P, F32, F32, P, P, P, P, P]
    lib.moe_dispatch.restype = ctypes.c_int
    lib.moe_dispatch.argtypes = [D, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_expert_forward.restype = ctypes.c_int
    lib.moe_expert_forward.argtypes = [D, I32, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_combine.argtypes = [D, P, P, P, P, P]
    lib.moe_calibrate_workspace_bytes.restype = SZ
    lib.moe_calibrate_workspace_bytes.argtypes = [D]
    lib.moe_calibrate_thresholds.restype = ctypes.c_int
    lib.moe_calibrate_thresholds.argtypes = [D, P, P, P, P, F32, P, P, P, SZ, P]
    lib.moe_pack_weights.restype = ctypes.c_int
    lib.moe_pack_weights.argtypes = [D, I32, P, P, P]
    lib.moe_router_packed_bytes.restype = SZ
    lib.moe_router_packed_bytes.argtypes = [D]
    lib.moe_pack_router.restype = ctypes.c_int
    lib.moe_pack_router.argtypes = [D, P, P, P]
    lib.moe_tables_workspace_bytes.restype = SZ
    lib.moe_tables_workspace_bytes.argtypes = [D]
    lib.moe_build_tables.restype = ctypes.c_int
    lib.moe_build_tables.argtypes = [D, F32, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward.argtypes = [D, I32, P, P, P, P, P, P, P, P, F32, F32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                P, SZ, P]
    lib.moe_forward_static.restype = ctypes.c_int
    lib.moe_forward_static.argtypes = [D, I32, P, P, P, P, P, P, P, P, F32, F32, P, P, P, P, P, P, P, P, P, P, P, P,
                                       P, P]
    lib.moe_hbm_read_probe.restype = ctypes.c_int
    lib.moe_hbm_read_probe.argtypes = [P, SZ, P, I32, P]
    lib.moe_l2_load_probe.restype = ctypes.c_int
    lib.moe_l2_load_probe.argtypes = [P, SZ, I32, I32, I32, I32, P, I32, P]
    lib.moe_set_kernel_events.restype = ctypes.c_int
    lib.moe_set_kernel_events.argtypes = [P, P]
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != ACE_OK:
        raise AceMoeError(status, where, load().moe_last_error().decode())


def moe_abi_version() -> int:
    return load().moe_abi_version()


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def moe_workspace_bytes(desc: MoeDesc) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(desc)))


def moe_route_skip(desc, x, gamma, w_router, router_bias, logits_in, logits_out, a_gsp, a_rcr, tau_gsp, tau_rcr,
                   h_out, topk_idx, topk_gate, keep, stream=None):
    _check(load().moe_route_skip(ctypes.byref(desc), _ptr(x), _ptr(gamma), _ptr(w_router), _ptr(router_bias),
                                 _ptr(logits_in), _ptr(logits_out), _ptr(a_gsp), _ptr(a_rcr), float(tau_gsp),
                                 float(tau_rcr), _ptr(h_out), _ptr(topk_idx), _ptr(topk_gate), _ptr(keep),
                                 _stream(stream)), "moe_route_skip")


def moe_dispatch(desc, topk_idx, topk_gate, keep, expert_offsets, sorted_token, sorted_gate, slot_pos, workspace,
                 workspace_bytes=None, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_dispatch(ctypes.byref(desc), _ptr(topk_idx), _ptr(topk_gate), _ptr(keep), _ptr(expert_offsets),
                               _ptr(sorted_token), _ptr(sorted_gate), _ptr(slot_pos), _ptr(workspace), int(nbytes),
                               _stream(stream)), "moe_dispatch")


def moe_expert_forward(desc, path, h, w_gate, w_up, w_down, expert_offsets, sorted_token, sorted_gate, act, slot_out,
                       workspace=None, workspace_bytes=None, stream=None):
    nbytes = 0
    if workspace is not None:
        nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_expert_forward(ctypes.byref(desc), int(path), _ptr(h), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                     _ptr(expert_offsets), _ptr(sorted_token), _ptr(sorted_gate), _ptr(act),
                                     _ptr(slot_out), _ptr(workspace), int(nbytes), _stream(stream)),
           "moe_expert_forward")


def moe_combine(desc, slot_pos, slot_out, residual, y, stream=None):
    _check(load().moe_combine(ctypes.byref(desc), _ptr(slot_pos), _ptr(slot_out), _ptr(residual), _ptr(y),
                              _stream(stream)), "moe_combine")


def moe_calibrate_workspace_bytes(desc: MoeDesc) -> int:
    return int(load().moe_calibrate_workspace_bytes(ctypes.byref(desc)))


def moe_calibrate_thresholds(desc, topk_idx, topk_gate, a_gsp, a_rcr, skip_rate, tau_out, level_out, workspace,
                             workspace_bytes=None, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_calibrate_thresholds(ctypes.byref(desc), _ptr(topk_idx), _ptr(topk_gate), _ptr(a_gsp),
                                           _ptr(a_rcr), float(skip_rate), _ptr(tau_out), _ptr(level_out),
                                           _ptr(workspace), int(nbytes), _stream(stream)),
           "moe_calibrate_thresholds")


def moe_pack_weights(desc, which, src, dst, stream=None):
    _check(load().moe_pack_weights(ctypes.byref(desc), int(which), _ptr(src), _ptr(dst), _stream(stream)),
           "moe_pack_weights")


def moe_router_packed_bytes(desc: MoeDesc) -> int:
    return int(load().moe_router_packed_bytes(ctypes.byref(desc)))


def moe_pack_router(desc, w_router, dst, stream=None):
    _check(load().moe_pack_router(ctypes.byref(desc), _ptr(w_router), _ptr(dst), _stream(stream)), "moe_pack_router")


def moe_tables_workspace_bytes(desc: MoeDesc) -> int:
    return int(load().moe_tables_workspace_bytes(ctypes.byref(desc)))


def moe_build_tables(desc, eps, gamma, w_router, w_gate, w_up, w_down, a_gsp, a_rcr, workspace,
                     workspace_bytes=None, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_build_tables(ctypes.byref(desc), float(eps), _ptr(gamma), _ptr(w_router), _ptr(w_gate),
                                   _ptr(w_up), _ptr(w_down), _ptr(a_gsp), _ptr(a_rcr), _ptr(workspace), int(nbytes),
                                   _stream(stream)), "moe_build_tables")


def moe_forward(desc, path, x, gamma, w_router, router_bias, logits_in, logits_out, a_gsp, a_rcr, tau_gsp, tau_rcr,
                w_gate, w_up, w_down, residual, h_out, topk_idx, topk_gate, keep, expert_offsets, sorted_token,
                sorted_gate, slot_pos, act, slot_out, y, workspace, workspace_bytes=None, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().moe_forward(ctypes.byref(desc), int(path), _ptr(x), _ptr(gamma), _ptr(w_router), _ptr(router_bias),
                              _ptr(logits_in), _ptr(logits_out), _ptr(a_gsp), _ptr(a_rcr), float(tau_gsp),
                              float(tau_rcr), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(residual), _ptr(h_out),
                              _ptr(topk_idx), _ptr(topk_gate), _ptr(keep), _ptr(expert_offsets), _ptr(sorted_token),
                              _ptr(sorted_gate), _ptr(slot_pos), _ptr(act), _ptr(slot_out), _ptr(y), _ptr(workspace),
                              int(nbytes), _stream(stream)), "moe_forward")


def moe_forward_static(desc, path, x, gamma, w_router, router_bias, logits_in, logits_out, a_gsp, a_rcr, tau_gsp,
                       tau_rcr, w_gate, w_up, w_down, residual, h_out, topk_idx, topk_gate, keep, expert_offsets,
                       sorted_token, sorted_gate, slot_pos, y, stream=None):
    _check(load().moe_forward_static(ctypes.byref(desc), int(path), _ptr(x), _ptr(gamma), _ptr(w_router),
                                     _ptr(router_bias), _ptr(logits_in), _ptr(logits_out), _ptr(a_gsp), _ptr(a_rcr),
                                     float(tau_gsp), float(tau_rcr), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                     _ptr(residual), _ptr(h_out), _ptr(topk_idx), _ptr(topk_gate), _ptr(keep),
                                     _ptr(expert_offsets), _ptr(sorted_token), _ptr(sorted_gate), _ptr(slot_pos),
                                     _ptr(y), _stream(stream)), "moe_forward_static")


def moe_l2_load_probe(buf, sink, workgroups, rounds, loads=6, mfma_per_load=0, stride_mode=0, nbytes=None,
                      stream=None):
    nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(load().moe_l2_load_probe(_ptr(buf), int(nbytes), int(rounds), int(loads), int(mfma_per_load),
                                    int(stride_mode), _ptr(sink), int(workgroups), _stream(stream)),
           "moe_l2_load_probe")


def moe_hbm_read_probe(buf, sink, workgroups, nbytes=None, stream=None):
    nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(load().moe_hbm_read_probe(_ptr(buf), int(nbytes), _ptr(sink), int(workgroups), _stream(stream)),
           "moe_hbm_read_probe")


def moe_set_kernel_events(start, stop):
    """start/stop: torch.cuda.Event (or raw hipEvent_t ints), or None to clear."""
    def ev(e):
        if e is None:
            return None
        return e if isinstance(e, int) else e.cuda_event
    _check(load().moe_set_kernel_events(ev(start), ev(stop)), "moe_set_kernel_events")
