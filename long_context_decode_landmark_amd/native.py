"""ctypes binding of liblowram.so (argument marshalling only).

Every function here takes torch tensors already resident on the GPU, passes
their device pointers and the current HIP stream to the C ABI declared in
include/lowram.h, and raises LowramError on a non-zero status.  No step of the
decode computation runs in Python: if the library is not built, calls fail.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblowram.so")
ABI_VERSION = 3  # LOWRAM_ABI_VERSION of the header these structs follow

FMT_BF16 = 0
FMT_INT4_G32 = 1

# every entry point include/lowram.h declares
SYMBOLS = (
    "lowram_abi_version",
    "lowram_strerror",
    "lowram_workspace_bytes",
    "lowram_decode_plan",
    "lowram_decode_step",
    "lowram_decode_step_noalloc",
    "lowram_decode_stages",
    "lowram_decode_step_events",
    "lowram_decode_shared",
    "dense_workspace_bytes",
    "dense_decode_step",
    "lowram_resid_chunk_desc",
    "lowram_build_coeff",
    "lowram_build_layer_workspace_bytes",
    "lowram_build_layer",
    "lowram_build_layer_events",
    "lowram_append_coeff",
    "lowram_append_layer",
    "lowram_fit_basis_workspace_bytes",
    "lowram_fit_basis",
)

ERRORS = {0: "OK", -1: "NULL", -2: "SHAPE", -3: "UNSUPPORTED", -4: "WORKSPACE", -5: "ALIGN", -6: "HIP",
          -7: "SCRATCH"}

# LOWRAM_NOALLOC_SCRATCH_BYTES of include/lowram.h
NOALLOC_SCRATCH_BYTES = 64 << 20


class LowramAttendPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kernel", "workgroups", "tiles_per_group", "groups_per_head", "partial_slots", "reserved_slots",
        "window_kernel")]


class LowramShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "prefix_len", "window", "chunk", "n_heads_q", "n_heads_kv", "head_dim", "rank",
        "mlp_hidden", "topk", "n_resid", "n_cand", "coeff_fmt", "resid_fmt")] + [
        ("rope_theta", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("prefix_cap", ctypes.c_int32), ("window_cap", ctypes.c_int32)]


CACHE_FIELDS = ("coeff", "coeff_scale", "basis", "landmark", "cand_ids", "w1", "b1", "w2", "b2",
                "res_idx", "res_val", "res_scale", "res_chunk_desc", "win_k", "win_v")


class LowramLayerCache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in CACHE_FIELDS]


class LowramBuildShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "ctx_len", "window", "chunk", "n_heads_kv", "head_dim", "rank", "group_layers",
        "mlp_hidden", "n_resid", "coeff_fmt", "resid_fmt")] + [("rope_theta", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("prefix_cap", "window_cap", "resid_cap")]


BUILD_FIELDS = ("keys", "group_basis", "coeff", "coeff_scale", "values", "w1", "b1", "w2", "b2",
                "basis", "landmark", "res_idx", "res_val", "res_scale", "res_chunk_desc", "win_k", "win_v",
                "res_thresh", "res_count")


class LowramLayerBuild(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUILD_FIELDS]


APPEND_FIELDS = ("keys_new", "res_thresh", "res_count", "res_dropped", "landmark", "res_idx", "res_val",
                 "res_scale", "res_chunk_desc", "win_k", "win_v")


class LowramLayerAppend(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in APPEND_FIELDS]


class LowramFitShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "ctx_len", "prefix_len", "group_dim", "rank", "power")]


class DenseShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "ctx_len", "n_heads_q", "n_heads_kv", "head_dim")] + [
        ("softmax_scale", ctypes.c_float)]


class DenseLayerCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class LowramError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({ERRORS.get(status, '?')}): {strerror(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(or python -m long_context_decode_landmark_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.lowram_abi_version.restype = ctypes.c_int
        L.lowram_strerror.restype = ctypes.c_char_p
        L.lowram_strerror.argtypes = [ctypes.c_int]
        L.lowram_workspace_bytes.argtypes = [ctypes.POINTER(LowramShape), ctypes.POINTER(sz)]
        L.lowram_decode_plan.argtypes = [ctypes.POINTER(LowramShape), ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(LowramAttendPlan)]
        L.lowram_decode_step.argtypes = [ctypes.POINTER(LowramShape), ctypes.POINTER(LowramLayerCache),
                                         vp, vp, vp, vp, sz, vp]
        L.lowram_decode_step_noalloc.argtypes = [ctypes.POINTER(LowramShape), ctypes.POINTER(LowramLayerCache),
                                                 vp, vp, vp, vp]
        L.lowram_decode_stages.argtypes = [ctypes.POINTER(LowramShape), ctypes.POINTER(LowramLayerCache),
                                           vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lowram_decode_step_events.argtypes = [ctypes.POINTER(LowramShape), ctypes.POINTER(LowramLayerCache),
                                                vp, vp, vp, vp, sz, vp, ctypes.POINTER(ctypes.c_void_p)]
        L.lowram_decode_shared.argtypes = [ctypes.POINTER(LowramShape), ctypes.POINTER(LowramLayerCache),
                                           vp, vp, vp, vp, sz, vp, ctypes.POINTER(ctypes.c_void_p)]
        L.dense_workspace_bytes.argtypes = [ctypes.POINTER(DenseShape), ctypes.POINTER(sz)]
        L.dense_decode_step.argtypes = [ctypes.POINTER(DenseShape), ctypes.POINTER(DenseLayerCache),
                                        vp, vp, vp, sz, vp]
        L.lowram_resid_chunk_desc.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, vp, vp]
        L.lowram_build_coeff.argtypes = [ctypes.POINTER(LowramBuildShape), vp, vp, vp, vp, vp]
        L.lowram_build_layer_workspace_bytes.argtypes = [ctypes.POINTER(LowramBuildShape), ctypes.POINTER(sz)]
        L.lowram_build_layer.argtypes = [ctypes.POINTER(LowramBuildShape), ctypes.c_int32,
                                         ctypes.POINTER(LowramLayerBuild), vp, sz, vp]
        L.lowram_build_layer_events.argtypes = [ctypes.POINTER(LowramBuildShape), ctypes.c_int32,
                                                ctypes.POINTER(LowramLayerBuild), vp, sz, vp,
                                                ctypes.POINTER(ctypes.c_void_p)]
        L.lowram_append_coeff.argtypes = [ctypes.POINTER(LowramShape), ctypes.c_int32, vp, vp, vp, vp, vp]
        L.lowram_append_layer.argtypes = [ctypes.POINTER(LowramShape), ctypes.c_int32, ctypes.c_int32,
                                          ctypes.POINTER(LowramLayerCache), ctypes.POINTER(LowramLayerAppend), vp]
        L.lowram_fit_basis_workspace_bytes.argtypes = [ctypes.POINTER(LowramFitShape), ctypes.POINTER(sz)]
        L.lowram_fit_basis.argtypes = [ctypes.POINTER(LowramFitShape), vp, vp, vp, vp, vp, sz, vp]
        for name in SYMBOLS:
            getattr(L, name).restype = getattr(L, name).restype or ctypes.c_int
        L.lowram_strerror.restype = ctypes.c_char_p
        # the structs above follow one version of include/lowram.h
        if L.lowram_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.lowram_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild it (__graft_entry__.build())")
        _lib = L
    return _lib


def strerror(status: int) -> str:
    try:
        return lib().lowram_strerror(status).decode()
    except RuntimeError:
        return ERRORS.get(status, "?")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LowramError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    """A raw hipStream_t handle, a torch.cuda.Stream, or None (torch's current stream)."""
    if stream is not None:
        return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------------ shapes --
def make_shape(cfg, batch: int | None = None, **over) -> LowramShape:
    """lowram_shape of one layer of a workload (synth.Config-like object)."""
    f = dict(batch=cfg.batch if batch is None else batch, prefix_len=cfg.prefix, window=cfg.window,
             chunk=cfg.chunk, n_heads_q=cfg.n_heads_q, n_heads_kv=cfg.n_heads_kv,
             head_dim=cfg.head_dim, rank=cfg.rank, mlp_hidden=cfg.mlp_hidden, topk=cfg.topk,
             n_resid=cfg.n_resid, n_cand=cfg.n_cand,
             coeff_fmt=FMT_INT4_G32 if cfg.int4 else FMT_BF16,
             resid_fmt=FMT_INT4_G32 if cfg.int4 else FMT_BF16,
             rope_theta=cfg.rope_theta, softmax_scale=cfg.head_dim ** -0.5)
    f.update(over)
    return LowramShape(**f)


def make_cache(tensors: dict) -> LowramLayerCache:
    """The C struct of device pointers. It keeps references to the tensors, so
    their memory stays allocated for as long as the struct is in use (a freed
    block can be returned to the HIP runtime, e.g. by torch.cuda.empty_cache())."""
    c = LowramLayerCache(**{n: (tensors[n].data_ptr() if tensors.get(n) is not None else None)
                            for n in CACHE_FIELDS})
    c._tensors = dict(tensors)
    return c


# ------------------------------------------------------------- entry points --
def abi_version() -> int:
    return lib().lowram_abi_version()


def workspace_bytes(shape: LowramShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().lowram_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)), "lowram_workspace_bytes")
    return n.value


def decode_plan(shape: LowramShape, n_cu: int, mode: int = 0) -> dict:
    """lowram_decode_plan: how the selected chunks are scheduled on n_cu CUs
    (mode 0 automatic, 1 producer/consumer forced, 2 4-wave forced)."""
    p = LowramAttendPlan()
    _check(lib().lowram_decode_plan(ctypes.byref(shape), int(n_cu), int(mode), ctypes.byref(p)),
           "lowram_decode_plan")
    return {n: getattr(p, n) for n, _ in LowramAttendPlan._fields_}


def decode_step(shape, cache, q, out, workspace, sel_out=None, stream=None) -> None:
    """lowram_decode_step on device tensors (cache: LowramLayerCache or dict)."""
    c = cache if isinstance(cache, LowramLayerCache) else make_cache(cache)
    _check(lib().lowram_decode_step(ctypes.byref(shape), ctypes.byref(c), _ptr(q), _ptr(out),
                                    _ptr(sel_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "lowram_decode_step")


def decode_step_noalloc(shape, cache, q, out, sel_out=None, stream=None) -> None:
    """lowram_decode_step_noalloc: the decode step on the library's fixed scratch (no workspace)."""
    c = cache if isinstance(cache, LowramLayerCache) else make_cache(cache)
    _check(lib().lowram_decode_step_noalloc(ctypes.byref(shape), ctypes.byref(c), _ptr(q), _ptr(out),
                                            _ptr(sel_out), _stream(stream)), "lowram_decode_step_noalloc")


def decode_step_events(shape, cache, q, out, workspace, events, sel_out=None, stream=None) -> None:
    """lowram_decode_step recording 5 torch.cuda.Event (enable_timing) around its kernels."""
    c = cache if isinstance(cache, LowramLayerCache) else make_cache(cache)
    arr = (ctypes.c_void_p * 5)(*[ctypes.c_void_p(e.cuda_event) for e in events])
    _check(lib().lowram_decode_step_events(ctypes.byref(shape), ctypes.byref(c), _ptr(q), _ptr(out),
                                           _ptr(sel_out), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream), arr),
           "lowram_decode_step_events")


def decode_shared(shape, cache, q, out, workspace, sel_out=None, events=None, stream=None) -> None:
    """lowram_decode_shared: shape.batch queries against one context (cache arrays for NB = 1)."""
    c = cache if isinstance(cache, LowramLayerCache) else make_cache(cache)
    arr = None if events is None else (ctypes.c_void_p * 5)(*[ctypes.c_void_p(e.cuda_event) for e in events])
    _check(lib().lowram_decode_shared(ctypes.byref(shape), ctypes.byref(c), _ptr(q), _ptr(out), _ptr(sel_out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream), arr), "lowram_decode_shared")


def decode_stages(shape, cache, q, out, workspace, sel_out=None, scores=None, kpre=None, kpost=None,
                  vhat=None, stream=None) -> None:
    c = cache if isinstance(cache, LowramLayerCache) else make_cache(cache)
    _check(lib().lowram_decode_stages(ctypes.byref(shape), ctypes.byref(c), _ptr(q), _ptr(out),
                                      _ptr(sel_out), _ptr(scores), _ptr(kpre), _ptr(kpost), _ptr(vhat),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "lowram_decode_stages")


def dense_shape(batch, ctx_len, n_heads_q, n_heads_kv, head_dim=128, softmax_scale=None) -> DenseShape:
    return DenseShape(batch=batch, ctx_len=ctx_len, n_heads_q=n_heads_q, n_heads_kv=n_heads_kv,
                      head_dim=head_dim, softmax_scale=head_dim ** -0.5 if softmax_scale is None else softmax_scale)


def dense_workspace_bytes(shape: DenseShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dense_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)), "dense_workspace_bytes")
    return n.value


def dense_decode_step(shape, k, v, q, out, workspace, stream=None) -> None:
    c = DenseLayerCache(k=k.data_ptr(), v=v.data_ptr())
    _check(lib().dense_decode_step(ctypes.byref(shape), ctypes.byref(c), _ptr(q), _ptr(out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "dense_decode_step")


def resid_chunk_desc(res_idx, n_lists: int, n_resid: int, n_chunks: int, chunk: int, out,
                     stream=None) -> None:
    """res_idx [n_lists][n_resid] int32 (ascending rows) -> out [n_lists][n_chunks] uint32 (int32 tensor)."""
    _check(lib().lowram_resid_chunk_desc(_ptr(res_idx), n_lists, n_resid, n_chunks, chunk, _ptr(out),
                                         _stream(stream)), "lowram_resid_chunk_desc")


# ------------------------------------------------------------ cache builder --
def make_build_shape(cfg, batch: int | None = None, **over) -> LowramBuildShape:
    """lowram_build_shape of a workload (synth.Config-like object)."""
    f = dict(batch=cfg.batch if batch is None else batch, ctx_len=cfg.ctx, window=cfg.window,
             chunk=cfg.chunk, n_heads_kv=cfg.n_heads_kv, head_dim=cfg.head_dim, rank=cfg.rank,
             group_layers=cfg.group_layers, mlp_hidden=cfg.mlp_hidden, n_resid=cfg.n_resid,
             coeff_fmt=FMT_INT4_G32 if cfg.int4 else FMT_BF16,
             resid_fmt=FMT_INT4_G32 if cfg.int4 else FMT_BF16, rope_theta=cfg.rope_theta)
    f.update(over)
    return LowramBuildShape(**f)


def build_coeff(shape, keys, basis, coeff, coeff_scale=None, stream=None) -> None:
    """lowram_build_coeff: keys [NB][T][D], basis [NB][r][D] -> coeff (+ scales)."""
    _check(lib().lowram_build_coeff(ctypes.byref(shape), _ptr(keys), _ptr(basis), _ptr(coeff), _ptr(coeff_scale),
                                    _stream(stream)), "lowram_build_coeff")


def build_layer_workspace_bytes(shape: LowramBuildShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().lowram_build_layer_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)),
           "lowram_build_layer_workspace_bytes")
    return n.value


def build_layer(shape, layer_in_group: int, io: dict, workspace, stream=None, events=None) -> None:
    """lowram_build_layer (or _events with 5 torch.cuda.Event); io maps the
    lowram_layer_build field names to device tensors (or None)."""
    b = LowramLayerBuild(**{n: (io[n].data_ptr() if io.get(n) is not None else None) for n in BUILD_FIELDS})
    ws_ptr = _ptr(workspace)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if events is None:
        _check(lib().lowram_build_layer(ctypes.byref(shape), layer_in_group, ctypes.byref(b), ws_ptr, ws_n,
                                        _stream(stream)), "lowram_build_layer")
        return
    arr = (ctypes.c_void_p * 5)(*[ctypes.c_void_p(e.cuda_event) for e in events])
    _check(lib().lowram_build_layer_events(ctypes.byref(shape), layer_in_group, ctypes.byref(b), ws_ptr, ws_n,
                                           _stream(stream), arr), "lowram_build_layer_events")


# ----------------------------------------------------------- window rollover --
def append_coeff(shape, group_layers: int, keys_new, basis, coeff, coeff_scale=None, stream=None) -> None:
    """lowram_append_coeff: coefficient rows P .. P+S-1 of the group."""
    _check(lib().lowram_append_coeff(ctypes.byref(shape), group_layers, _ptr(keys_new), _ptr(basis), _ptr(coeff),
                                     _ptr(coeff_scale), _stream(stream)), "lowram_append_coeff")


def append_layer(shape, group_layers: int, layer_in_group: int, cache, io: dict, stream=None) -> None:
    """lowram_append_layer; io maps the lowram_layer_append field names to device tensors."""
    c = cache if isinstance(cache, LowramLayerCache) else make_cache(cache)
    a = LowramLayerAppend(**{n: (io[n].data_ptr() if io.get(n) is not None else None) for n in APPEND_FIELDS})
    _check(lib().lowram_append_layer(ctypes.byref(shape), group_layers, layer_in_group, ctypes.byref(c),
                                     ctypes.byref(a), _stream(stream)), "lowram_append_layer")


# ------------------------------------------------------------------ basis fit --
def fit_shape(batch, ctx_len, prefix_len, group_dim, rank, power=1) -> LowramFitShape:
    return LowramFitShape(batch=batch, ctx_len=ctx_len, prefix_len=prefix_len, group_dim=group_dim, rank=rank,
                          power=power)


def fit_basis_workspace_bytes(shape: LowramFitShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().lowram_fit_basis_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)),
           "lowram_fit_basis_workspace_bytes")
    return n.value


def fit_basis(shape, keys, omega_t, basis, status, workspace, stream=None) -> None:
    """lowram_fit_basis: keys [NB][T][D], omega_t [NB][r][P] -> basis [NB][r][D], status [NB]."""
    _check(lib().lowram_fit_basis(ctypes.byref(shape), _ptr(keys), _ptr(omega_t), _ptr(basis), _ptr(status),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "lowram_fit_basis")
