"""Python binding of libshardmm (include/shardmm.h), the sharded-matmul hot
path on one MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. The functions carry the C-ABI names (``sm_plan``,
``sm_local_gemm``, ``sm_reduce_partials``, ``sm_gather_shards``, ...) and
raise ``ShardmmError`` for any non-OK status. PyTorch provides device
memory and streams; buffers are passed as ``sm_buf`` descriptors built by
``buf()`` from tensors.

There is no fallback: if libshardmm.so cannot be loaded the import of the
device entry points raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Iterable, Mapping, Optional, Sequence, Tuple, Union

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libshardmm.so")

SM_MAX_AXES = 4
SM_NAME_LEN = 8
SM_ABI_VERSION = 2

# sm_status
SM_OK = 0
SM_ERR_ARG = 1
SM_ERR_MESH = 2
SM_ERR_SPEC = 3
SM_ERR_AXIS_REUSED = 4
SM_ERR_SHAPE = 5
SM_ERR_INDIVISIBLE = 6
SM_ERR_J_MISMATCH = 7
SM_ERR_NEEDS_GATHER = 8
SM_ERR_UNREDUCED = 9
SM_ERR_CASE = 10
SM_ERR_DTYPE = 11
SM_ERR_ALIGN = 12
SM_ERR_HIP = 13
# sm_case
SM_CASE1, SM_CASE2, SM_CASE3, SM_CASE4 = 1, 2, 3, 4
# sm_dtype
SM_BF16, SM_F32 = 0, 1
# sm_reduce_mode
SM_ALLREDUCE, SM_REDUCESCATTER = 0, 1
# sm_epilogue
SM_EPI_STORE, SM_EPI_GELU_TANH = 0, 1
# sm_what
SM_WHAT_A, SM_WHAT_B, SM_WHAT_C_BLOCKS, SM_WHAT_C_SCATTERED, SM_WHAT_C_PARTIAL = 0, 1, 2, 3, 4

EXPORTED = (
    "sm_abi_version", "sm_plan_size", "sm_build_digest", "sm_status_str", "sm_last_error", "sm_mesh_init",
    "sm_parse_spec", "sm_plan", "sm_rank_info", "sm_local_gemm", "sm_reduce_partials",
    "sm_gather_shards", "sm_plan_gathered", "sm_local_gemm_reduce", "sm_reduce_scatter_layernorm",
    "sm_reshard", "sm_gemm_reduce_workspace", "sm_local_gemm_reduce_ws", "sm_local_gemm_reduce_noalloc",
)


class sm_mesh(ctypes.Structure):
    _fields_ = [("n_axes", ctypes.c_int32),
                ("names", (ctypes.c_char * SM_NAME_LEN) * SM_MAX_AXES),
                ("sizes", ctypes.c_int32 * SM_MAX_AXES)]

    def axes(self):
        return [(self.names[a].value.decode(), self.sizes[a]) for a in range(self.n_axes)]


class sm_spec(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32 * 2),
                ("axes", (ctypes.c_int32 * SM_MAX_AXES) * 2)]

    def dims(self) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
        return tuple(tuple(self.axes[d][k] for k in range(self.n[d])) for d in range(2))  # type: ignore


class sm_plan_t(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("kase", ctypes.c_int32), ("n_ranks", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("n_partials", ctypes.c_int32), ("n_groups", ctypes.c_int32), ("n_units", ctypes.c_int32),
                ("I", ctypes.c_int64), ("J", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a_local", ctypes.c_int64 * 2), ("b_local", ctypes.c_int64 * 2), ("c_local", ctypes.c_int64 * 2),
                ("a_grid", ctypes.c_int32 * 2), ("b_grid", ctypes.c_int32 * 2), ("c_grid", ctypes.c_int32 * 2),
                ("a_copies", ctypes.c_int32), ("b_copies", ctypes.c_int32), ("c_copies", ctypes.c_int32),
                ("reduce_axes", ctypes.c_uint32), ("gather_operand", ctypes.c_int32),
                ("gather_axes", ctypes.c_uint32),
                ("mesh", sm_mesh), ("a", sm_spec), ("b", sm_spec), ("c", sm_spec), ("c_rs", sm_spec)]


class sm_rank_info_t(ctypes.Structure):
    _fields_ = [("coords", ctypes.c_int32 * SM_MAX_AXES),
                ("unit", ctypes.c_int32), ("group", ctypes.c_int32), ("partial", ctypes.c_int32),
                ("a_block", ctypes.c_int32 * 2), ("b_block", ctypes.c_int32 * 2), ("c_block", ctypes.c_int32 * 2),
                ("a_row0", ctypes.c_int64), ("a_col0", ctypes.c_int64),
                ("b_row0", ctypes.c_int64), ("b_col0", ctypes.c_int64),
                ("c_row0", ctypes.c_int64), ("c_col0", ctypes.c_int64),
                ("rs_row0", ctypes.c_int64), ("rs_rows", ctypes.c_int64)]


class sm_buf(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("ld", ctypes.c_int64),
                ("block_stride", ctypes.c_int64), ("elems", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ShardmmError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} ({status}): {detail}")
        self.status = status
        self.name = name
        self.detail = detail


_lib = None
_lib_path = None
_lock = threading.Lock()


def ensure_fresh(path: str = LIB_PATH) -> None:
    """Build the in-tree library when it is missing or its source stamp
    differs from the current sources; raise if that is needed and cannot be
    done (no hipcc), so that a stale build is never loaded."""
    from . import build as _build

    want = _build.source_digest()
    have = _build.library_digest(path)
    if have == want:
        return
    try:
        _build.build()
    except Exception as e:  # noqa: BLE001 - any build failure is reported the same way
        raise ShardmmError(SM_ERR_ARG, "SM_ERR_ARG",
                           f"{path} is {'missing' if have is None else 'older than its sources'} and could not be "
                           f"rebuilt: {e}") from e
    if _build.library_digest(path) != want:
        raise ShardmmError(SM_ERR_ARG, "SM_ERR_ARG", f"{path}: the rebuilt library carries another source stamp")


def load(path: Optional[str] = None):
    """Load libshardmm. The default is the in-tree libshardmm.so, rebuilt
    first if it is missing or older than its sources; the environment
    variable SHARDMM_LIB names another build to load instead (as is; a
    build of the host planner alone binds only the host calls)."""
    global _lib, _lib_path
    with _lock:
        if _lib is not None:
            return _lib
        path = path or os.environ.get("SHARDMM_LIB") or LIB_PATH
        if os.path.abspath(path) == os.path.abspath(LIB_PATH):
            ensure_fresh(path)
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.sm_abi_version.restype = i32
        lib.sm_abi_version.argtypes = []
        lib.sm_plan_size.restype = ctypes.c_size_t
        lib.sm_plan_size.argtypes = []
        lib.sm_build_digest.restype = ctypes.c_char_p
        lib.sm_build_digest.argtypes = []
        lib.sm_status_str.restype = ctypes.c_char_p
        lib.sm_status_str.argtypes = [i32]
        lib.sm_last_error.restype = ctypes.c_char_p
        lib.sm_last_error.argtypes = []
        lib.sm_mesh_init.restype = i32
        lib.sm_mesh_init.argtypes = [P(sm_mesh), i32, P(ctypes.c_char_p), P(i32)]
        lib.sm_parse_spec.restype = i32
        lib.sm_parse_spec.argtypes = [P(sm_mesh), ctypes.c_char_p, P(sm_spec)]
        lib.sm_plan.restype = i32
        lib.sm_plan.argtypes = [P(sm_mesh), P(sm_spec), P(sm_spec), i64, i64, i64, i32, i32, P(sm_plan_t)]
        lib.sm_rank_info.restype = i32
        lib.sm_rank_info.argtypes = [P(sm_plan_t), i32, P(sm_rank_info_t)]
        lib.sm_plan_gathered.restype = i32
        lib.sm_plan_gathered.argtypes = [P(sm_plan_t), P(sm_plan_t)]
        if hasattr(lib, "sm_local_gemm"):
            _bind_device_calls(lib)
        if lib.sm_abi_version() != SM_ABI_VERSION:
            raise ShardmmError(SM_ERR_ARG, "SM_ERR_ARG", "libshardmm ABI version mismatch")
        if lib.sm_plan_size() != ctypes.sizeof(sm_plan_t):
            raise ShardmmError(SM_ERR_ARG, "SM_ERR_ARG", "sm_plan_t layout mismatch")
        _lib, _lib_path = lib, path
        return lib


def _bind_device_calls(lib) -> None:
    P = ctypes.POINTER
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.sm_local_gemm.restype = i32
    lib.sm_local_gemm.argtypes = [P(sm_plan_t), P(sm_buf), P(sm_buf), P(sm_buf), i32, i32, i32, vp]
    lib.sm_reduce_partials.restype = i32
    lib.sm_reduce_partials.argtypes = [P(sm_plan_t), P(sm_buf), P(sm_buf), i32, i32, i32, vp]
    lib.sm_gather_shards.restype = i32
    lib.sm_gather_shards.argtypes = [P(sm_plan_t), i32, P(sm_buf), P(sm_buf), vp]
    lib.sm_local_gemm_reduce.restype = i32
    lib.sm_local_gemm_reduce.argtypes = [P(sm_plan_t), P(sm_buf), P(sm_buf), P(sm_buf), i32, i32, i32, vp]
    lib.sm_gemm_reduce_workspace.restype = i32
    lib.sm_gemm_reduce_workspace.argtypes = [P(sm_plan_t), i32, P(i64)]
    lib.sm_local_gemm_reduce_ws.restype = i32
    lib.sm_local_gemm_reduce_ws.argtypes = [P(sm_plan_t), P(sm_buf), P(sm_buf), P(sm_buf), i32, i32, i32, vp, i64,
                                            vp]
    lib.sm_local_gemm_reduce_noalloc.restype = i32
    lib.sm_local_gemm_reduce_noalloc.argtypes = [P(sm_plan_t), P(sm_buf), P(sm_buf), P(sm_buf), i32, i32, i32,
                                                 vp]
    lib.sm_reduce_scatter_layernorm.restype = i32
    lib.sm_reduce_scatter_layernorm.argtypes = [P(sm_plan_t), P(sm_buf), P(sm_buf), vp, vp, ctypes.c_float,
                                                i32, i32, vp]
    lib.sm_reshard.restype = i32
    lib.sm_reshard.argtypes = [P(sm_mesh), P(sm_spec), P(sm_spec), i64, i64, i32, P(sm_buf), P(sm_buf), vp]


def _check(status: int) -> None:
    if status != SM_OK:
        lib = load()
        raise ShardmmError(status, lib.sm_status_str(status).decode(), lib.sm_last_error().decode())


def sm_status_str(status: int) -> str:
    return load().sm_status_str(status).decode()


def sm_last_error() -> str:
    return load().sm_last_error().decode()


def sm_mesh_init(axes: Union[Mapping[str, int], Iterable[Tuple[str, int]]]) -> sm_mesh:
    items = list(axes.items()) if isinstance(axes, Mapping) else list(axes)
    names = (ctypes.c_char_p * len(items))(*[n.encode() for n, _ in items])
    sizes = (ctypes.c_int32 * len(items))(*[int(s) for _, s in items])
    m = sm_mesh()
    _check(load().sm_mesh_init(ctypes.byref(m), len(items), names, sizes))
    return m


def sm_parse_spec(mesh: sm_mesh, text: str) -> sm_spec:
    s = sm_spec()
    _check(load().sm_parse_spec(ctypes.byref(mesh), text.encode(), ctypes.byref(s)))
    return s


def sm_plan(mesh, a, b, I: int, J: int, K: int, in_dtype: int = SM_BF16, out_dtype: int = SM_F32) -> sm_plan_t:
    """Plan A[I,J].B[J,K]; ``mesh`` may be an sm_mesh or a {name: size}
    mapping, ``a`` / ``b`` an sm_spec or spec text."""
    if not isinstance(mesh, sm_mesh):
        mesh = sm_mesh_init(mesh)
    if isinstance(a, str):
        a = sm_parse_spec(mesh, a)
    if isinstance(b, str):
        b = sm_parse_spec(mesh, b)
    p = sm_plan_t()
    _check(load().sm_plan(ctypes.byref(mesh), ctypes.byref(a), ctypes.byref(b), I, J, K, in_dtype, out_dtype,
                          ctypes.byref(p)))
    return p


def sm_rank_info(plan: sm_plan_t, rank: int) -> sm_rank_info_t:
    r = sm_rank_info_t()
    _check(load().sm_rank_info(ctypes.byref(plan), rank, ctypes.byref(r)))
    return r


def _dtype_of(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return SM_BF16
    if t.dtype == torch.float32:
        return SM_F32
    raise ValueError(f"buffers hold bfloat16 or float32 elements, not {t.dtype}")


def buf(t, ld: Optional[int] = None, block_stride: Optional[int] = None) -> sm_buf:
    """sm_buf for a contiguous tensor: 2-D [rows, ld] = global layout
    (block_stride 0), 3-D [blocks, rows, ld] = stacked layout."""
    if not t.is_contiguous():
        raise ValueError("buffers must be contiguous tensors")
    if ld is None:
        ld = t.shape[-1]
    if block_stride is None:
        block_stride = t.shape[-2] * t.shape[-1] if t.dim() == 3 else 0
    b = sm_buf(ctypes.c_void_p(t.data_ptr()), int(ld), int(block_stride), int(t.numel()), _dtype_of(t), 0)
    b._tensor = t  # keep the memory alive as long as the descriptor
    return b


def _stream(stream):
    if stream is None:
        import torch

        if not torch.cuda.is_available():
            return ctypes.c_void_p(0)  # no device: the call can only fail validation
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _as_buf(x) -> sm_buf:
    return x if isinstance(x, sm_buf) else buf(x)


def sm_local_gemm(plan: sm_plan_t, A, B, C, epilogue: int = SM_EPI_STORE, unit_begin: int = 0,
                  unit_count: Optional[int] = None, stream=None) -> None:
    if unit_count is None:
        unit_count = plan.n_units - unit_begin
    a, b, c = _as_buf(A), _as_buf(B), _as_buf(C)
    _check(load().sm_local_gemm(ctypes.byref(plan), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                epilogue, unit_begin, unit_count, _stream(stream)))


def sm_reduce_partials(plan: sm_plan_t, partials, out, mode: int = SM_ALLREDUCE, group_begin: int = 0,
                       group_count: Optional[int] = None, stream=None) -> None:
    if group_count is None:
        group_count = plan.n_groups - group_begin
    p, o = _as_buf(partials), _as_buf(out)
    _check(load().sm_reduce_partials(ctypes.byref(plan), ctypes.byref(p), ctypes.byref(o), mode,
                                     group_begin, group_count, _stream(stream)))


def sm_plan_gathered(plan: sm_plan_t) -> sm_plan_t:
    q = sm_plan_t()
    _check(load().sm_plan_gathered(ctypes.byref(plan), ctypes.byref(q)))
    return q


def sm_local_gemm_reduce(plan: sm_plan_t, A, B, out, mode: int = SM_ALLREDUCE, group_begin: int = 0,
                         group_count: Optional[int] = None, stream=None) -> None:
    if group_count is None:
        group_count = plan.n_groups - group_begin
    a, b, o = _as_buf(A), _as_buf(B), _as_buf(out)
    _check(load().sm_local_gemm_reduce(ctypes.byref(plan), ctypes.byref(a), ctypes.byref(b), ctypes.byref(o),
                                       mode, group_begin, group_count, _stream(stream)))


def sm_gemm_reduce_workspace(plan: sm_plan_t, group_count: Optional[int] = None) -> int:
    """Workspace bytes sm_local_gemm_reduce_ws needs for ``group_count``
    groups (all of the plan's by default)."""
    if group_count is None:
        group_count = plan.n_groups
    n = ctypes.c_int64()
    _check(load().sm_gemm_reduce_workspace(ctypes.byref(plan), group_count, ctypes.byref(n)))
    return n.value


def sm_local_gemm_reduce_ws(plan: sm_plan_t, A, B, out, workspace, mode: int = SM_ALLREDUCE, group_begin: int = 0,
                            group_count: Optional[int] = None, stream=None) -> None:
    """``workspace``: a device tensor (zero-filled before its first use; each
    call leaves its counters zero) of at least sm_gemm_reduce_workspace
    bytes, a (pointer, bytes) pair, or None when the plan needs none."""
    if group_count is None:
        group_count = plan.n_groups - group_begin
    a, b, o = _as_buf(A), _as_buf(B), _as_buf(out)
    if workspace is None:
        wp, wn = ctypes.c_void_p(0), 0
    elif isinstance(workspace, tuple):
        wp, wn = ctypes.c_void_p(int(workspace[0])), int(workspace[1])
    else:
        if not workspace.is_contiguous():
            raise ValueError("the workspace must be a contiguous tensor")
        wp, wn = ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    _check(load().sm_local_gemm_reduce_ws(ctypes.byref(plan), ctypes.byref(a), ctypes.byref(b), ctypes.byref(o),
                                          mode, group_begin, group_count, wp, wn, _stream(stream)))


def sm_local_gemm_reduce_noalloc(plan: sm_plan_t, A, B, out, mode: int = SM_ALLREDUCE, group_begin: int = 0,
                                 group_count: Optional[int] = None, stream=None) -> None:
    """sm_local_gemm_reduce_ws on the library's static scratch: no workspace
    argument and no device allocation."""
    if group_count is None:
        group_count = plan.n_groups - group_begin
    a, b, o = _as_buf(A), _as_buf(B), _as_buf(out)
    _check(load().sm_local_gemm_reduce_noalloc(ctypes.byref(plan), ctypes.byref(a), ctypes.byref(b),
                                               ctypes.byref(o), mode, group_begin, group_count, _stream(stream)))


def sm_reduce_scatter_layernorm(plan: sm_plan_t, partials, out, gamma=None, beta=None, eps: float = 1e-5,
                                group_begin: int = 0, group_count: Optional[int] = None, stream=None) -> None:
    """gamma / beta: float32 device tensors of the row length, or None."""
    if group_count is None:
        group_count = plan.n_groups - group_begin
    p, o = _as_buf(partials), _as_buf(out)
    g = ctypes.c_void_p(gamma.data_ptr() if gamma is not None else 0)
    b = ctypes.c_void_p(beta.data_ptr() if beta is not None else 0)
    _check(load().sm_reduce_scatter_layernorm(ctypes.byref(plan), ctypes.byref(p), ctypes.byref(o), g, b,
                                              float(eps), group_begin, group_count, _stream(stream)))


def sm_reshard(mesh, frm, to, rows: int, cols: int, dtype: int, src, dst, stream=None) -> None:
    """``mesh``: sm_mesh or {name: size}; ``frm`` / ``to``: sm_spec or spec text."""
    if not isinstance(mesh, sm_mesh):
        mesh = sm_mesh_init(mesh)
    if isinstance(frm, str):
        frm = sm_parse_spec(mesh, frm)
    if isinstance(to, str):
        to = sm_parse_spec(mesh, to)
    s, d = _as_buf(src), _as_buf(dst)
    _check(load().sm_reshard(ctypes.byref(mesh), ctypes.byref(frm), ctypes.byref(to), rows, cols, dtype,
                             ctypes.byref(s), ctypes.byref(d), _stream(stream)))


def sm_gather_shards(plan: sm_plan_t, what: int, shards, out, stream=None) -> None:
    s, o = _as_buf(shards), _as_buf(out)
    _check(load().sm_gather_shards(ctypes.byref(plan), what, ctypes.byref(s), ctypes.byref(o), _stream(stream)))


def loaded_library_path() -> str:
    load()
    return _lib_path
