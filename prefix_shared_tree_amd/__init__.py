"""Python binding of libpst: prefix-shared tree decode attention on MI355X.

Argument marshalling only.  Every step of the computation (index, plan, the
partial-attention and reduction kernels) runs in the native library built
from ``csrc/`` (``python prefix_shared_tree_amd/build.py``).  If the library
is missing, importing this package raises: there is no fallback.

    import prefix_shared_tree_amd as pst
    tree = pst.Tree(parent, kv_offset, kv_len, query_node, num_q_heads=32,
                    num_kv_heads=8, head_dim=128, dtype="bf16")
    plan = pst.Plan(tree)                 # reusable across decode steps
    out, lse = pst.decode_attn(plan, q, k_pool, v_pool)

PyTorch is used for device memory and streams only: tensors are passed to
the library as raw pointers, kernels run on torch's current stream.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpst.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python prefix_shared_tree_amd/build.py` "
        "(the HIP library is required; there is no fallback path)")

# libpst.so links against libamdhip64.so.7.  PyTorch ships its own HIP
# runtime under the same soname: importing torch first makes the library bind
# to that one, so device pointers and stream handles from torch are valid in
# the library (one HIP runtime per process).
try:
    import torch as _torch  # noqa: F401
except ImportError:  # pragma: no cover - torch is the memory/stream plumbing
    _torch = None

_lib = C.CDLL(LIB_PATH)

PST_F32, PST_BF16 = 0, 1
TREE_HOST_ONLY = 1
PLAN_QUERY_GUIDED, PLAN_NO_SPLIT, PLAN_HOST_ONLY, PLAN_DOT_SMALL, PLAN_FLATTEN = 1, 2, 4, 8, 16
TASK_FIELDS = 8

STATUS = {
    0: "PST_OK", 1: "PST_E_INVALID_ARG", 2: "PST_E_INVALID_TREE", 3: "PST_E_UNSUPPORTED",
    4: "PST_E_OOM", 5: "PST_E_PLAN_STALE", 6: "PST_E_WORKSPACE", 7: "PST_E_HIP", 8: "PST_E_NO_DEVICE",
}

EXPORTS = [
    "pst_tree_build", "pst_tree_set_lengths", "pst_tree_get_index", "pst_cost_model_create",
    "pst_cost_model_lookup", "pst_plan", "pst_plan_workspace_size", "pst_plan_get", "pst_decode_attn",
    "pst_pac", "pst_por", "pst_free", "pst_last_error", "pst_device_info", "pst_bench_flush",
    "pst_bench_read", "pst_cost_model_load", "pst_baseline_workspace_size", "pst_decode_attn_baseline",
    "pst_decode_attn_noalloc", "pst_write_kv_rows", "pst_tree_append",
]
NOALLOC_SCRATCH_BYTES = 128 << 20  # PST_NOALLOC_SCRATCH_BYTES


class PstError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.code = STATUS.get(status, str(status))
        super().__init__(f"{self.code}: {message}")


class _TreeDesc(C.Structure):
    _fields_ = [("num_nodes", C.c_int32), ("parent", C.c_void_p), ("kv_offset", C.c_void_p),
                ("kv_len", C.c_void_p), ("num_queries", C.c_int32), ("query_node", C.c_void_p),
                ("query_mask", C.c_void_p), ("node_masked", C.c_void_p), ("page_size", C.c_int32),
                ("page_ptr", C.c_void_p), ("page_idx", C.c_void_p)]


class _Shape(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("in_dtype", C.c_int32), ("out_dtype", C.c_int32), ("scale", C.c_float),
                ("kv_stride_head", C.c_int64), ("kv_stride_token", C.c_int64), ("pool_tokens", C.c_int64)]


class _IndexView(C.Structure):
    _fields_ = [("num_nodes", C.c_int32), ("num_queries", C.c_int32), ("num_entries", C.c_int64),
                ("depth", C.c_void_p), ("n_q", C.c_void_p), ("qn_ptr", C.c_void_p), ("qn_idx", C.c_void_p),
                ("nq_ptr", C.c_void_p), ("nq_idx", C.c_void_p), ("nq_mask", C.c_void_p), ("visible", C.c_void_p),
                ("page_size", C.c_int32), ("page_ptr", C.c_void_p), ("page_idx", C.c_void_p)]


class _PlanOpts(C.Structure):
    _fields_ = [("num_bins", C.c_int32), ("max_rows", C.c_int32), ("tile", C.c_int32),
                ("grid_steps", C.c_int32), ("fixed_chunk", C.c_int32), ("flags", C.c_uint32)]


class _PlanView(C.Structure):
    _fields_ = [("num_bins", C.c_int32), ("num_tasks", C.c_int32), ("num_queries", C.c_int32),
                ("num_nodes", C.c_int32), ("num_slots", C.c_int64), ("num_entries", C.c_int64),
                ("tasks", C.c_void_p), ("bin_ptr", C.c_void_p), ("slot_ptr", C.c_void_p),
                ("entry_slot", C.c_void_p), ("piece_len", C.c_void_p), ("b_eff", C.c_void_p),
                ("rows_per_group", C.c_void_p), ("bin_load", C.c_void_p), ("makespan", C.c_int64),
                ("cost_l", C.c_int64), ("chosen_k", C.c_int32), ("max_rows", C.c_int32),
                ("mfma_min_rows", C.c_int32), ("flat_chunk", C.c_int32), ("num_chunks", C.c_int32),
                ("flat_ptr", C.c_void_p), ("flat_query", C.c_void_p), ("flat_mask", C.c_void_p),
                ("flat_rows", C.c_void_p)]


_P = C.c_void_p
_sig = {
    "pst_tree_build": [C.POINTER(_TreeDesc), C.POINTER(_Shape), C.c_uint32, _P, C.POINTER(_P)],
    "pst_tree_set_lengths": [_P, _P, _P],
    "pst_tree_get_index": [_P, C.POINTER(_IndexView)],
    "pst_cost_model_create": [C.c_int32, _P, C.c_int32, _P, _P, C.POINTER(_P)],
    "pst_cost_model_lookup": [_P, C.c_int32, C.c_int64, C.POINTER(C.c_int64)],
    "pst_plan": [_P, _P, C.POINTER(_PlanOpts), _P, C.POINTER(_P)],
    "pst_plan_workspace_size": [_P, C.POINTER(C.c_size_t)],
    "pst_plan_get": [_P, C.POINTER(_PlanView)],
    "pst_decode_attn": [_P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P],
    "pst_pac": [_P, _P, _P, _P, _P, C.c_size_t, _P],
    "pst_por": [_P, _P, _P, _P, C.c_size_t, _P],
    "pst_free": [_P],
    "pst_device_info": [C.POINTER(C.c_int32), C.POINTER(C.c_int32)],
    "pst_bench_flush": [_P, C.c_size_t, _P],
    "pst_bench_read": [_P, C.c_size_t, _P, _P],
    "pst_cost_model_load": [C.c_char_p, C.POINTER(_P)],
    "pst_baseline_workspace_size": [_P, _P, _P, C.POINTER(C.c_size_t)],
    "pst_decode_attn_baseline": [_P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P],
    "pst_decode_attn_noalloc": [_P, _P, _P, _P, _P, _P, _P],
    "pst_write_kv_rows": [_P, _P, _P, _P, C.c_int32, _P, _P, _P],
    "pst_tree_append": [_P, C.c_int32, _P, _P, _P, _P, _P, _P],
}
for _name, _args in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = C.c_int
_lib.pst_last_error.argtypes = []
_lib.pst_last_error.restype = C.c_char_p


def _check(status: int):
    if status != 0:
        raise PstError(status, _lib.pst_last_error().decode())


def _arr(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(C.c_void_p)


def _view(ptr, count, dtype):
    if count == 0 or not ptr:
        return np.zeros(0, dtype=dtype)
    buf = (C.c_char * (count * np.dtype(dtype).itemsize)).from_address(ptr)
    return np.frombuffer(buf, dtype=dtype, count=count).copy()


def _stream(stream):
    """A hipStream_t for the C ABI: a raw handle, a torch stream, or None (torch's current stream)."""
    if stream is not None:
        return C.c_void_p(int(getattr(stream, "cuda_stream", stream)))
    import torch

    if torch.cuda.is_available():
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return C.c_void_p(0)


def _dtype_code(dtype) -> int:
    if dtype in ("f32", "float32", PST_F32):
        return PST_F32
    if dtype in ("bf16", "bfloat16", PST_BF16):
        return PST_BF16
    import torch

    if dtype == torch.float32:
        return PST_F32
    if dtype == torch.bfloat16:
        return PST_BF16
    raise ValueError(f"unsupported dtype {dtype}")


class Tree:
    """A validated tree and its index (``pst_tree_build``).

    Contiguous K/V: node i is the run of ``kv_len[i]`` pool rows from
    ``kv_offset[i]``.  Paged K/V (``page_size`` > 0, ``kv_offset`` may be
    None): token j of node i is pool row
    ``page_idx[page_ptr[i] + j // page_size] * page_size + j % page_size``.
    """

    def __init__(self, parent, kv_offset, kv_len, query_node, *, num_q_heads, num_kv_heads, head_dim,
                 dtype="bf16", out_dtype=None, query_mask=None, node_masked=None, scale=0.0,
                 kv_stride_head=0, kv_stride_token=0, pool_tokens=0, page_size=0, page_ptr=None, page_idx=None,
                 host_only=False, stream=None):
        self._h = C.c_void_p()
        parent, p_parent = _arr(parent, np.int32)
        kv_len, p_len = _arr(kv_len, np.int32)
        if kv_offset is None:
            kv_offset = np.zeros(len(kv_len), dtype=np.int64)
        kv_offset, p_off = _arr(kv_offset, np.int64)
        query_node, p_qn = _arr(query_node, np.int32)
        keep = [parent, kv_offset, kv_len, query_node]
        p_pp = p_pi = None
        if page_size:
            page_ptr, p_pp = _arr(page_ptr, np.int32)
            page_idx, p_pi = _arr(page_idx if page_idx is not None else np.zeros(0), np.int32)
            keep += [page_ptr, page_idx]
        p_qm = p_nm = None
        if query_mask is not None:
            qm, p_qm = _arr(query_mask, np.uint64)
            keep.append(qm)
        if node_masked is not None:
            nm, p_nm = _arr(node_masked, np.uint8)
            keep.append(nm)
        desc = _TreeDesc(len(parent), p_parent, p_off, p_len, len(query_node), p_qn, p_qm, p_nm, int(page_size),
                         p_pp, p_pi)
        self.in_dtype = _dtype_code(dtype)
        self.out_dtype = self.in_dtype if out_dtype is None else _dtype_code(out_dtype)
        shape = _Shape(num_q_heads, num_kv_heads, head_dim, self.in_dtype, self.out_dtype, scale,
                       kv_stride_head, kv_stride_token, pool_tokens)
        if not host_only:
            _init_device()
        strm = C.c_void_p(0) if host_only else _stream(stream)
        _check(_lib.pst_tree_build(C.byref(desc), C.byref(shape), TREE_HOST_ONLY if host_only else 0, strm,
                                   C.byref(self._h)))
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.num_nodes, self.num_queries = len(parent), len(query_node)
        self.host_only = host_only
        self.page_size = int(page_size)
        # Elements the K/V layout addresses (the last channel of the last token of the last head).
        if pool_tokens > 0:
            pool = pool_tokens
        elif page_size:
            pool = (int(page_idx.max()) + 1) * int(page_size) if len(page_idx) else 0
        else:
            pool = int((kv_offset + kv_len).max()) if len(kv_len) else 0
        st_tok = kv_stride_token if kv_stride_token > 0 else head_dim
        st_head = kv_stride_head if kv_stride_head > 0 else pool * head_dim
        self.kv_extent = 0 if pool == 0 else (num_kv_heads - 1) * st_head + (pool - 1) * st_tok + head_dim

    @classmethod
    def from_spec(cls, spec, **kw):
        """Build from a ``workloads.TreeSpec``-like object (attributes of the same names)."""
        return cls(spec.parent, spec.kv_offset, spec.kv_len, spec.query_node, num_q_heads=spec.num_q_heads,
                   num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim, dtype=spec.dtype,
                   query_mask=spec.query_mask, node_masked=spec.node_masked, **kw)

    @classmethod
    def from_paged(cls, spec, paged, **kw):
        """Build ``spec``'s tree over a paged pool: ``paged`` holds ``page_size``,
        ``page_ptr`` and ``page_idx`` (see ``workloads.page_pools``)."""
        return cls(spec.parent, None, spec.kv_len, spec.query_node, num_q_heads=spec.num_q_heads,
                   num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim, dtype=spec.dtype,
                   query_mask=spec.query_mask, node_masked=spec.node_masked, page_size=paged["page_size"],
                   page_ptr=paged["page_ptr"], page_idx=paged["page_idx"], **kw)

    def index(self) -> dict:
        v = _IndexView()
        _check(_lib.pst_tree_get_index(self._h, C.byref(v)))
        N, B, E = v.num_nodes, v.num_queries, v.num_entries
        return {
            "depth": _view(v.depth, N, np.int32), "n_q": _view(v.n_q, N, np.int32),
            "qn_ptr": _view(v.qn_ptr, B + 1, np.int32), "qn_idx": _view(v.qn_idx, E, np.int32),
            "nq_ptr": _view(v.nq_ptr, N + 1, np.int32), "nq_idx": _view(v.nq_idx, E, np.int32),
            "nq_mask": _view(v.nq_mask, E, np.uint64), "visible": _view(v.visible, B, np.int64),
            "page_size": int(v.page_size),
            "page_ptr": _view(v.page_ptr, N + 1, np.int32) if v.page_size else None,
            "page_idx": (_view(v.page_idx, int(_view(v.page_ptr, N + 1, np.int32)[-1]), np.int32)
                         if v.page_size else None),
        }

    def set_lengths(self, kv_len, stream=None):
        kv_len, p = _arr(kv_len, np.int32)
        if kv_len.shape != (self.num_nodes,):
            raise ValueError(f"kv_len needs one length per node ({self.num_nodes}), got shape {kv_len.shape}")
        _check(_lib.pst_tree_set_lengths(self._h, p, _stream(stream) if not self.host_only else C.c_void_p(0)))

    def append(self, nodes, k_new, v_new, k_pool, v_pool, stream=None):
        """``pst_tree_append``: node ``nodes[i]`` gains one token whose K/V are
        ``k_new[i]``, ``v_new[i]`` ([n, H_kv, d] on the GPU), written at the
        node's next position in the pools."""
        import torch

        nodes, p = _arr(nodes, np.int32)
        idt = torch.float32 if self.in_dtype == PST_F32 else torch.bfloat16
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            _check_one(name, t, idt)
            if t.numel() != len(nodes) * self.num_kv_heads * self.head_dim:
                raise ValueError(f"{name} must hold [n, num_kv_heads, head_dim] elements")
        for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
            _check_one(name, t, idt)
            if t.numel() < self.kv_extent:
                raise ValueError(f"{name} holds fewer than the {self.kv_extent} elements the tree's layout addresses")
        _check(_lib.pst_tree_append(self._h, len(nodes), p, _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                    _stream(stream)))

    def free(self):
        if self._h:
            _check(_lib.pst_free(self._h))
            self._h = C.c_void_p()

    def __del__(self):
        try:
            if self._h:
                _lib.pst_free(self._h)
        except Exception:
            pass


class CostModel:
    """C_est table (``pst_cost_model_create``): rows grid x length grid, integer ns."""

    def __init__(self, rows_grid, len_grid, table):
        self._h = C.c_void_p()
        rg, p_rg = _arr(rows_grid, np.int32)
        lg, p_lg = _arr(len_grid, np.int32)
        tb, p_tb = _arr(np.asarray(table).reshape(len(rg), len(lg)), np.int64)
        _check(_lib.pst_cost_model_create(len(rg), p_rg, len(lg), p_lg, p_tb, C.byref(self._h)))
        self.path = None

    @classmethod
    def load(cls, path):
        """A fitted table from its JSON file (``pst_cost_model_load``)."""
        self = cls.__new__(cls)
        self._h = C.c_void_p()
        _check(_lib.pst_cost_model_load(os.fsencode(path), C.byref(self._h)))
        self.path = path
        return self

    def lookup(self, rows: int, length: int) -> int:
        out = C.c_int64()
        _check(_lib.pst_cost_model_lookup(self._h, rows, length, C.byref(out)))
        return out.value

    def __del__(self):
        try:
            if self._h:
                _lib.pst_free(self._h)
        except Exception:
            pass


def default_cost_model(head_dim: int, num_q_heads: int, num_kv_heads: int, dtype) -> Optional[CostModel]:
    """The fitted gfx950 table shipped for this head layout, if there is one."""
    name = f"gfx950_{'bf16' if _dtype_code(dtype) == PST_BF16 else 'f32'}_q{num_q_heads}_kv{num_kv_heads}_d{head_dim}.json"
    path = os.path.join(_HERE, "cost_tables", name)
    if path not in _COST_CACHE:
        _COST_CACHE[path] = CostModel.load(path) if os.path.exists(path) else None
    return _COST_CACHE[path]


_COST_CACHE: dict = {}  # fitted tables by path (read-only once loaded)


class Plan:
    """A partition of the tree's partial attention (``pst_plan``); reusable across decode steps."""

    def __init__(self, tree: Tree, cost: Optional[CostModel] = None, *, num_bins=0, max_rows=0, tile=0,
                 grid_steps=0, fixed_chunk=0, query_guided=False, no_split=False, host_only=False, stream=None,
                 use_fitted=True, dot_small=False, flatten=0):
        """``flatten`` > 0: the DEFT-Flatten partition with chunks of that many
        tokens (a multiple of 128) instead of the cost-model partition."""
        self.tree = tree
        if cost is None and use_fitted:
            cost = default_cost_model(tree.head_dim, tree.num_q_heads, tree.num_kv_heads, tree.in_dtype)
        self.cost = cost
        flags = (PLAN_QUERY_GUIDED if query_guided else 0) | (PLAN_NO_SPLIT if no_split else 0) | \
                (PLAN_HOST_ONLY if host_only else 0) | (PLAN_DOT_SMALL if dot_small else 0) | \
                (PLAN_FLATTEN if flatten else 0)
        if flatten:
            fixed_chunk = int(flatten)
        opts = _PlanOpts(num_bins, max_rows, tile, grid_steps, fixed_chunk, flags)
        self._h = C.c_void_p()
        host = host_only or tree.host_only
        _check(_lib.pst_plan(tree._h, cost._h if cost is not None else None, C.byref(opts),
                             C.c_void_p(0) if host else _stream(stream), C.byref(self._h)))
        n = C.c_size_t()
        _check(_lib.pst_plan_workspace_size(self._h, C.byref(n)))
        self.workspace_bytes = n.value

    def view(self) -> dict:
        v = _PlanView()
        _check(_lib.pst_plan_get(self._h, C.byref(v)))
        return {
            "num_bins": v.num_bins, "num_slots": v.num_slots, "makespan": v.makespan, "cost_l": v.cost_l,
            "chosen_k": v.chosen_k, "max_rows": v.max_rows, "mfma_min_rows": v.mfma_min_rows,
            "tasks": _view(v.tasks, v.num_tasks * TASK_FIELDS, np.int32).reshape(-1, TASK_FIELDS),
            "bin_ptr": _view(v.bin_ptr, v.num_bins + 1, np.int32),
            "slot_ptr": _view(v.slot_ptr, v.num_queries + 1, np.int64),
            "entry_slot": _view(v.entry_slot, v.num_entries, np.int64),
            "piece_len": _view(v.piece_len, v.num_nodes, np.int32),
            "b_eff": _view(v.b_eff, v.num_nodes, np.int32),
            "rows_per_group": _view(v.rows_per_group, v.num_nodes, np.int32),
            "bin_load": _view(v.bin_load, v.num_bins, np.int64),
            **self._flat_view(v),
        }

    @staticmethod
    def _flat_view(v) -> dict:
        if not v.flat_chunk:
            return {"flat_chunk": 0}
        W = v.flat_chunk // 64
        return {
            "flat_chunk": v.flat_chunk, "num_chunks": v.num_chunks,
            "flat_ptr": _view(v.flat_ptr, v.num_chunks + 1, np.int32),
            "flat_query": _view(v.flat_query, v.num_entries, np.int32),
            "flat_mask": _view(v.flat_mask, v.num_entries * W, np.uint64),
            "flat_rows": _view(v.flat_rows, v.num_chunks * v.flat_chunk, np.int32),
        }

    def free(self):
        if self._h:
            _check(_lib.pst_free(self._h))
            self._h = C.c_void_p()

    def __del__(self):
        try:
            if self._h:
                _lib.pst_free(self._h)
        except Exception:
            pass


def _check_one(name, t, dt):
    if t.dtype != dt:
        raise ValueError(f"{name} must be {dt}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")


def _check_tensors(tree, q, k_pool, v_pool, out, lse):
    """Sizes, dtypes and devices against the tree's shape: the C ABI only sees
    pointers, and the kernels size their reads from the plan, not from the
    tensors."""
    _check_inputs(tree, q, k_pool, v_pool)
    _check_outputs(tree, out, lse)


def _ptr(t):
    return C.c_void_p(0 if t is None else t.data_ptr())


def workspace(plan: Plan, device="cuda"):
    """A caller-owned workspace tensor of the plan's size (256-byte aligned by the caching allocator)."""
    import torch

    return torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=device)


def decode_attn(plan: Plan, q, k_pool, v_pool, *, out=None, lse=None, want_lse=True, ws=None, stream=None):
    """``pst_decode_attn``: returns (out [B, H_q, d], lse [B, H_q] float32 or None)."""
    import torch

    tree = plan.tree
    if out is None:
        odt = torch.float32 if tree.out_dtype == PST_F32 else torch.bfloat16
        out = torch.empty((tree.num_queries, tree.num_q_heads, tree.head_dim), dtype=odt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((tree.num_queries, tree.num_q_heads), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(plan, q.device)
    _check_tensors(tree, q, k_pool, v_pool, out, lse)
    _check(_lib.pst_decode_attn(plan._h, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)))
    return out, lse


def decode_attn_baseline(tree: Tree, q, k_pool, v_pool, *, cost=None, out=None, lse=None, want_lse=True, ws=None,
                         stream=None):
    """``pst_decode_attn_baseline`` (the FlashDecoding-style comparator: shared
    nodes read once per query): returns (out, lse) like :func:`decode_attn`.
    ``cost`` None selects the fitted table shipped for the tree's head layout."""
    import torch

    if cost is None:
        cost = default_cost_model(tree.head_dim, tree.num_q_heads, tree.num_kv_heads, tree.in_dtype)
    ch = cost._h if cost is not None else None
    if out is None:
        odt = torch.float32 if tree.out_dtype == PST_F32 else torch.bfloat16
        out = torch.empty((tree.num_queries, tree.num_q_heads, tree.head_dim), dtype=odt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((tree.num_queries, tree.num_q_heads), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(baseline_workspace_bytes(tree, cost, stream), 256), dtype=torch.uint8, device=q.device)
    _check_tensors(tree, q, k_pool, v_pool, out, lse)
    _check(_lib.pst_decode_attn_baseline(tree._h, ch, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse),
                                         _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out, lse


def decode_attn_noalloc(plan: Plan, q, k_pool, v_pool, *, out, lse=None, stream=None):
    """``pst_decode_attn_noalloc``: the hot path with the partial outputs in
    the library's per-device scratch array instead of a workspace.  The C
    call allocates nothing; the caller passes the outputs."""
    _check_tensors(plan.tree, q, k_pool, v_pool, out, lse)
    _check(_lib.pst_decode_attn_noalloc(plan._h, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse),
                                        _stream(stream)))
    return out, lse


def write_kv_rows(tree: Tree, k_new, v_new, rows, k_pool, v_pool, stream=None):
    """``pst_write_kv_rows``: new K/V rows ``k_new``, ``v_new`` [n, H_kv, d]
    into pool tokens ``rows`` (int64 [n] on the GPU) of every kv head."""
    import torch

    idt = torch.float32 if tree.in_dtype == PST_F32 else torch.bfloat16
    n = int(rows.numel())
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _check_one(name, t, idt)
        if t.numel() != n * tree.num_kv_heads * tree.head_dim:
            raise ValueError(f"{name} must hold [n, num_kv_heads, head_dim] = [{n}, {tree.num_kv_heads}, "
                             f"{tree.head_dim}] elements")
    _check_one("k_pool", k_pool, idt)
    _check_one("v_pool", v_pool, idt)
    if rows.dtype != torch.int64 or rows.device.type != "cuda" or not rows.is_contiguous():
        raise ValueError("rows must be a contiguous int64 GPU tensor")
    if k_pool.numel() < tree.kv_extent or v_pool.numel() < tree.kv_extent:
        raise ValueError(f"K/V pools hold fewer than the {tree.kv_extent} elements the tree's layout addresses")
    _check(_lib.pst_write_kv_rows(tree._h, _ptr(k_new), _ptr(v_new), _ptr(rows), n, _ptr(k_pool), _ptr(v_pool),
                                  _stream(stream)))


def baseline_workspace_bytes(tree: Tree, cost=None, stream=None) -> int:
    """``pst_baseline_workspace_size`` (makes the tree's query-guided plan if needed)."""
    n = C.c_size_t()
    _check(_lib.pst_baseline_workspace_size(tree._h, cost._h if cost is not None else None, _stream(stream),
                                            C.byref(n)))
    return n.value


def _check_inputs(tree, q, k_pool, v_pool):
    """q and the K/V pools against the tree's shape (see :func:`_check_tensors`)."""
    import torch

    idt = torch.float32 if tree.in_dtype == PST_F32 else torch.bfloat16
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _check_one(name, t, idt)
    if q.numel() < tree.num_queries * tree.num_q_heads * tree.head_dim:
        raise ValueError("q smaller than [num_queries, num_q_heads, head_dim]")
    need = tree.kv_extent
    if k_pool.numel() < need or v_pool.numel() < need:
        raise ValueError(f"K/V pools hold fewer than the {need} elements the tree's layout addresses")


def _check_outputs(tree, out, lse):
    import torch

    odt = torch.float32 if tree.out_dtype == PST_F32 else torch.bfloat16
    _check_one("out", out, odt)
    if out.numel() < tree.num_queries * tree.num_q_heads * tree.head_dim:
        raise ValueError("out smaller than [num_queries, num_q_heads, head_dim]")
    if lse is not None and (lse.dtype != torch.float32 or lse.numel() < tree.num_queries * tree.num_q_heads
                            or not lse.is_contiguous() or lse.device.type != "cuda"):
        raise ValueError("lse must be a contiguous float32 GPU tensor with num_queries * num_q_heads elements")


def _check_ws(plan, ws):
    if ws is None or ws.device.type != "cuda" or ws.numel() * ws.element_size() < plan.workspace_bytes:
        raise ValueError(f"the workspace must be a GPU tensor of at least {plan.workspace_bytes} bytes")


def pac(plan: Plan, q, k_pool, v_pool, ws, stream=None):
    _check_inputs(plan.tree, q, k_pool, v_pool)
    _check_ws(plan, ws)
    _check(_lib.pst_pac(plan._h, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(ws), ws.numel() * ws.element_size(),
                        _stream(stream)))


def por(plan: Plan, out, lse, ws, stream=None):
    _check_outputs(plan.tree, out, lse)
    _check_ws(plan, ws)
    _check(_lib.pst_por(plan._h, _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def _init_device():
    """Let torch initialise its HIP state before the library makes its first device call."""
    if _torch is not None and _torch.cuda.is_available():
        _torch.cuda.init()


def device_info():
    _init_device()
    cu, per = C.c_int32(), C.c_int32()
    _check(_lib.pst_device_info(C.byref(cu), C.byref(per)))
    return cu.value, per.value


def bench_flush(buf, stream=None):
    _check(_lib.pst_bench_flush(_ptr(buf), buf.numel() * buf.element_size(), _stream(stream)))


def bench_read(buf, sink, stream=None):
    _check(_lib.pst_bench_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))
