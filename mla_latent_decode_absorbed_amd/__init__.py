"""Python binding of libmla_decode.so: absorbed-MQA MLA decode + LSE merge on gfx950.

Argument marshalling only.  Every step of the decode (planning, paged KV
streaming, both contractions, the online softmax, the split combine and the
shard merge) runs in the library's HIP kernels; PyTorch supplies device memory
and the current stream.  The entry points mirror include/mla_decode.h:

    workspace_size(desc) -> int
    decode_partial(desc, q, kv_cache, kv_scale, block_table, seq_lens, scale,
                   out, lse, workspace, stream=None)
    decode_partial_noalloc(desc, q, kv_cache, kv_scale, block_table, seq_lens, scale,
                           out, lse, stream=None)
    merge_states(outs, lses, n, rows, out, lse, out_dtype=F32, stream=None)
    query_prep(q_nope, q_pe, w_uk, q_out, q_scale=None, stream=None)
    up_project(o_lat, w_uv, out, stream=None)
    merge_up_project(outs, lses, n, w_uv, out, lse=None, stream=None)
    gather_cache(kv_cache, block_table, seq_starts, cu_lens, total_rows, out, kv_scale=None, stream=None)
    merge_two_states(prefix_out, prefix_lse, suffix_out, suffix_lse, out, lse=None, stream=None)

plus ``Decoder``, which owns a workspace and allocates outputs.

Importing this package loads the shared library and raises if it is missing
or unloadable: there is no fallback implementation.

PyTorch is imported before the library is loaded.  PyTorch ships its own HIP
runtime with the same soname (libamdhip64.so.7) as the system one the library
is linked against; whichever is loaded first serves the whole process.  Loading
PyTorch's first makes the library run on the runtime that owns the tensors
and streams it is handed (the other order makes kernel launches fail).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the library load, see above)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_decode.so")

BF16, FP8_E4M3, F32 = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH_LIMIT = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 128 << 20
LATENT_DIM, ROPE_DIM, QK_DIM, PAGE_SIZE = 512, 64, 576, 64

#: every symbol include/mla_decode.h declares
EXPORTS = (
    "mla_decode_workspace_size",
    "mla_decode_partial",
    "mla_decode_partial_timed",
    "mla_decode_plan",
    "mla_decode_partial_planned",
    "mla_decode_partial_noalloc",
    "mla_merge_states",
    "mla_query_prep",
    "mla_up_project",
    "mla_merge_up_project",
    "mla_gather_cache",
    "mla_merge_two_states",
    "mla_status_string",
)


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class DecodeDesc(ctypes.Structure):
    """mla_decode_desc of include/mla_decode.h."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
    ]

    def __repr__(self):
        return "DecodeDesc(" + ", ".join(f"{k}={getattr(self, k)}" for k, _ in self._fields_) + ")"


class QueryPrepDesc(ctypes.Structure):
    """mla_query_prep_desc of include/mla_decode.h."""
    _fields_ = [
        ("rows", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("nope_dim", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
    ]


class UpProjectDesc(ctypes.Structure):
    """mla_up_project_desc of include/mla_decode.h."""
    _fields_ = [
        ("rows", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("v_head_dim", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python mla_latent_decode_absorbed_amd/build.py` "
                          "or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    pdesc = ctypes.POINTER(DecodeDesc)
    lib.mla_decode_workspace_size.argtypes = [pdesc, ctypes.POINTER(sz)]
    lib.mla_decode_workspace_size.restype = ctypes.c_int
    dec_args = [pdesc, vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.mla_decode_partial.argtypes = dec_args
    lib.mla_decode_partial.restype = ctypes.c_int
    lib.mla_decode_partial_timed.argtypes = dec_args + [vp, vp]
    lib.mla_decode_partial_timed.restype = ctypes.c_int
    lib.mla_decode_plan.argtypes = [pdesc, vp, vp, sz, vp]
    lib.mla_decode_plan.restype = ctypes.c_int
    lib.mla_decode_partial_planned.argtypes = dec_args
    lib.mla_decode_partial_planned.restype = ctypes.c_int
    lib.mla_decode_partial_noalloc.argtypes = [pdesc, vp, vp, vp, vp, vp, f32, vp, vp, vp]
    lib.mla_decode_partial_noalloc.restype = ctypes.c_int
    lib.mla_merge_states.argtypes = [vp, vp, i32, i32, vp, vp, i32, vp]
    lib.mla_merge_states.restype = ctypes.c_int
    lib.mla_query_prep.argtypes = [ctypes.POINTER(QueryPrepDesc), vp, vp, vp, vp, vp, vp]
    lib.mla_query_prep.restype = ctypes.c_int
    lib.mla_up_project.argtypes = [ctypes.POINTER(UpProjectDesc), vp, vp, vp, vp]
    lib.mla_up_project.restype = ctypes.c_int
    lib.mla_merge_up_project.argtypes = [vp, vp, i32, ctypes.POINTER(UpProjectDesc), vp, vp, vp, vp]
    lib.mla_merge_up_project.restype = ctypes.c_int
    lib.mla_gather_cache.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp, ctypes.c_int64, vp, vp]
    lib.mla_gather_cache.restype = ctypes.c_int
    lib.mla_merge_two_states.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.mla_merge_two_states.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.mla_status_string(int(status)).decode()


def _ptr(x) -> int | None:
    """Device address of a tensor (or a raw int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(batch, q_len, num_heads, num_pages, max_pages_per_seq, kv_dtype=BF16,
              out_dtype=F32, causal=None, num_splits=0, page_size=PAGE_SIZE) -> DecodeDesc:
    if causal is None:
        causal = 1 if q_len > 1 else 0
    return DecodeDesc(int(batch), int(q_len), int(num_heads), int(page_size), int(num_pages),
                      int(max_pages_per_seq), int(kv_dtype), int(out_dtype), int(causal),
                      int(num_splits))


def workspace_size(desc: DecodeDesc) -> int:
    n = ctypes.c_size_t(0)
    st = lib.mla_decode_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != OK:
        raise MlaError(st, "mla_decode_workspace_size")
    return n.value


def _nbytes(x) -> int | None:
    """Bytes of a tensor argument (None for a raw address, which cannot be checked)."""
    if x is None or isinstance(x, int):
        return None
    return x.numel() * x.element_size()


def _need(name: str, x, nbytes: int, itemsize: int | None = None) -> None:
    if x is None or isinstance(x, int):
        return
    if itemsize is not None and x.element_size() != itemsize:
        raise ValueError(f"{name}: element size {x.element_size()}, expected {itemsize}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _nbytes(x) < nbytes:
        raise ValueError(f"{name}: {_nbytes(x)} bytes, the descriptor needs {nbytes}")


def check_decode_buffers(desc: DecodeDesc, q, kv_cache, kv_scale, block_table, seq_lens, out, lse) -> None:
    """Host-side check of tensor arguments against the descriptor (sizes and
    element sizes; raw integer addresses are not checked).  The C ABI takes
    plain pointers and cannot see a buffer's size, so a too-small buffer would
    otherwise be read or written out of bounds on the device."""
    e = 2 if desc.kv_dtype == BF16 else 1
    rows = desc.batch * desc.q_len * desc.num_heads
    _need("q", q, rows * QK_DIM * e, e)
    _need("kv_cache", kv_cache, desc.num_pages * desc.page_size * QK_DIM * e, e)
    _need("block_table", block_table, desc.batch * desc.max_pages_per_seq * 4, 4)
    _need("seq_lens", seq_lens, desc.batch * 4, 4)
    _need("out", out, rows * LATENT_DIM * (4 if desc.out_dtype == F32 else 2), 4 if desc.out_dtype == F32 else 2)
    _need("lse", lse, rows * 4, 4)
    if desc.kv_dtype == FP8_E4M3:
        if kv_scale is None:
            raise ValueError("kv_scale is required for an fp8 cache")
        _need("kv_scale", kv_scale, 4, 4)
    elif kv_scale is not None:
        raise ValueError("kv_scale must be None for a bf16 cache")


def decode_partial(desc: DecodeDesc, q, kv_cache, kv_scale, block_table, seq_lens, scale: float,
                   out, lse, workspace, workspace_bytes: int | None = None, stream=None,
                   events=None) -> None:
    """Enqueue mla_decode_partial on ``stream`` (default: torch's current stream).
    Tensor arguments are checked against the descriptor first (ValueError)."""
    check_decode_buffers(desc, q, kv_cache, kv_scale, block_table, seq_lens, out, lse)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    args = [ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(kv_scale), _ptr(block_table),
            _ptr(seq_lens), ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
            ctypes.c_size_t(workspace_bytes), _stream(stream)]
    if events is None:
        st = lib.mla_decode_partial(*args)
    else:
        st = lib.mla_decode_partial_timed(*args, events[0], events[1])
    if st != OK:
        raise MlaError(st, "mla_decode_partial")


def decode_plan(desc: DecodeDesc, seq_lens, workspace, workspace_bytes: int | None = None, stream=None) -> None:
    """Enqueue mla_decode_plan: the split plan of seq_lens into ``workspace``,
    for the decodes of every layer of one step (decode_partial_planned)."""
    if seq_lens.numel() != desc.batch or seq_lens.element_size() != 4:
        raise ValueError(f"seq_lens: expected {desc.batch} int32 values")
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib.mla_decode_plan(ctypes.byref(desc), _ptr(seq_lens), _ptr(workspace), ctypes.c_size_t(workspace_bytes),
                             _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_decode_plan")


def decode_partial_planned(desc: DecodeDesc, q, kv_cache, kv_scale, block_table, seq_lens, scale: float,
                           out, lse, workspace, workspace_bytes: int | None = None, stream=None) -> None:
    """Enqueue mla_decode_partial_planned: decode_partial following the plan an
    earlier decode_plan left in ``workspace`` (same descriptor and seq_lens)."""
    check_decode_buffers(desc, q, kv_cache, kv_scale, block_table, seq_lens, out, lse)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib.mla_decode_partial_planned(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(kv_scale),
                                        _ptr(block_table), _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
                                        _ptr(lse), _ptr(workspace), ctypes.c_size_t(workspace_bytes),
                                        _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_decode_partial_planned")


def decode_partial_noalloc(desc: DecodeDesc, q, kv_cache, kv_scale, block_table, seq_lens, scale: float,
                           out, lse, stream=None) -> None:
    """Enqueue mla_decode_partial_noalloc: decode_partial on the library's static
    device scratch (no workspace argument, no allocation).  Calls on one GPU
    share that scratch and must not overlap in time."""
    check_decode_buffers(desc, q, kv_cache, kv_scale, block_table, seq_lens, out, lse)
    st = lib.mla_decode_partial_noalloc(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(kv_scale),
                                        _ptr(block_table), _ptr(seq_lens), ctypes.c_float(scale), _ptr(out),
                                        _ptr(lse), _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_decode_partial_noalloc")


def merge_states(outs, lses, n: int, rows: int, out, lse, out_dtype: int = F32, stream=None) -> None:
    """Enqueue mla_merge_states: outs [n][rows][512] f32, lses [n][rows] -> out, lse.
    Tensor arguments are size-checked first (ValueError)."""
    _need("outs", outs, n * rows * LATENT_DIM * 4, 4)
    _need("lses", lses, n * rows * 4, 4)
    _need("out", out, rows * LATENT_DIM * (4 if out_dtype == F32 else 2), 4 if out_dtype == F32 else 2)
    _need("lse", lse, rows * 4, 4)
    st = lib.mla_merge_states(_ptr(outs), _ptr(lses), int(n), int(rows), _ptr(out), _ptr(lse),
                              int(out_dtype), _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_merge_states")


def query_prep(q_nope, q_pe, w_uk, q_out, q_scale=None, stream=None) -> None:
    """Enqueue mla_query_prep: q_nope [R][H][P] bf16, q_pe [R][H][64] bf16,
    w_uk [H][512][P] bf16 (latent-major W_UK_T) -> q_out [R][H][576], bf16 when
    q_scale is None, else e4m3 codes of value / q_scale (q_scale: a device
    float).  Shapes and element sizes are checked first (ValueError)."""
    if q_nope.dim() != 3 or q_pe.dim() != 3 or w_uk.dim() != 3:
        raise ValueError("q_nope, q_pe and w_uk must be 3-d")
    R, H, P = q_nope.shape
    if tuple(q_pe.shape) != (R, H, ROPE_DIM) or tuple(w_uk.shape) != (H, LATENT_DIM, P):
        raise ValueError(f"shapes {tuple(q_pe.shape)}, {tuple(w_uk.shape)} do not match q_nope {tuple(q_nope.shape)}")
    fp8 = q_scale is not None
    for name, x in (("q_nope", q_nope), ("q_pe", q_pe), ("w_uk", w_uk)):
        _need(name, x, x.numel() * 2, 2)
    _need("q_out", q_out, R * H * QK_DIM * (1 if fp8 else 2), 1 if fp8 else 2)
    if fp8:
        _need("q_scale", q_scale, 4, 4)
    desc = QueryPrepDesc(int(R), int(H), int(P), FP8_E4M3 if fp8 else BF16)
    st = lib.mla_query_prep(ctypes.byref(desc), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(q_scale),
                            _ptr(q_out), _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_query_prep")


def up_project(o_lat, w_uv, out, stream=None) -> None:
    """Enqueue mla_up_project: o_lat [R][H][512] (fp32 or bf16), w_uv [H][Vd][512]
    bf16 -> out [R][H][Vd] (fp32 or bf16, by the tensor's element size).
    Shapes and element sizes are checked first (ValueError)."""
    if o_lat.dim() != 3 or w_uv.dim() != 3:
        raise ValueError("o_lat and w_uv must be 3-d")
    R, H, L = o_lat.shape
    Vd = w_uv.shape[1]
    if L != LATENT_DIM or tuple(w_uv.shape) != (H, Vd, LATENT_DIM):
        raise ValueError(f"shapes {tuple(o_lat.shape)}, {tuple(w_uv.shape)} do not match")
    if o_lat.element_size() not in (2, 4) or out.element_size() not in (2, 4):
        raise ValueError("o_lat and out must be fp32 or bf16")
    _need("o_lat", o_lat, R * H * LATENT_DIM * o_lat.element_size())
    _need("w_uv", w_uv, H * Vd * LATENT_DIM * 2, 2)
    _need("out", out, R * H * Vd * out.element_size())
    desc = UpProjectDesc(int(R), int(H), int(Vd), F32 if o_lat.element_size() == 4 else BF16,
                         F32 if out.element_size() == 4 else BF16)
    st = lib.mla_up_project(ctypes.byref(desc), _ptr(o_lat), _ptr(w_uv), _ptr(out), _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_up_project")


def merge_up_project(outs, lses, n: int, w_uv, out, lse=None, stream=None) -> None:
    """Enqueue mla_merge_up_project: n fp32 partials outs [n][R][H][512] with
    lses [n][R][H] -> out [R][H][Vd] (fp32 or bf16 by element size) through
    W_UV [H][Vd][512], and optionally the merged lse [R][H]."""
    if outs.dim() != 4 or outs.shape[0] != n or outs.shape[-1] != LATENT_DIM:
        raise ValueError(f"outs must be [n][R][H][512], got {tuple(outs.shape)}")
    _, R, H, _ = outs.shape
    Vd = w_uv.shape[1]
    if tuple(w_uv.shape) != (H, Vd, LATENT_DIM):
        raise ValueError(f"w_uv {tuple(w_uv.shape)} does not match {H} heads")
    _need("outs", outs, n * R * H * LATENT_DIM * 4, 4)
    _need("lses", lses, n * R * H * 4, 4)
    _need("w_uv", w_uv, H * Vd * LATENT_DIM * 2, 2)
    _need("out", out, R * H * Vd * out.element_size())
    if lse is not None:
        _need("lse", lse, R * H * 4, 4)
    desc = UpProjectDesc(int(R), int(H), int(Vd), F32, F32 if out.element_size() == 4 else BF16)
    st = lib.mla_merge_up_project(_ptr(outs), _ptr(lses), int(n), ctypes.byref(desc), _ptr(w_uv), _ptr(out),
                                  _ptr(lse), _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_merge_up_project")


def gather_cache(kv_cache, block_table, seq_starts, cu_lens, total_rows: int, out, kv_scale=None,
                 stream=None) -> None:
    """Enqueue mla_gather_cache: rows seq_starts[b] .. of each request's chunk
    (cu_lens [B + 1] output offsets) out of the paged cache [P][64][576]
    (bf16, or e4m3 codes with kv_scale) into out [total_rows][576] bf16."""
    if kv_cache.dim() != 3 or tuple(kv_cache.shape[1:]) != (PAGE_SIZE, QK_DIM):
        raise ValueError(f"kv_cache must be [pages][64][576], got {tuple(kv_cache.shape)}")
    fp8 = kv_cache.element_size() == 1
    if fp8 != (kv_scale is not None):
        raise ValueError("kv_scale is required for an e4m3 cache and must be None for bf16")
    B, maxp = block_table.shape
    _need("block_table", block_table, B * maxp * 4, 4)
    _need("seq_starts", seq_starts, B * 4, 4)
    _need("cu_lens", cu_lens, (B + 1) * 4, 4)
    _need("out", out, int(total_rows) * QK_DIM * 2, 2)
    if kv_scale is not None:
        _need("kv_scale", kv_scale, 4, 4)
    st = lib.mla_gather_cache(_ptr(kv_cache), FP8_E4M3 if fp8 else BF16, _ptr(kv_scale), _ptr(block_table),
                              int(B), int(kv_cache.shape[0]), int(maxp), _ptr(seq_starts), _ptr(cu_lens),
                              ctypes.c_int64(int(total_rows)), _ptr(out), _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_gather_cache")


def merge_two_states(prefix_out, prefix_lse, suffix_out, suffix_lse, out, lse=None, stream=None) -> None:
    """Enqueue mla_merge_two_states: [rows][head_dim] prefix and suffix partials
    (fp32 or bf16) and their LSEs -> out (fp32 or bf16) and optionally lse."""
    rows, hd = prefix_out.shape[0], prefix_out.shape[-1]
    if prefix_out.numel() != rows * hd or tuple(suffix_out.shape) != tuple(prefix_out.shape):
        raise ValueError("prefix and suffix outputs must both be [rows][head_dim]")
    if prefix_out.dtype != suffix_out.dtype or prefix_out.element_size() not in (2, 4):
        raise ValueError("prefix and suffix outputs must share an fp32 or bf16 dtype")
    for name, x in (("prefix_lse", prefix_lse), ("suffix_lse", suffix_lse)) + ((("lse", lse),) if lse is not None else ()):
        _need(name, x, rows * 4, 4)
    _need("prefix_out", prefix_out, rows * hd * prefix_out.element_size())
    _need("suffix_out", suffix_out, rows * hd * suffix_out.element_size())
    _need("out", out, rows * hd * out.element_size())
    st = lib.mla_merge_two_states(int(rows), int(hd), F32 if prefix_out.element_size() == 4 else BF16,
                                  F32 if out.element_size() == 4 else BF16, _ptr(prefix_out), _ptr(prefix_lse),
                                  _ptr(suffix_out), _ptr(suffix_lse), _ptr(out), _ptr(lse), _stream(stream))
    if st != OK:
        raise MlaError(st, "mla_merge_two_states")


class Decoder:
    """Owns the workspace for one descriptor and allocates outputs (torch tensors)."""

    def __init__(self, desc: DecodeDesc, device="cuda"):
        import torch
        self.desc = desc
        self.ws_bytes = workspace_size(desc)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)

    def __call__(self, q, kv_cache, block_table, seq_lens, scale: float, kv_scale=None,
                 out=None, lse=None, stream=None, events=None):
        import torch
        d = self.desc
        rows = d.q_len * d.num_heads
        if out is None:
            dt = torch.float32 if d.out_dtype == F32 else torch.bfloat16
            out = torch.empty((d.batch, d.q_len, d.num_heads, LATENT_DIM), dtype=dt, device=q.device)
        if lse is None:
            lse = torch.empty((d.batch, d.q_len, d.num_heads), dtype=torch.float32, device=q.device)
        assert out.numel() == d.batch * rows * LATENT_DIM and lse.numel() == d.batch * rows
        decode_partial(d, q, kv_cache, kv_scale, block_table, seq_lens, scale, out, lse,
                       self.workspace, self.ws_bytes, stream=stream, events=events)
        return out, lse

    def plan(self, seq_lens, stream=None) -> None:
        """Plan the splits of one step once (mla_decode_plan); then call
        ``planned`` for each layer's decode with the same seq_lens."""
        decode_plan(self.desc, seq_lens, self.workspace, self.ws_bytes, stream=stream)

    def planned(self, q, kv_cache, block_table, seq_lens, scale: float, kv_scale=None, out=None, lse=None,
                stream=None):
        """One layer's decode on the plan of the last ``plan`` call."""
        import torch
        d = self.desc
        if out is None:
            dt = torch.float32 if d.out_dtype == F32 else torch.bfloat16
            out = torch.empty((d.batch, d.q_len, d.num_heads, LATENT_DIM), dtype=dt, device=q.device)
        if lse is None:
            lse = torch.empty((d.batch, d.q_len, d.num_heads), dtype=torch.float32, device=q.device)
        decode_partial_planned(d, q, kv_cache, kv_scale, block_table, seq_lens, scale, out, lse,
                               self.workspace, self.ws_bytes, stream=stream)
        return out, lse
