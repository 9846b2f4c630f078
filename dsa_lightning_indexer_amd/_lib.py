"""ctypes view of include/dsa.h."""
import ctypes
import os

# torch ships its own HIP runtime (SONAME libamdhip64.so.7).  Load it before
# libdsa.so so that the library's NEEDED entry resolves to that same copy: a
# process must not hold two HIP/HSA runtimes.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python dsa_lightning_indexer_amd/build.py` "
        "(there is no fallback implementation)")

LIB = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}


class IndexerArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", c_i32), ("batch", c_i32), ("n_q", c_i32), ("n_k", c_i32), ("heads", c_i32),
        ("dim", c_i32), ("q_pos0", c_i64), ("q", c_vp), ("q_scale", c_vp), ("k", c_vp),
        ("k_batch_stride", c_i64), ("k_scale", c_vp), ("k_scale_batch_stride", c_i64), ("w", c_vp),
    ]


class SparseAttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", c_i32), ("batch", c_i32), ("n_q", c_i32), ("n_k", c_i32), ("heads", c_i32),
        ("kv_heads", c_i32), ("d_qk", c_i32), ("d_v", c_i32), ("topk", c_i32), ("q", c_vp),
        ("kv", c_vp), ("kv_batch_stride", c_i64), ("v", c_vp), ("v_batch_stride", c_i64),
        ("idx", c_vp), ("scale", c_f32), ("out", c_vp),
    ]


class Layer(ctypes.Structure):
    _fields_ = [("ix", IndexerArgs), ("sa", SparseAttnArgs), ("idx_out", c_vp)]


class DistillArgs(ctypes.Structure):
    _fields_ = [("ix", IndexerArgs), ("topk", c_i32), ("n_teachers", c_i32), ("idx", c_vp), ("teachers", c_vp),
                ("loss", c_vp), ("delta", c_vp), ("dq", c_vp), ("dw", c_vp), ("dk", c_vp)]


def _sig(name, res, *args):
    f = getattr(LIB, name)
    f.restype = res
    f.argtypes = list(args)
    return f


P_IX, P_SA, P_LAYER = ctypes.POINTER(IndexerArgs), ctypes.POINTER(SparseAttnArgs), ctypes.POINTER(Layer)
dsa_abi_version = _sig("dsa_abi_version", c_i32)
dsa_status_string = _sig("dsa_status_string", ctypes.c_char_p, c_i32)
dsa_last_error = _sig("dsa_last_error", ctypes.c_char_p)
dsa_indexer_scores = _sig("dsa_indexer_scores", c_i32, P_IX, c_i64, c_i64, c_vp, c_vp)
dsa_topk_workspace_size = _sig("dsa_topk_workspace_size", c_sz, P_IX, c_vp, c_i32)
dsa_topk = _sig("dsa_topk", c_i32, P_IX, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp)
dsa_sparse_attn_workspace_size = _sig("dsa_sparse_attn_workspace_size", c_sz, P_SA)
dsa_sparse_attn = _sig("dsa_sparse_attn", c_i32, P_SA, c_vp, c_sz, c_vp)
indexcache_forward_workspace_size = _sig("indexcache_forward_workspace_size", c_sz, ctypes.c_char_p, c_i32,
                                         P_LAYER, c_i32)
indexcache_forward_c = _sig("indexcache_forward", c_i32, ctypes.c_char_p, c_i32, P_LAYER, c_i32,
                            ctypes.POINTER(c_i32), c_vp, c_sz, c_vp)
indexcache_forward_mli_workspace_size = _sig("indexcache_forward_mli_workspace_size", c_sz, ctypes.c_char_p, c_i32,
                                             P_LAYER, c_i32)
indexcache_forward_mli_c = _sig("indexcache_forward_mli", c_i32, ctypes.c_char_p, c_i32, P_LAYER, c_i32,
                                ctypes.POINTER(c_i32), c_vp, c_sz, c_vp, c_vp)
indexcache_forward_noalloc_c = _sig("indexcache_forward_noalloc", c_i32, ctypes.c_char_p, c_i32, P_LAYER, c_i32,
                                   ctypes.POINTER(c_i32), c_vp)
NOALLOC_SCRATCH_BYTES = 64 << 20      # DSA_NOALLOC_SCRATCH_BYTES
dsa_gather_probe_out_words = _sig("dsa_gather_probe_out_words", c_i64, c_i64, c_i32)
dsa_gather_probe = _sig("dsa_gather_probe", c_i32, c_vp, c_i32, c_vp, c_i64, c_i32, c_i32, c_vp, c_vp)
dsa_stream_probe = _sig("dsa_stream_probe", c_i32, c_vp, c_i64, c_i32, c_i32, c_vp, c_vp)
dsa_index_overlap = _sig("dsa_index_overlap", c_i32, c_vp, c_vp, c_i64, c_i32, c_vp, c_vp, c_vp)
dsa_indexer_distill = _sig("dsa_indexer_distill", c_i32, ctypes.POINTER(DistillArgs), c_vp)
dsa_row_cosine = _sig("dsa_row_cosine", c_i32, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp)
dsa_similarity_matrix_workspace_size = _sig("dsa_similarity_matrix_workspace_size", c_sz, c_i32, P_LAYER, c_i32)
dsa_similarity_matrix = _sig("dsa_similarity_matrix", c_i32, c_i32, P_LAYER, c_i32, c_vp, c_vp, c_sz, c_vp)
dsa_pattern_search = _sig("dsa_pattern_search", c_i32, ctypes.POINTER(ctypes.c_double), c_i32, c_i32,
                          ctypes.c_char_p, ctypes.POINTER(ctypes.c_double))

EXPORTS = ["dsa_abi_version", "dsa_status_string", "dsa_last_error", "dsa_indexer_scores",
           "dsa_topk_workspace_size", "dsa_topk", "dsa_sparse_attn_workspace_size", "dsa_sparse_attn",
           "indexcache_forward_workspace_size", "indexcache_forward", "indexcache_forward_mli_workspace_size",
           "indexcache_forward_mli", "indexcache_forward_noalloc", "dsa_index_overlap",
           "dsa_indexer_distill", "dsa_row_cosine", "dsa_similarity_matrix_workspace_size",
           "dsa_similarity_matrix", "dsa_pattern_search", "dsa_gather_probe_out_words", "dsa_gather_probe",
           "dsa_stream_probe"]


class DsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def check(status):
    if status != 0:
        raise DsaError(status, dsa_last_error().decode(errors="replace"))


def abi_version():
    return dsa_abi_version()


def dtype_code(t):
    import torch
    m = {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16, torch.float8_e4m3fn: DSA_FP8_E4M3}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dense(name, t):
    """The kernels read these tensors as dense row-major arrays."""
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (got strides {tuple(t.stride())} for shape {tuple(t.shape)})")


def _rows(name, t, row):
    """Tensors passed with a batch stride: every dimension after the batch one must
    be dense (rows of `row` elements back to back); the batch stride is free."""
    if t is None:
        return
    expect = 1
    for dim in range(t.dim() - 1, 0, -1):
        if t.shape[dim] != 1 and t.stride(dim) != expect:
            raise ValueError(f"{name} must be dense after its batch dimension (rows of {row} elements); "
                             f"got strides {tuple(t.stride())} for shape {tuple(t.shape)}")
        expect *= t.shape[dim]


def indexer_args(q, k, w, q_scale=None, k_scale=None, q_pos0=0):
    """q [B, n_q, H, d], k [B, n_k, d] (rows dense, any batch stride), w [B, n_q, H] fp32."""
    B, n_q, H, d = q.shape
    for name, t in (("q", q), ("w", w), ("q_scale", q_scale)):
        _dense(name, t)
    _rows("k", k, d)
    _rows("k_scale", k_scale, 1)
    a = IndexerArgs()
    a.dtype = dtype_code(q)
    a.batch, a.n_q, a.n_k, a.heads, a.dim = B, n_q, k.shape[1], H, d
    a.q_pos0 = int(q_pos0)
    a.q, a.q_scale, a.k, a.k_scale, a.w = _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w)
    a.k_batch_stride = k.stride(0) if B > 1 else 0
    a.k_scale_batch_stride = (k_scale.stride(0) if (k_scale is not None and B > 1) else 0)
    return a


def sparse_attn_args(q, kv, idx, scale, out, v=None, d_v=None):
    """q [B, n_q, H, d_qk], kv [B, n_k, G, d_qk], idx [B, n_q, topk] int32, out [B, n_q, H, d_v]."""
    B, n_q, H, d_qk = q.shape
    for name, t in (("q", q), ("idx", idx)):
        _dense(name, t)
    if out is not None and out.numel() > 0:
        _dense("out", out)
    _rows("kv", kv, d_qk)
    _rows("v", v, None if v is None else v.shape[-1])
    a = SparseAttnArgs()
    a.dtype = dtype_code(q)
    a.batch, a.n_q, a.n_k, a.heads, a.kv_heads, a.d_qk = B, n_q, kv.shape[1], H, kv.shape[2], d_qk
    a.d_v = int(out.shape[-1] if d_v is None else d_v)
    a.topk = 0 if idx is None else idx.shape[-1]
    a.q, a.kv, a.v, a.idx, a.out = _ptr(q), _ptr(kv), _ptr(v), _ptr(idx), _ptr(out)
    a.kv_batch_stride = kv.stride(0) if B > 1 else 0
    a.v_batch_stride = (v.stride(0) if (v is not None and B > 1) else 0)
    a.scale = float(scale)
    return a
