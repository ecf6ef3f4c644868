"""Python binding of libgdn.so: argument marshalling only.

Each function fills the C argument struct declared in ``include/gdn.h`` from
torch tensors (device pointers, dtype codes, sizes) and calls the entry point of
the same name on the current HIP stream.  Every step of the computation runs in
the library's kernels; nothing here computes, and there is no fallback: if the
library is missing, importing this module raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the same library (an instrumented host
# build, say); by default the in-tree libgdn.so is loaded.
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_PKG, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = range(5)
GDN_DTYPE_F32, GDN_DTYPE_BF16, GDN_DTYPE_F16 = 0, 1, 2
GDN_GATES_DIRECT, GDN_GATES_RAW = 0, 1
GDN_NORM_GATE_SILU, GDN_NORM_GATE_SIGMOID = 0, 1
VERIFY_WY_TABLE_SEQS = 128
VERIFY_WY_TABLES_PER_LAYER = 16
PREFILL_CHUNK = 64
DECODE_MAX_TOKENS = 17

if not os.path.exists(LIB_PATH):
    raise ImportError("%s is not built (run `python -m linear_attention_ssm_core_amd.build`); "
                      "there is no fallback path" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class gdn_dims(ctypes.Structure):
    _fields_ = [("num_k_heads", _i32), ("num_v_heads", _i32), ("head_dim_k", _i32),
                ("head_dim_v", _i32), ("conv_kernel", _i32), ("reserved", _i32)]


class gdn_options(ctypes.Structure):
    _fields_ = [("state_dtype", _i32), ("gate_mode", _i32), ("norm_gate", _i32), ("reserved", _i32)]


class gdn_conv_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("act_dtype", _i32), ("out_dtype", _i32),
                ("dims", gdn_dims), ("num_seqs", _i32), ("total_tokens", ctypes.c_int64),
                ("cu_seqlens", _vp), ("x", _vp), ("conv_w", _vp), ("conv_state", _vp), ("y", _vp),
                ("l2_eps", ctypes.c_float)]


class gdn_prefill_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("act_dtype", _i32), ("out_dtype", _i32),
                ("dims", gdn_dims), ("num_seqs", _i32), ("total_tokens", ctypes.c_int64),
                ("chunk_size", _i32), ("reserved", _i32), ("cu_seqlens", _vp), ("y", _vp), ("x", _vp),
                ("conv_w", _vp), ("conv_state", _vp), ("a", _vp), ("b", _vp), ("h_state", _vp),
                ("z", _vp), ("norm_w", _vp), ("out", _vp), ("scale", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float), ("reserved_f", ctypes.c_float),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t), ("opt", gdn_options)]


class gdn_decode_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("act_dtype", _i32), ("out_dtype", _i32),
                ("dims", gdn_dims), ("num_seqs", _i32), ("x", _vp), ("conv_w", _vp), ("conv_state", _vp),
                ("a", _vp), ("b", _vp), ("h_state", _vp), ("z", _vp), ("norm_w", _vp), ("out", _vp),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("reserved_f", ctypes.c_float), ("opt", gdn_options)]


class gdn_verify_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("act_dtype", _i32), ("out_dtype", _i32),
                ("dims", gdn_dims), ("num_seqs", _i32), ("max_k", _i32), ("total_rows", _i32),
                ("reserved", _i32), ("cu_ks", _vp), ("x", _vp), ("conv_w", _vp), ("conv_state", _vp),
                ("a", _vp), ("b", _vp), ("wy_tables", _vp), ("z", _vp), ("norm_w", _vp), ("out", _vp),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("reserved_f", ctypes.c_float), ("opt", gdn_options)]


class gdn_commit_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("act_dtype", _i32), ("dims", gdn_dims),
                ("num_seqs", _i32), ("reserved", _i32), ("cu_ks", _vp), ("n_accepted", _vp),
                ("wy_tables", _vp), ("x", _vp), ("conv_state", _vp), ("opt", gdn_options)]


class gdn_norm_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("in_dtype", _i32), ("act_dtype", _i32),
                ("out_dtype", _i32), ("dims", gdn_dims), ("total_tokens", ctypes.c_int64), ("o", _vp),
                ("z", _vp), ("norm_w", _vp), ("out", _vp), ("eps", ctypes.c_float),
                ("reserved_f", ctypes.c_float), ("opt", gdn_options)]


class gdn_woa_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("act_dtype", _i32), ("out_dtype", _i32),
                ("dims", gdn_dims), ("num_seqs", _i32), ("max_k", _i32), ("total_rows", _i32),
                ("reserved", _i32), ("cu_ks", _vp), ("x", _vp), ("conv_w", _vp), ("conv_state", _vp),
                ("a", _vp), ("b", _vp), ("h_state", _vp), ("z", _vp), ("norm_w", _vp), ("out", _vp),
                ("stash", _vp), ("stash_bytes", ctypes.c_size_t), ("scale", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float), ("reserved_f", ctypes.c_float),
                ("opt", gdn_options)]


class gdn_fold_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("act_dtype", _i32), ("dims", gdn_dims),
                ("num_seqs", _i32), ("total_rows", _i32), ("cu_ks", _vp), ("n_accepted", _vp),
                ("h_state", _vp), ("stash", _vp), ("stash_bytes", ctypes.c_size_t), ("x", _vp),
                ("conv_state", _vp), ("opt", gdn_options)]


class gdn_tokens_args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("act_dtype", _i32), ("out_dtype", _i32),
                ("dims", gdn_dims), ("num_seqs", _i32), ("max_tokens", _i32), ("total_rows", _i32),
                ("reserved", _i32), ("cu_tokens", _vp), ("x", _vp), ("conv_w", _vp), ("conv_state", _vp),
                ("a", _vp), ("b", _vp), ("h_state", _vp), ("z", _vp), ("norm_w", _vp), ("out", _vp),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("reserved_f", ctypes.c_float), ("opt", gdn_options)]


for _name, _st in [("gdn_conv_l2norm", gdn_conv_args), ("gdn_prefill_chunked", gdn_prefill_args),
                   ("gdn_prefill_chunked_noalloc", gdn_prefill_args),
                   ("gdn_decode_batched", gdn_decode_args), ("gdn_verify_multi", gdn_verify_args),
                   ("gdn_verify_commit", gdn_commit_args), ("gdn_gated_rmsnorm", gdn_norm_args),
                   ("gdn_verify_woa", gdn_woa_args), ("gdn_fold_accepted", gdn_fold_args),
                   ("gdn_decode_tokens", gdn_tokens_args)]:
    _f = getattr(_lib, _name)
    _f.argtypes = [ctypes.POINTER(_st), _vp]
    _f.restype = ctypes.c_int
_lib.gdn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(gdn_prefill_args), ctypes.POINTER(ctypes.c_size_t)]
_lib.gdn_prefill_workspace_bytes.restype = ctypes.c_int
_lib.gdn_woa_stash_bytes.argtypes = [ctypes.POINTER(gdn_woa_args), ctypes.POINTER(ctypes.c_size_t)]
_lib.gdn_woa_stash_bytes.restype = ctypes.c_int
_lib.gdn_status_string.argtypes = [ctypes.c_int]
_lib.gdn_status_string.restype = ctypes.c_char_p
_lib.gdn_abi_version.restype = _i32


class GdnError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(status_string(status))


def status_string(status):
    return _lib.gdn_status_string(int(status)).decode()


def abi_version():
    return int(_lib.gdn_abi_version())


def library():
    """The loaded ctypes handle of libgdn.so."""
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _dt(t):
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    raise TypeError("unsupported dtype %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libgdn must be contiguous")
    return t.data_ptr()


def _dims(d):
    return gdn_dims(d.Hk, d.Hv, d.dk, d.dv, d.K, 0)


def options(state=None, gates="direct", norm_gate="silu"):
    """gdn_options from readable names: ``state`` is a state tensor (its dtype
    decides: float32 or float16), a torch dtype, or None (fp32)."""
    if state is None:
        sd = GDN_DTYPE_F32
    else:
        dt = state.dtype if hasattr(state, "dtype") else state
        if dt == torch.float32:
            sd = GDN_DTYPE_F32
        elif dt == torch.float16:
            sd = GDN_DTYPE_F16
        else:
            raise TypeError("recurrent states are float32 or float16, not %s" % dt)
    gm = {"direct": GDN_GATES_DIRECT, "raw": GDN_GATES_RAW}[gates]
    ng = {"silu": GDN_NORM_GATE_SILU, "sigmoid": GDN_NORM_GATE_SIGMOID}[norm_gate]
    return gdn_options(sd, gm, ng, 0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status):
    if status != GDN_OK:
        raise GdnError(status)


def ptr_array(tensors, device=None):
    """Device int64 array of the data pointers of ``tensors`` (per-sequence state
    or conv-state pointer arrays)."""
    dev = device if device is not None else tensors[0].device
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=dev)


def wy_tables(state_ptrs_per_table, device):
    """[16][128] pointer table from a list of per-table lists of tensors (or
    None): ``state_ptrs_per_table[t][i]`` is sequence i's buffer in table t."""
    tab = torch.zeros((VERIFY_WY_TABLES_PER_LAYER, VERIFY_WY_TABLE_SEQS), dtype=torch.int64)
    for t, row in enumerate(state_ptrs_per_table):
        for i, ten in enumerate(row):
            if ten is not None:
                tab[t, i] = ten.data_ptr()
    return tab.to(device)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def gdn_conv_l2norm(x, conv_w, conv_state_ptrs, cu_seqlens, y, dims, *, l2_eps=1e-6, stream=None):
    args = gdn_conv_args(ctypes.sizeof(gdn_conv_args), _dt(x), _dt(y), _dims(dims),
                         cu_seqlens.numel() - 1, x.shape[0], _ptr(cu_seqlens), _ptr(x), _ptr(conv_w),
                         _ptr(conv_state_ptrs), _ptr(y), l2_eps)
    _check(_lib.gdn_conv_l2norm(ctypes.byref(args), _stream(stream)))


def _prefill_args(dims, cu_seqlens, a, b, h_state_ptrs, out, *, y=None, x=None, conv_w=None,
                  conv_state_ptrs=None, z=None, norm_w=None, scale=1.0, l2_eps=1e-6, norm_eps=1e-6,
                  workspace=None, opt=None):
    act = y if y is not None else x
    return gdn_prefill_args(ctypes.sizeof(gdn_prefill_args), _dt(act), _dt(out), _dims(dims),
                            cu_seqlens.numel() - 1, act.shape[0], PREFILL_CHUNK, 0, _ptr(cu_seqlens),
                            _ptr(y), _ptr(x), _ptr(conv_w), _ptr(conv_state_ptrs), _ptr(a), _ptr(b),
                            _ptr(h_state_ptrs), _ptr(z), _ptr(norm_w), _ptr(out), scale, l2_eps,
                            norm_eps, 0.0, _ptr(workspace),
                            0 if workspace is None else workspace.numel() * workspace.element_size(),
                            opt if opt is not None else gdn_options())


def gdn_prefill_workspace_bytes(dims, cu_seqlens, a, b, h_state_ptrs, out, **kw):
    args = _prefill_args(dims, cu_seqlens, a, b, h_state_ptrs, out, **kw)
    n = ctypes.c_size_t(0)
    _check(_lib.gdn_prefill_workspace_bytes(ctypes.byref(args), ctypes.byref(n)))
    return int(n.value)


def gdn_prefill_chunked(dims, cu_seqlens, a, b, h_state_ptrs, out, *, workspace=None, stream=None, **kw):
    """Chunked prefill.  Pass ``y`` (= [q_hat | k_hat | v] rows) or ``x`` with
    ``conv_w`` and ``conv_state_ptrs`` for the fused front; ``z``/``norm_w`` for
    the gated-norm epilogue; ``opt`` a ``gdn_options`` (see ``options``).
    ``workspace``: a uint8 device tensor of at least ``gdn_prefill_workspace_bytes``
    bytes (allocated here when None)."""
    if workspace is None:
        nbytes = gdn_prefill_workspace_bytes(dims, cu_seqlens, a, b, h_state_ptrs, out, **kw)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=out.device)
    args = _prefill_args(dims, cu_seqlens, a, b, h_state_ptrs, out, workspace=workspace, **kw)
    _check(_lib.gdn_prefill_chunked(ctypes.byref(args), _stream(stream)))
    return workspace


PREFILL_SCRATCH_BYTES = 64 << 20


def gdn_prefill_chunked_noalloc(dims, cu_seqlens, a, b, h_state_ptrs, out, *, stream=None, **kw):
    """gdn_prefill_chunked in the library's own per-GPU scratch array (no workspace,
    no allocation); the call's workspace need must fit PREFILL_SCRATCH_BYTES."""
    args = _prefill_args(dims, cu_seqlens, a, b, h_state_ptrs, out, **kw)
    _check(_lib.gdn_prefill_chunked_noalloc(ctypes.byref(args), _stream(stream)))


def _opt(opt):
    return opt if opt is not None else gdn_options()


def gdn_decode_batched(x, conv_w, conv_state_ptrs, a, b, h_state_ptrs, out, dims, *, z=None,
                       norm_w=None, scale=1.0, l2_eps=1e-6, norm_eps=1e-6, opt=None, stream=None):
    args = gdn_decode_args(ctypes.sizeof(gdn_decode_args), _dt(x), _dt(out), _dims(dims), x.shape[0],
                           _ptr(x), _ptr(conv_w), _ptr(conv_state_ptrs), _ptr(a), _ptr(b),
                           _ptr(h_state_ptrs), _ptr(z), _ptr(norm_w), _ptr(out), scale, l2_eps,
                           norm_eps, 0.0, _opt(opt))
    _check(_lib.gdn_decode_batched(ctypes.byref(args), _stream(stream)))


def gdn_verify_multi(x, conv_w, conv_state_ptrs, a, b, wy_table, cu_ks, max_k, out, dims, *, z=None,
                     norm_w=None, scale=1.0, l2_eps=1e-6, norm_eps=1e-6, opt=None, stream=None):
    args = gdn_verify_args(ctypes.sizeof(gdn_verify_args), _dt(x), _dt(out), _dims(dims),
                           cu_ks.numel() - 1, max_k, x.shape[0], 0, _ptr(cu_ks), _ptr(x), _ptr(conv_w),
                           _ptr(conv_state_ptrs), _ptr(a), _ptr(b), _ptr(wy_table), _ptr(z),
                           _ptr(norm_w), _ptr(out), scale, l2_eps, norm_eps, 0.0, _opt(opt))
    _check(_lib.gdn_verify_multi(ctypes.byref(args), _stream(stream)))


def gdn_verify_commit(x, conv_state_ptrs, wy_table, cu_ks, n_accepted, dims, *, opt=None, stream=None):
    args = gdn_commit_args(ctypes.sizeof(gdn_commit_args), _dt(x), _dims(dims), cu_ks.numel() - 1, 0,
                           _ptr(cu_ks), _ptr(n_accepted), _ptr(wy_table), _ptr(x), _ptr(conv_state_ptrs),
                           _opt(opt))
    _check(_lib.gdn_verify_commit(ctypes.byref(args), _stream(stream)))


def gdn_gated_rmsnorm(o, z, norm_w, out, dims, *, eps=1e-6, opt=None, stream=None):
    T = o.shape[0]
    args = gdn_norm_args(ctypes.sizeof(gdn_norm_args), _dt(o), _dt(z), _dt(out), _dims(dims), T,
                         _ptr(o), _ptr(z), _ptr(norm_w), _ptr(out), eps, 0.0, _opt(opt))
    _check(_lib.gdn_gated_rmsnorm(ctypes.byref(args), _stream(stream)))


def _woa_args(x, conv_w, conv_state_ptrs, a, b, h_state_ptrs, cu_ks, max_k, out, dims, stash, z, norm_w,
              scale, l2_eps, norm_eps, opt):
    return gdn_woa_args(ctypes.sizeof(gdn_woa_args), _dt(x), _dt(out), _dims(dims), cu_ks.numel() - 1, max_k,
                        x.shape[0], 0, _ptr(cu_ks), _ptr(x), _ptr(conv_w), _ptr(conv_state_ptrs), _ptr(a),
                        _ptr(b), _ptr(h_state_ptrs), _ptr(z), _ptr(norm_w), _ptr(out), _ptr(stash),
                        0 if stash is None else stash.numel() * stash.element_size(), scale, l2_eps,
                        norm_eps, 0.0, _opt(opt))


def gdn_woa_stash_bytes(x, cu_ks, max_k, out, dims):
    args = _woa_args(x, None, None, None, None, None, cu_ks, max_k, out, dims, None, None, None, 1.0, 1e-6,
                     1e-6, None)
    n = ctypes.c_size_t(0)
    _check(_lib.gdn_woa_stash_bytes(ctypes.byref(args), ctypes.byref(n)))
    return int(n.value)


def gdn_verify_woa(x, conv_w, conv_state_ptrs, a, b, h_state_ptrs, cu_ks, max_k, out, dims, *, stash=None,
                   z=None, norm_w=None, scale=1.0, l2_eps=1e-6, norm_eps=1e-6, opt=None, stream=None):
    """Write-on-accept verify.  ``stash``: an fp32 device tensor of at least
    ``gdn_woa_stash_bytes`` bytes (allocated here when None); returned."""
    if stash is None:
        nbytes = gdn_woa_stash_bytes(x, cu_ks, max_k, out, dims)
        stash = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=out.device)
    args = _woa_args(x, conv_w, conv_state_ptrs, a, b, h_state_ptrs, cu_ks, max_k, out, dims, stash, z, norm_w,
                     scale, l2_eps, norm_eps, opt)
    _check(_lib.gdn_verify_woa(ctypes.byref(args), _stream(stream)))
    return stash


def gdn_fold_accepted(x, conv_state_ptrs, h_state_ptrs, stash, cu_ks, n_accepted, dims, *, opt=None,
                      stream=None):
    args = gdn_fold_args(ctypes.sizeof(gdn_fold_args), _dt(x), _dims(dims), cu_ks.numel() - 1, x.shape[0],
                         _ptr(cu_ks), _ptr(n_accepted), _ptr(h_state_ptrs), _ptr(stash),
                         stash.numel() * stash.element_size(), _ptr(x), _ptr(conv_state_ptrs), _opt(opt))
    _check(_lib.gdn_fold_accepted(ctypes.byref(args), _stream(stream)))


def gdn_decode_tokens(x, conv_w, conv_state_ptrs, a, b, h_state_ptrs, cu_tokens, max_tokens, out, dims, *,
                      z=None, norm_w=None, scale=1.0, l2_eps=1e-6, norm_eps=1e-6, opt=None, stream=None):
    args = gdn_tokens_args(ctypes.sizeof(gdn_tokens_args), _dt(x), _dt(out), _dims(dims), cu_tokens.numel() - 1,
                           max_tokens, x.shape[0], 0, _ptr(cu_tokens), _ptr(x), _ptr(conv_w),
                           _ptr(conv_state_ptrs), _ptr(a), _ptr(b), _ptr(h_state_ptrs), _ptr(z), _ptr(norm_w),
                           _ptr(out), scale, l2_eps, norm_eps, 0.0, _opt(opt))
    _check(_lib.gdn_decode_tokens(ctypes.byref(args), _stream(stream)))
