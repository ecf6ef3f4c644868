"""C ABI checks that need no GPU: the library loads, exports every declared
entry point, its structs match the ctypes mirror byte for byte, and invalid
arguments are refused with the documented status before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_attention_ssm_core_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
FAKE = 0x1000  # never dereferenced: validation fails before any launch


def _declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(gdn_[a-z0-9_]+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"gdn_conv_l2norm", "gdn_prefill_chunked", "gdn_decode_batched", "gdn_verify_multi",
            "gdn_verify_commit", "gdn_gated_rmsnorm", "gdn_prefill_workspace_bytes",
            "gdn_verify_woa", "gdn_woa_stash_bytes", "gdn_fold_accepted", "gdn_decode_tokens",
            "gdn_status_string", "gdn_abi_version"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for n in names:
        assert n in exported, n
        assert hasattr(B.library(), n)
    assert B.abi_version() == 2


def test_struct_layout_matches_header(tmp_path):
    structs = ["gdn_dims", "gdn_options", "gdn_conv_args", "gdn_prefill_args", "gdn_decode_args",
               "gdn_verify_args", "gdn_commit_args", "gdn_norm_args", "gdn_woa_args", "gdn_fold_args",
               "gdn_tokens_args"]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gdn.h"', "int main(void) {"]
    for s in structs:
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (s, s))
        for f, _ in getattr(B, s)._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (s, f, s, f))
    lines.append("return 0; }")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    for s in structs:
        cls = getattr(B, s)
        assert int(got[s]) == ctypes.sizeof(cls), s
        for f, _ in cls._fields_:
            assert int(got["%s.%s" % (s, f)]) == getattr(cls, f).offset, (s, f)


def test_status_strings():
    for s in range(5):
        assert B.status_string(s).startswith("GDN_")
    assert "unknown" in B.status_string(99)


def _dims(Hk=16, Hv=32, d=128, K=4):
    return B.gdn_dims(Hk, Hv, d, d, K, 0)


def _decode(**kw):
    a = B.gdn_decode_args(ctypes.sizeof(B.gdn_decode_args), 1, 1, _dims(), 4, FAKE, FAKE, FAKE, FAKE,
                          FAKE, FAKE, None, None, FAKE, 1.0, 1e-6, 1e-6, 0.0)
    for k, v in kw.items():
        setattr(a, k, v)
    return B.library().gdn_decode_batched(ctypes.byref(a), None)


def test_decode_validation():
    assert _decode(struct_size=12) == B.GDN_ERR_INVALID_ARG
    assert _decode(num_seqs=-1) == B.GDN_ERR_INVALID_ARG
    assert _decode(x=None) == B.GDN_ERR_INVALID_ARG
    assert _decode(h_state=None) == B.GDN_ERR_INVALID_ARG
    assert _decode(z=FAKE) == B.GDN_ERR_INVALID_ARG          # z without norm_w
    assert _decode(act_dtype=7) == B.GDN_ERR_INVALID_ARG
    assert _decode(scale=float("nan")) == B.GDN_ERR_INVALID_ARG
    assert _decode(l2_eps=-1.0) == B.GDN_ERR_INVALID_ARG
    assert _decode(reserved_f=1.0) == B.GDN_ERR_INVALID_ARG
    assert _decode(dims=_dims(d=96)) == B.GDN_ERR_UNSUPPORTED
    assert _decode(dims=_dims(Hk=4, Hv=32)) == B.GDN_ERR_UNSUPPORTED   # 8 value heads per key head
    assert _decode(dims=_dims(Hk=3, Hv=32)) == B.GDN_ERR_INVALID_ARG   # not a multiple
    assert _decode(dims=B.gdn_dims(16, 32, 128, 64, 4, 0)) == B.GDN_ERR_UNSUPPORTED
    assert _decode(dims=_dims(K=5)) == B.GDN_ERR_UNSUPPORTED
    assert _decode(dims=B.gdn_dims(16, 32, 128, 128, 4, 1)) == B.GDN_ERR_INVALID_ARG
    # nothing to do: accepted without touching the device
    assert _decode(num_seqs=0, x=None, h_state=None) == B.GDN_OK
    assert B.library().gdn_decode_batched(None, None) == B.GDN_ERR_INVALID_ARG


def _verify(**kw):
    a = B.gdn_verify_args(ctypes.sizeof(B.gdn_verify_args), 1, 1, _dims(), 64, 16, 576, 0, FAKE, FAKE,
                          FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1.0, 1e-6, 1e-6, 0.0)
    for k, v in kw.items():
        setattr(a, k, v)
    return B.library().gdn_verify_multi(ctypes.byref(a), None)


def test_verify_validation():
    # tables are staged only for k in 2..16, at most 128 sequences (transformer_layer.rs page)
    assert _verify(max_k=1) == B.GDN_ERR_INVALID_ARG
    assert _verify(max_k=17) == B.GDN_ERR_INVALID_ARG
    assert _verify(num_seqs=129) == B.GDN_ERR_INVALID_ARG
    assert _verify(total_rows=64 * 16 + 1) == B.GDN_ERR_INVALID_ARG
    assert _verify(wy_tables=None) == B.GDN_ERR_INVALID_ARG
    assert _verify(cu_ks=None) == B.GDN_ERR_INVALID_ARG
    assert _verify(reserved=3) == B.GDN_ERR_INVALID_ARG
    assert _verify(dims=_dims(d=256)) == B.GDN_ERR_UNSUPPORTED
    assert _verify(num_seqs=0, total_rows=0) == B.GDN_OK


def _commit(**kw):
    a = B.gdn_commit_args(ctypes.sizeof(B.gdn_commit_args), 1, _dims(), 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return B.library().gdn_verify_commit(ctypes.byref(a), None)


def test_commit_validation():
    assert _commit(num_seqs=129) == B.GDN_ERR_INVALID_ARG
    assert _commit(n_accepted=None) == B.GDN_ERR_INVALID_ARG
    assert _commit(struct_size=0) == B.GDN_ERR_INVALID_ARG
    assert _commit(num_seqs=0) == B.GDN_OK


def _conv(**kw):
    a = B.gdn_conv_args(ctypes.sizeof(B.gdn_conv_args), 1, 1, _dims(), 8, 65536, FAKE, FAKE, FAKE, FAKE,
                        FAKE + 64, 1e-6)
    for k, v in kw.items():
        setattr(a, k, v)
    return B.library().gdn_conv_l2norm(ctypes.byref(a), None)


def test_conv_validation():
    assert _conv(y=FAKE) == B.GDN_ERR_INVALID_ARG          # y aliases x
    assert _conv(num_seqs=0) == B.GDN_ERR_INVALID_ARG      # tokens without sequences
    assert _conv(conv_state=None) == B.GDN_ERR_INVALID_ARG
    assert _conv(l2_eps=float("inf")) == B.GDN_ERR_INVALID_ARG
    assert _conv(total_tokens=0, x=None, y=None) == B.GDN_OK


def _norm(**kw):
    a = B.gdn_norm_args(ctypes.sizeof(B.gdn_norm_args), 0, 1, 1, _dims(), 100, FAKE, FAKE, FAKE, FAKE, 1e-6, 0.0)
    for k, v in kw.items():
        setattr(a, k, v)
    return B.library().gdn_gated_rmsnorm(ctypes.byref(a), None)


def test_norm_validation():
    assert _norm(z=None) == B.GDN_ERR_INVALID_ARG
    assert _norm(in_dtype=2) == B.GDN_ERR_INVALID_ARG
    assert _norm(eps=-1.0) == B.GDN_ERR_INVALID_ARG
    assert _norm(dims=_dims(d=48)) == B.GDN_ERR_UNSUPPORTED
    assert _norm(total_tokens=0, o=None) == B.GDN_OK


def _prefill_args(**kw):
    a = B.gdn_prefill_args(ctypes.sizeof(B.gdn_prefill_args), 1, 1, _dims(), 1, 4096, 64, 0, FAKE, FAKE,
                           None, None, None, FAKE, FAKE, FAKE, None, None, FAKE, 1.0, 1e-6, 1e-6, 0.0,
                           None, 0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _ws(a):
    n = ctypes.c_size_t(0)
    st = B.library().gdn_prefill_workspace_bytes(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_prefill_validation_and_workspace():
    st, need = _ws(_prefill_args())
    assert st == B.GDN_OK and need > 0
    st_f, need_f = _ws(_prefill_args(x=FAKE, conv_w=FAKE, conv_state=FAKE))
    st_e, need_e = _ws(_prefill_args(z=FAKE, norm_w=FAKE))
    assert st_f == st_e == B.GDN_OK and need_f > need and need_e > need
    L = B.library()
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(chunk_size=32)), None) == B.GDN_ERR_UNSUPPORTED
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args()), None) == B.GDN_ERR_WORKSPACE
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(workspace=FAKE, workspace_bytes=need - 1)),
                                 None) == B.GDN_ERR_WORKSPACE
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(y=None)), None) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(z=FAKE)), None) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(x=FAKE)), None) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(h_state=None)), None) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(num_seqs=0)), None) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(reserved_f=2.0)), None) == B.GDN_ERR_INVALID_ARG
    assert _ws(_prefill_args(dims=_dims(d=80)))[0] == B.GDN_ERR_UNSUPPORTED
    ok = _prefill_args(num_seqs=0, total_tokens=0)
    assert L.gdn_prefill_chunked(ctypes.byref(ok), None) == B.GDN_OK


def test_prefill_noalloc_refusals():
    """The allocation-free prefill validates like gdn_prefill_chunked, refuses a
    workspace argument, and refuses a call whose workspace need exceeds its
    per-GPU scratch array -- all before any HIP call."""
    L = B.library()
    call = lambda **kw: L.gdn_prefill_chunked_noalloc(ctypes.byref(_prefill_args(**kw)), None)
    assert B.PREFILL_SCRATCH_BYTES == 64 << 20
    # 512 tokens of 32 heads at d = 128 need about 24 MB; 4096 tokens about 101 MB
    assert _ws(_prefill_args(total_tokens=512))[1] <= B.PREFILL_SCRATCH_BYTES
    assert _ws(_prefill_args(total_tokens=4096))[1] > B.PREFILL_SCRATCH_BYTES
    assert call(total_tokens=4096) == B.GDN_ERR_WORKSPACE
    assert call(total_tokens=512, workspace=FAKE, workspace_bytes=1 << 30) == B.GDN_ERR_INVALID_ARG
    assert call(total_tokens=512, workspace_bytes=1) == B.GDN_ERR_INVALID_ARG
    assert call(total_tokens=512, chunk_size=32) == B.GDN_ERR_UNSUPPORTED
    assert call(total_tokens=512, y=None) == B.GDN_ERR_INVALID_ARG
    assert call(total_tokens=512, h_state=None) == B.GDN_ERR_INVALID_ARG
    assert call(total_tokens=512, dims=_dims(d=80)) == B.GDN_ERR_UNSUPPORTED
    assert call(num_seqs=0, total_tokens=0) == B.GDN_OK


def test_options_are_refused_where_not_taken():
    """Every entry point validates its options before any launch: an unknown value,
    the reserved word, or an option the entry point does not take."""
    F16, RAW, SIG = B.GDN_DTYPE_F16, B.GDN_GATES_RAW, B.GDN_NORM_GATE_SIGMOID
    # decode takes all three: an unknown value or the bf16 "state" is refused
    assert _decode(opt=B.gdn_options(B.GDN_DTYPE_BF16, 0, 0, 0)) == B.GDN_ERR_INVALID_ARG
    assert _decode(opt=B.gdn_options(0, 2, 0, 0)) == B.GDN_ERR_INVALID_ARG
    assert _decode(opt=B.gdn_options(0, 0, 2, 0)) == B.GDN_ERR_INVALID_ARG
    assert _decode(opt=B.gdn_options(0, 0, 0, 1)) == B.GDN_ERR_INVALID_ARG
    assert _decode(num_seqs=0, opt=B.gdn_options(F16, RAW, SIG, 0)) == B.GDN_OK
    assert _verify(num_seqs=0, total_rows=0, opt=B.gdn_options(F16, RAW, SIG, 0)) == B.GDN_OK
    # commit takes only the state dtype, the norm only the norm gate
    assert _commit(num_seqs=0, opt=B.gdn_options(F16, 0, 0, 0)) == B.GDN_OK
    assert _commit(opt=B.gdn_options(0, RAW, 0, 0)) == B.GDN_ERR_INVALID_ARG
    assert _commit(opt=B.gdn_options(0, 0, SIG, 0)) == B.GDN_ERR_INVALID_ARG
    assert _norm(total_tokens=0, o=None, opt=B.gdn_options(0, 0, SIG, 0)) == B.GDN_OK
    assert _norm(opt=B.gdn_options(F16, 0, 0, 0)) == B.GDN_ERR_INVALID_ARG
    assert _norm(opt=B.gdn_options(0, RAW, 0, 0)) == B.GDN_ERR_INVALID_ARG
    ok = _prefill_args(num_seqs=0, total_tokens=0, opt=B.gdn_options(F16, RAW, SIG, 0))
    assert B.library().gdn_prefill_chunked(ctypes.byref(ok), None) == B.GDN_OK


def _woa_args(**kw):
    a = B.gdn_woa_args(struct_size=ctypes.sizeof(B.gdn_woa_args), act_dtype=1, out_dtype=1, dims=_dims(),
                       num_seqs=64, max_k=16, total_rows=576, cu_ks=FAKE, x=FAKE, conv_w=FAKE,
                       conv_state=FAKE, a=FAKE, b=FAKE, h_state=FAKE, out=FAKE, stash=FAKE,
                       stash_bytes=0, scale=1.0, l2_eps=1e-6, norm_eps=1e-6)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_woa_validation_and_stash_size():
    L = B.library()
    n = ctypes.c_size_t(0)
    assert L.gdn_woa_stash_bytes(ctypes.byref(_woa_args()), ctypes.byref(n)) == B.GDN_OK
    # per row: k_hat of 16 key heads, u and a of 32 value heads (16*128 + 32*128 + 32 floats)
    assert n.value == 576 * (16 * 128 + 32 * 128 + 32) * 4
    n2 = ctypes.c_size_t(0)
    assert L.gdn_woa_stash_bytes(ctypes.byref(_woa_args(dims=B.gdn_dims(1, 1, 32, 32, 4, 0), total_rows=3)),
                                 ctypes.byref(n2)) == B.GDN_OK
    assert n2.value == 3 * 68 * 4  # 32 + 32 + 1 floats, rounded up to 68
    run = lambda **kw: L.gdn_verify_woa(ctypes.byref(_woa_args(**kw)), None)
    assert run() == B.GDN_ERR_WORKSPACE
    assert run(stash_bytes=n.value - 4) == B.GDN_ERR_WORKSPACE
    assert run(stash=None, stash_bytes=n.value) == B.GDN_ERR_WORKSPACE
    assert run(max_k=17, stash_bytes=n.value) == B.GDN_ERR_INVALID_ARG
    assert run(num_seqs=129, stash_bytes=n.value) == B.GDN_ERR_INVALID_ARG
    assert run(h_state=None, stash_bytes=n.value) == B.GDN_ERR_INVALID_ARG
    assert run(reserved_f=1.0, stash_bytes=n.value) == B.GDN_ERR_INVALID_ARG
    assert run(num_seqs=0, total_rows=0, stash=None) == B.GDN_OK


def _fold(**kw):
    a = B.gdn_fold_args(struct_size=ctypes.sizeof(B.gdn_fold_args), act_dtype=1, dims=_dims(), num_seqs=64,
                        total_rows=576, cu_ks=FAKE, n_accepted=FAKE, h_state=FAKE, stash=FAKE,
                        stash_bytes=576 * 6176 * 4, x=FAKE, conv_state=FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return B.library().gdn_fold_accepted(ctypes.byref(a), None)


def test_fold_validation():
    assert _fold(stash_bytes=576 * 6176 * 4 - 1) == B.GDN_ERR_WORKSPACE
    assert _fold(n_accepted=None) == B.GDN_ERR_INVALID_ARG
    assert _fold(num_seqs=129) == B.GDN_ERR_INVALID_ARG
    assert _fold(opt=B.gdn_options(0, B.GDN_GATES_RAW, 0, 0)) == B.GDN_ERR_INVALID_ARG
    assert _fold(num_seqs=0, opt=B.gdn_options(B.GDN_DTYPE_F16, 0, 0, 0)) == B.GDN_OK


def _tokens(**kw):
    a = B.gdn_tokens_args(struct_size=ctypes.sizeof(B.gdn_tokens_args), act_dtype=1, out_dtype=1, dims=_dims(),
                          num_seqs=8, max_tokens=17, total_rows=100, cu_tokens=FAKE, x=FAKE, conv_w=FAKE,
                          conv_state=FAKE, a=FAKE, b=FAKE, h_state=FAKE, out=FAKE, scale=1.0, l2_eps=1e-6,
                          norm_eps=1e-6)
    for k, v in kw.items():
        setattr(a, k, v)
    return B.library().gdn_decode_tokens(ctypes.byref(a), None)


def test_tokens_validation():
    assert _tokens(max_tokens=18) == B.GDN_ERR_INVALID_ARG
    assert _tokens(max_tokens=0) == B.GDN_ERR_INVALID_ARG
    assert _tokens(total_rows=8 * 17 + 1) == B.GDN_ERR_INVALID_ARG
    assert _tokens(num_seqs=129) == B.GDN_ERR_INVALID_ARG
    assert _tokens(cu_tokens=None) == B.GDN_ERR_INVALID_ARG
    assert _tokens(z=FAKE) == B.GDN_ERR_INVALID_ARG
    assert _tokens(num_seqs=0, total_rows=0) == B.GDN_OK


def test_misaligned_buffers_are_refused():
    # buffers passed directly in the argument structs start on a 16-byte boundary
    # (the kernels move them in 8- and 16-byte vectors); the check precedes any launch
    bad = FAKE + 8
    L = B.library()
    assert _decode(x=bad) == B.GDN_ERR_INVALID_ARG
    assert _decode(out=bad) == B.GDN_ERR_INVALID_ARG
    assert _verify(conv_w=bad) == B.GDN_ERR_INVALID_ARG
    assert _commit(x=bad) == B.GDN_ERR_INVALID_ARG
    assert _conv(y=FAKE + 72) == B.GDN_ERR_INVALID_ARG
    assert _norm(o=bad) == B.GDN_ERR_INVALID_ARG
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(out=bad)), None) == B.GDN_ERR_INVALID_ARG
    need = _ws(_prefill_args())[1]
    assert L.gdn_prefill_chunked(ctypes.byref(_prefill_args(workspace=bad, workspace_bytes=need)),
                                 None) == B.GDN_ERR_INVALID_ARG
    stash = 576 * (16 * 128 + 32 * 128 + 32) * 4
    assert L.gdn_verify_woa(ctypes.byref(_woa_args(stash=bad, stash_bytes=stash)), None) == B.GDN_ERR_INVALID_ARG
    assert _fold(stash=bad) == B.GDN_ERR_INVALID_ARG
    assert _tokens(x=bad) == B.GDN_ERR_INVALID_ARG
