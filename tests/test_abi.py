"""CPU checks of the C ABI: the library builds and loads, exports every function that
include/kda.h declares, its struct layout matches the Python binding, and host-side
validation returns the documented status codes without launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

import linear_attention_recurrence_07_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = _declared_functions()
    for n in ("kda_chunk_prefill", "kda_chunk_prefill_workspace_size", "kda_recurrent_step", "kda_short_conv", "kda_gated_norm_proj", "kda_out_proj", "kda_out_proj_workspace_size",
              "kda_gated_rmsnorm", "kda_status_string", "kda_last_error", "kda_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = K.load_library()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", K.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\S+)", out))
    for n in _declared_functions():
        assert n in exported, n


def test_params_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(f'''#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu", sizeof(kda_params_t));
#define F(x) printf(" %zu", offsetof(kda_params_t, x));
  F(B) F(T) F(H) F(dk) F(dv) F(num_seqs) F(chunk) F(scale) F(use_qk_l2norm) F(in_dtype) F(out_dtype) F(norm_eps)
  F(decay_per_head)
  return 0;
}}''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(K.KdaParams)] + [getattr(K.KdaParams, f).offset for f, _ in K.KdaParams._fields_]
    assert got == want


def _p(**kw):
    base = dict(B=1, T=64, H=2, dk=128, dv=128)
    base.update({k: v for k, v in kw.items() if k in base})
    rest = {k: v for k, v in kw.items() if k not in base}
    return K._params(base["B"], base["T"], base["H"], base["dk"], base["dv"], **rest)


A = ctypes.c_void_p(1 << 20)          # a 16-byte-aligned stand-in address; never dereferenced
MIS = ctypes.c_void_p((1 << 20) + 4)  # misaligned
WS, UNSUP = K.KDA_ERR_WORKSPACE, K.KDA_ERR_UNSUPPORTED


def _prefill(p, ws=None, ws_bytes=0, **ptrs):
    """Call kda_chunk_prefill with stand-in pointers.  Every call here must fail host
    validation: a call that passed it would launch kernels on these addresses."""
    lib = K.load_library()
    names = ["q", "k", "v", "g", "beta", "init", "cu", "mask", "o", "fs", "gate", "w", "y"]
    default = dict(q=A, k=A, v=A, g=A, beta=A, init=None, cu=None, mask=None, o=A, fs=A,
                   gate=None, w=None, y=None)
    default.update(ptrs)
    return lib.kda_chunk_prefill(None if p is None else ctypes.byref(p),
                                 *[default[n] for n in names], ws, ws_bytes, None)


def test_prefill_validation_codes():
    assert _prefill(None) == 1
    assert _prefill(_p(), q=None) == 1
    assert _prefill(_p(), o=None) == 1
    # o may be NULL when y is wanted: these get past the o check and stop at a later one
    assert _prefill(_p(), o=None, gate=A, w=A, y=A) == WS                   # the workspace check
    assert _prefill(_p(chunk=16), o=None, gate=A, w=A, y=MIS) == 4         # y's alignment
    assert _prefill(_p(B=0)) == 2
    assert _prefill(_p(T=-1)) == 2
    assert _prefill(_p(in_dtype=7)) == 3
    assert _prefill(_p(), k=MIS) == 4
    assert _prefill(_p(B=1, num_seqs=1), cu=A, mask=A) == 5
    assert _prefill(_p(B=2, num_seqs=2), cu=A) == 5
    assert _prefill(_p(), gate=A) == 5                       # gate without weight and y
    assert _prefill(_p(chunk=64)) == WS                      # 64-token chunks: the matrix-core kernel (needs the workspace)
    assert _prefill(_p(chunk=48)) == UNSUP
    assert _prefill(_p(dk=16, dv=16, chunk=64)) == UNSUP     # 32/64-token chunks only on the MFMA path
    assert _prefill(_p(dk=96, dv=96)) == UNSUP
    assert _prefill(_p(dk=16, dv=16, chunk=32)) == UNSUP         # 32-token chunks only on the MFMA path
    assert _prefill(_p(in_dtype=0, chunk=32)) == UNSUP
    assert _prefill(_p(scale=float("nan"))) == 2
    bad = _p()
    bad.decay_per_head = 2
    assert _prefill(bad) == 2
    assert _prefill(_p(), g=ctypes.c_void_p((1 << 20) + 4)) == 4            # per-channel g: 16-byte aligned
    assert _prefill(_p(decay_per_head=1), g=ctypes.c_void_p((1 << 20) + 4), o=None) == 1   # per-head g: 4 bytes


def test_prefill_workspace_size_and_checks():
    lib = K.load_library()
    size = lambda p, packed=0: lib.kda_chunk_prefill_workspace_size(ctypes.byref(p), packed)
    rec = 32272 + 512                                      # bytes per (chunk, head): record + norm exchange
    tail = 256                                             # the status word of the partner waits
    assert size(_p(B=1, T=64, H=2)) == 1 * 2 * 2 * rec + tail   # B * ceil(T/32) * H records
    assert size(_p(B=3, T=65, H=2)) == 3 * 3 * 2 * rec + tail
    assert size(_p(B=1, T=64, H=2, num_seqs=3), 1) == (3 + 2) * 2 * rec + tail   # (N + ceil(T/32)) * H
    assert size(_p(B=1, T=64, H=2), 1) == 0                 # packed without num_seqs: invalid
    assert size(_p(chunk=16)) == 0                          # vector-ALU kernel: no workspace
    assert size(_p(chunk=64)) == size(_p(chunk=32)) == size(_p())   # 64-token chunks run as two 32-token halves
    assert size(_p(dk=64, dv=64)) == 0
    assert size(_p(in_dtype=0)) == 0
    assert lib.kda_chunk_prefill_workspace_size(None, 0) == 0
    need = size(_p())
    assert _prefill(_p()) == WS                              # missing workspace
    assert _prefill(_p(), ws=A, ws_bytes=need - 1) == WS     # too small
    assert _prefill(_p(), ws=MIS, ws_bytes=need) == 4       # misaligned
    assert lib.kda_status_string(WS) == b"KDA_ERR_WORKSPACE"


def test_chunk_states_workspace_size_and_checks():
    """kda_chunk_prefill_states: the prefill's workspace plus 32 x 128 fp32 U rows per
    chunk and head; host validation before anything is launched."""
    lib = K.load_library()
    size = lambda p, packed=0: lib.kda_chunk_prefill_states_workspace_size(ctypes.byref(p), packed)
    per = 32272 + 512 + 32 * 128 * 4
    assert size(_p(B=1, T=64, H=2)) == 1 * 2 * 2 * per + 256
    assert size(_p(B=3, T=65, H=2)) == 3 * 3 * 2 * per + 256
    assert size(_p(B=1, T=64, H=2, num_seqs=3), 1) == (3 + 2) * 2 * per + 256
    assert size(_p(B=1, T=64, H=2), 1) == 0
    assert size(_p(chunk=16)) == 0 and size(_p(dk=64, dv=64)) == 0 and size(_p(in_dtype=0)) == 0
    assert lib.kda_chunk_prefill_states_workspace_size(None, 0) == 0
    need = size(_p())

    def call(p, ws=None, nbytes=0, **ptrs):
        names = ["q", "k", "v", "g", "beta", "init", "cu", "mask", "o", "fs", "gate", "w", "y", "states"]
        d = dict(q=A, k=A, v=A, g=A, beta=A, init=None, cu=None, mask=None, o=A, fs=A, gate=None, w=None, y=None,
                 states=A)
        d.update(ptrs)
        return lib.kda_chunk_prefill_states(ctypes.byref(p), *[d[n] for n in names], ws, nbytes, None)

    assert call(_p()) == WS                                          # a valid call stops at the missing workspace
    assert call(_p(), ws=A, nbytes=need - 1) == WS
    assert call(_p(), ws=A, nbytes=lib.kda_chunk_prefill_workspace_size(ctypes.byref(_p()), 0)) == WS
    assert call(_p(), states=None) == 1
    assert call(_p(), states=MIS) == 4
    assert call(_p(), o=None, gate=A, w=A, y=A) == 1                 # o is required here
    assert call(_p(dk=64, dv=64)) == UNSUP                          # only the matrix-core prefill
    assert call(_p(in_dtype=0)) == UNSUP
    assert call(_p(chunk=16)) == UNSUP
    assert call(_p(), q=None) == 1


def test_stage_validation_codes():
    lib = K.load_library()
    need = lib.kda_chunk_prefill_workspace_size(ctypes.byref(_p()), 0)

    def prep(p, ws=A, nbytes=need, **ptrs):
        d = dict(q=A, k=A, g=A, beta=A, cu=None, mask=None)
        d.update(ptrs)
        return lib.kda_chunk_prepare(None if p is None else ctypes.byref(p),
                                     *[d[n] for n in ("q", "k", "g", "beta", "cu", "mask")], ws, nbytes, None)

    def scan(p, ws=A, nbytes=need, **ptrs):
        d = dict(v=A, init=None, cu=None, o=A, fs=A, gate=None, w=None, y=None)
        d.update(ptrs)
        return lib.kda_chunk_scan(None if p is None else ctypes.byref(p), d["v"], d["init"], d["cu"],
                                  ws, nbytes, d["o"], d["fs"], d["gate"], d["w"], d["y"], None)

    for f in (prep, scan):
        assert f(None) == 1
        assert f(_p(B=0)) == 2
        assert f(_p(in_dtype=0)) == UNSUP                       # fp32: no two-stage kernel
        assert f(_p(chunk=16)) == UNSUP
        assert f(_p(dk=64, dv=64)) == UNSUP
        assert f(_p(), ws=None, nbytes=0) == WS
        assert f(_p(), nbytes=need - 1) == WS
        assert f(_p(), ws=MIS) == 4
        assert f(_p(B=2, num_seqs=2), cu=A) == 5
    assert prep(_p(), q=None) == 1
    assert prep(_p(), g=MIS) == 4
    assert prep(_p(B=1, num_seqs=1), cu=A, mask=A) == 5
    assert scan(_p(), v=None) == 1
    assert scan(_p(), fs=None) == 1
    assert scan(_p(), o=None) == 1                          # o is required without y
    assert scan(_p(), o=None, gate=A, w=A, y=A, nbytes=need - 1) == WS   # ... and optional with it
    assert scan(_p(), init=MIS) == 4
    assert scan(_p(), y=A) == 5                             # gate, norm_weight, y: all or none
    assert scan(_p(), gate=A, w=A) == 5
    assert scan(_p(), gate=A, w=A, y=MIS) == 4


def test_recurrent_and_norm_validation_codes():
    lib = K.load_library()
    names = ["q", "k", "v", "g", "beta", "state", "mask", "o", "gate", "w", "y"]

    def rec(p, **ptrs):
        d = dict(q=A, k=A, v=A, g=A, beta=A, state=A, mask=None, o=A, gate=None, w=None, y=None)
        d.update(ptrs)
        return lib.kda_recurrent_step(ctypes.byref(p), *[d[n] for n in names], None)

    assert rec(_p(), state=None) == 1
    assert rec(_p(), o=None, gate=A, w=A, y=A) == 1           # o is required here, even with y
    assert rec(_p(dk=128, dv=64)) == UNSUP
    assert rec(_p(), y=A) == 5
    assert rec(_p(), g=MIS) == 4
    assert rec(_p(T=0)) == 0                                  # nothing to do, nothing launched
    st_names = names[:-1] + ["y", "states"]

    def rec_states(p, **ptrs):
        d = dict(q=A, k=A, v=A, g=A, beta=A, state=A, mask=None, o=A, gate=None, w=None, y=None, states=A)
        d.update(ptrs)
        return lib.kda_recurrent_states(ctypes.byref(p), *[d[n] for n in names], d["states"], None)

    assert rec_states(_p(), states=None) == 1
    assert rec_states(_p(), states=MIS) == 4
    assert rec_states(_p(), state=None) == 1
    assert rec_states(_p(dk=128, dv=64)) == UNSUP
    norm = lib.kda_gated_rmsnorm
    assert norm(A, A, A, A, 10, 100, 1e-6, 1, 1, None) == UNSUP
    assert norm(A, A, A, A, -1, 128, 1e-6, 1, 1, None) == 2
    assert norm(None, A, A, A, 10, 128, 1e-6, 1, 1, None) == 1
    assert norm(A, A, A, A, 10, 128, 1e-6, 5, 1, None) == 3
    assert norm(A, A, A, A, 10, 128, -1.0, 1, 1, None) == 2
    assert norm(A, A, A, A, 0, 128, 1e-6, 1, 1, None) == 0   # zero rows: no launch


def test_conv_params_struct_layout_matches_header(tmp_path):
    src = tmp_path / "conv_layout.c"
    src.write_text(f'''#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu", sizeof(kda_conv_params_t));
#define F(x) printf(" %zu", offsetof(kda_conv_params_t, x));
  F(B) F(T) F(D) F(num_seqs) F(width) F(activation) F(in_dtype) F(out_dtype)
  return 0;
}}''')
    exe = tmp_path / "conv_layout"
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(K.KdaConvParams)] + [getattr(K.KdaConvParams, f).offset for f, _ in K.KdaConvParams._fields_]
    assert got == want


def test_conv_validation_codes():
    lib = K.load_library()

    def conv(B=1, T=64, D=64, N=0, W=4, act=1, ind=1, outd=1, **ptrs):
        p = K.KdaConvParams(B, T, D, N, W, act, ind, outd)
        d = dict(x=A, w=A, init=None, cu=None, mask=None, y=ctypes.c_void_p(1 << 30), fs=None)
        d.update(ptrs)
        return lib.kda_short_conv(ctypes.byref(p), *[d[n] for n in ("x", "w", "init", "cu", "mask", "y", "fs")], None)

    assert lib.kda_short_conv(None, A, A, None, None, None, A, None, None) == 1
    assert conv(x=None) == 1
    assert conv(w=None) == 1
    assert conv(y=None) == 1
    assert conv(B=0) == 2
    assert conv(T=-1) == 2
    assert conv(act=2) == 2
    assert conv(ind=5) == 3
    assert conv(x=MIS) == 4
    assert conv(init=MIS) == 4
    assert conv(cu=A, mask=A, N=1) == 5
    assert conv(B=2, cu=A, N=2) == 5
    assert conv(y=A) == 5                                    # y overlapping x
    assert conv(D=60) == UNSUP
    assert conv(W=5) == UNSUP
    assert conv(W=1) == UNSUP
    assert conv(B=70000) == UNSUP
    assert conv(cu=A, N=0) == 2


def test_fused_conv_struct_layout_matches_header(tmp_path):
    src = tmp_path / "fused_conv_layout.c"
    src.write_text(f'''#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu", sizeof(kda_conv_t));
#define F(x) printf(" %zu", offsetof(kda_conv_t, x));
  F(width) F(activation) F(weight_q) F(weight_k) F(weight_v) F(initial_q) F(initial_k) F(initial_v)
  F(final_q) F(final_k) F(final_v)
  return 0;
}}''')
    exe = tmp_path / "fused_conv_layout"
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(K.KdaConv)] + [getattr(K.KdaConv, f).offset for f, _ in K.KdaConv._fields_]
    assert got == want


def _cv(**kw):
    f = dict(width=4, activation=1, weight_q=A, weight_k=A, weight_v=A, initial_q=None, initial_k=None,
             initial_v=None, final_q=None, final_k=None, final_v=None)
    f.update(kw)
    return K.KdaConv(*[f[n] for n, _ in K.KdaConv._fields_])


def test_fused_conv_validation_codes():
    """Every call fails host validation (none may launch on the stand-in addresses)."""
    lib = K.load_library()

    def pre(p, cv, **ptrs):
        names = ["q", "k", "v", "g", "beta", "init", "cu", "mask", "o", "fs", "gate", "w", "y"]
        d = dict(q=A, k=A, v=A, g=A, beta=A, init=None, cu=None, mask=None, o=A, fs=A, gate=None, w=None, y=None)
        d.update(ptrs)
        return lib.kda_chunk_prefill_conv(ctypes.byref(p), None if cv is None else ctypes.byref(cv),
                                          *[d[n] for n in names], None, 0, None)

    def rec(p, cv, **ptrs):
        names = ["q", "k", "v", "g", "beta", "state", "mask", "o", "gate", "w", "y"]
        d = dict(q=A, k=A, v=A, g=A, beta=A, state=A, mask=None, o=A, gate=None, w=None, y=None)
        d.update(ptrs)
        return lib.kda_recurrent_step_conv(ctypes.byref(p), None if cv is None else ctypes.byref(cv),
                                           *[d[n] for n in names], None)

    assert pre(_p(), None) == 1
    assert pre(_p(), _cv(weight_k=None)) == 1
    assert pre(_p(), _cv(activation=2)) == 2
    assert pre(_p(), _cv(width=5)) == UNSUP
    assert pre(_p(), _cv(width=1)) == UNSUP
    assert pre(_p(), _cv(weight_v=MIS)) == 4
    assert pre(_p(), _cv(initial_q=MIS)) == 4
    assert pre(_p(), _cv(final_v=MIS)) == 4
    assert pre(_p(), _cv()) == WS                              # a valid call stops at the missing workspace
    assert pre(_p(dk=16, dv=16), _cv()) == UNSUP               # only the matrix-core prefill filters in-kernel
    assert pre(_p(in_dtype=0), _cv()) == UNSUP
    assert pre(_p(chunk=16), _cv()) == UNSUP
    assert pre(_p(), _cv(), q=None) == 1                       # the ordinary checks still run first
    assert pre(_p(B=70000, T=1, H=1), _cv()) == UNSUP          # more sequences than the carry launch takes
    assert rec(_p(T=1), None) == 1
    assert rec(_p(T=1), _cv(weight_q=None)) == 1
    assert rec(_p(T=1), _cv(activation=-1)) == 2
    assert rec(_p(T=1), _cv(width=7)) == UNSUP
    assert rec(_p(T=1), _cv(final_k=MIS)) == 4
    assert rec(_p(T=1, dk=128, dv=64), _cv()) == UNSUP


def test_fused_conv_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16)
    g = torch.zeros((1, 4, 2, 128))
    b = torch.zeros((1, 4, 2))
    w = torch.zeros((256, 4))
    with pytest.raises(ValueError):
        K.chunk_prefill_conv(q, q, q, g, b, conv_weights=(w, w, w))
    with pytest.raises(ValueError):
        K.recurrent_step_conv(q, q, q, g, b, torch.zeros((1, 2, 128, 128)), conv_weights=(w, w, w))


def test_out_proj_validation_codes():
    lib = K.load_library()
    ws = lib.kda_out_proj_workspace_size
    assert ws(64, 12288, 7168) == 4 * 64 * 7168 * 4          # K split 4 ways: fp32 partials
    assert ws(64, 512, 64) == 2 * 64 * 64 * 4
    assert ws(64, 256, 64) == 0                              # one K slice: no partials
    assert ws(65, 12288, 7168) == 0                          # more than 64 rows: not split
    assert ws(64, 300, 64) == 0                              # unsupported sizes

    def op(x=A, w=A, out=A, rows=64, K=256, N=64, dt=1, wsp=None, nb=0):
        return lib.kda_out_proj(x, w, out, rows, K, N, dt, wsp, nb, None)

    assert op(x=None) == 1
    assert op(out=None) == 1
    assert op(rows=-1) == 2
    assert op(K=0) == 2
    assert op(dt=9) == 3
    assert op(x=MIS) == 4
    assert op(K=300) == UNSUP                                    # in_features % 256
    assert op(N=96) == UNSUP                                     # out_features % 64
    assert op(K=1024) == WS                                   # split K needs the workspace
    assert op(K=1024, wsp=MIS, nb=ws(64, 1024, 64)) == 4
    assert op(rows=0) == 0                                   # no rows: nothing launched

    def gp(o=A, gate=A, w=A, pw=A, y=A, out=A, rows=64, heads=96, hd=128, N=7168, eps=1e-6, dt=1, wsp=None, nb=0):
        return lib.kda_gated_norm_proj(o, gate, w, pw, y, out, rows, heads, hd, N, eps, dt, wsp, nb, None)

    assert gp(o=None) == 1
    assert gp(y=None) == 1
    assert gp(heads=0) == 2
    assert gp(eps=-1.0) == 2
    assert gp(hd=100) == UNSUP                                   # head_dim not a power of two
    assert gp(heads=3, hd=64) == UNSUP                           # heads * head_dim % 256
    assert gp(N=7000) == UNSUP                                   # out_features % 64
    assert gp(gate=MIS) == 4
    assert gp() == WS                                         # the decode shape needs the workspace


def test_status_codes_match_the_boundary_table():
    """kda_status_t keeps the numbering of the boundary's status table (NULL 1 .. HIP 8);
    the timeout of a bounded wait comes after it."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    got = {n: int(v) for n, v in re.findall(r"\b(KDA_(?:OK|ERR_[A-Z]+))\s*=\s*(\d+)", text)}
    assert got == {"KDA_OK": 0, "KDA_ERR_NULL": 1, "KDA_ERR_SHAPE": 2, "KDA_ERR_DTYPE": 3, "KDA_ERR_ALIGN": 4,
                   "KDA_ERR_CONFLICT": 5, "KDA_ERR_WORKSPACE": 6, "KDA_ERR_UNSUPPORTED": 7, "KDA_ERR_HIP": 8,
                   "KDA_ERR_TIMEOUT": 9}
    assert {K._STATUS[v]: v for v in K._STATUS} == got


def test_status_strings_and_version():
    lib = K.load_library()
    for code, name in K._STATUS.items():
        assert lib.kda_status_string(code).decode() == name
    assert "gfx950" in K.version()


def test_binding_rejects_cpu_tensors():
    import torch
    t = torch.zeros((1, 4, 2, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        K.chunk_prefill(t, t, t, t.float(), torch.zeros((1, 4, 2)))


def test_binding_checks_caller_buffers_before_any_launch():
    """Caller-supplied outputs are checked for shape and dtype on the host: the library
    only sees addresses, so a short or narrower buffer would be written past its end.
    With CPU tensors every call stops either at such a check or at the device check."""
    import torch
    B, T, H, d = 1, 4, 2, 16
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros((B, T, H, d), dtype=bf)
    g = torch.zeros((B, T, H, d))
    beta = torch.zeros((B, T, H))
    gate, w = torch.zeros((B, T, H, d), dtype=bf), torch.ones(d)
    with pytest.raises(ValueError, match="out must have shape"):
        K.chunk_prefill(q, q, q, g, beta, out=torch.zeros((B, T, H, d // 2), dtype=bf))
    with pytest.raises(TypeError, match="y must be"):          # o and y share out's dtype
        K.chunk_prefill(q, q, q, g, beta, gate=gate, norm_weight=w, out=torch.zeros((B, T, H, d), dtype=bf),
                        y=torch.zeros((B, T, H, d), dtype=f32), output_dtype=f32)
    with pytest.raises(ValueError, match="final_state must have shape"):   # one slab per packed sequence
        K.chunk_prefill(q, q, q, g, beta, cu_seqlens=torch.tensor([0, 2, 4], dtype=torch.int32),
                        final_state=torch.zeros((1, H, d, d)))
    with pytest.raises(TypeError, match="final_state must be"):
        K.chunk_prefill(q, q, q, g, beta, final_state=torch.zeros((B, H, d, d), dtype=bf))
    with pytest.raises(ValueError, match="initial_state must have shape"):
        K.chunk_prefill(q, q, q, g, beta, torch.zeros((2, H, d, d)))
    with pytest.raises(ValueError, match="must be a GPU tensor"):          # all shapes right: device check
        K.chunk_prefill(q, q, q, g, beta, out=torch.zeros((B, T, H, d), dtype=f32),
                        final_state=torch.zeros((B, H, d, d)))
    with pytest.raises(ValueError, match="out must have shape"):
        K.chunk_scan(q, torch.zeros(16, dtype=torch.uint8), out=torch.zeros((B, T, H + 1, d), dtype=bf))
    with pytest.raises(TypeError, match="y must be"):
        K.chunk_scan(q, torch.zeros(16, dtype=torch.uint8), gate=gate, norm_weight=w, output_dtype=f32,
                     y=torch.zeros((B, T, H, d), dtype=bf))
    st = torch.zeros((B, H, d, d))
    with pytest.raises(ValueError, match="out must have shape"):
        K.recurrent_step(q, q, q, g, beta, st, out=torch.zeros((B, T - 1, H, d), dtype=bf))
    with pytest.raises(ValueError, match="states must have shape"):
        K.recurrent_step(q, q, q, g, beta, st, states=torch.zeros((B, T, H, d, d // 2)))
    with pytest.raises(TypeError, match="state must be"):
        K.recurrent_step(q, q, q, g, beta, st.to(bf))
    with pytest.raises(ValueError, match="out must have shape"):
        K.gated_rmsnorm(q, gate, w, out=torch.zeros((B, T, H, d + 8), dtype=bf))


def test_prefill_status_validation():
    """kda_chunk_prefill_status fails host validation before it touches the stream or the
    workspace (stand-in pointers are never read here)."""
    lib = K.load_library()
    st = lambda p, packed=0, ws=A, nbytes=1 << 30: lib.kda_chunk_prefill_status(
        None if p is None else ctypes.byref(p), packed, ws, nbytes, None)
    need = lib.kda_chunk_prefill_workspace_size(ctypes.byref(_p()), 0)
    assert st(None) == 1
    assert st(_p(), ws=None) == 1
    assert st(_p(), nbytes=need - 1) == WS
    assert st(_p(), ws=MIS) == 4
    assert st(_p(in_dtype=0)) == UNSUP
    assert st(_p(chunk=16)) == UNSUP
    assert st(_p(), packed=1) == 2                         # packed without num_seqs


def test_noalloc_exit_rejects_sizes_beyond_its_static_scratch():
    """kda_gated_norm_proj_noalloc: the split-K partials of 64 rows x 16,448 features
    (4 x 64 x 16,448 x 4 bytes) exceed the 16 MiB static scratch -> KDA_ERR_WORKSPACE,
    decided on the host before anything touches the GPU; the usual validation first."""
    lib = K.load_library()
    f = lambda rows=64, heads=96, hd=128, N=7168, o=A: lib.kda_gated_norm_proj_noalloc(
        o, A, A, A, A, A, rows, heads, hd, N, ctypes.c_float(1e-6), 1, None)
    assert f(N=16448) == WS
    assert f(o=None) == 1
    assert f(hd=100) == UNSUP
    assert f(rows=-1) == 2
    assert f(o=MIS) == 4
