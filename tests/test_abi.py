"""The C-ABI library loads, exports every entry point the header declares, and rejects bad
arguments on the host before any HIP call (no GPU is needed for these)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_ns.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:MNS_API\s+)?(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    from newton_schulz_matrix_muon_amd import ops
    return ops.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("muon_ns_batched", "gram_ns_batched", "muon_step", "mns_workspace_bytes",
              "mns_status_string", "mns_last_hip_error"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 18
    for name in names:
        assert hasattr(L, name), name


def test_library_exports_nothing_else():
    """Built with hidden visibility: the dynamic symbol table holds the header's functions and
    no internal host function or kernel launch stub."""
    import shutil
    import subprocess
    from newton_schulz_matrix_muon_amd import ops
    if not shutil.which("nm"):
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    funcs = {l.split()[-1] for l in out.splitlines() if len(l.split()) == 3 and l.split()[1] == "T"}
    assert funcs == set(declared_functions())


def test_status_strings_and_version(L):
    for code in (0, -1, -2, -3, -4, -5, -6, 12345):
        assert L.mns_status_string(code)
    assert L.mns_version() >= 100
    assert L.mns_last_hip_error() == 0


def _t(ops, ptr=0x10000, dtype=1, batch=2, rows=8, cols=16, ld=None, stride=None):
    ld = cols if ld is None else ld
    stride = rows * ld if stride is None else stride
    return ops.MnsTensor(ptr, dtype, batch, rows, cols, ld, stride)


def test_workspace_query_is_host_only_and_monotone(L):
    from newton_schulz_matrix_muon_amd import ops
    p = ops.ns_params(io_dtype=ops.BF16)
    G = _t(ops, batch=648, rows=2048, cols=7168)
    out = {}
    for variant in (ops.STANDARD, ops.GRAM):
        b1, ball = ctypes.c_size_t(), ctypes.c_size_t()
        assert L.mns_workspace_bytes(variant, ctypes.byref(G), ctypes.byref(p), 1, ctypes.byref(b1)) == 0
        assert L.mns_workspace_bytes(variant, ctypes.byref(G), ctypes.byref(p), 0, ctypes.byref(ball)) == 0
        assert 50e6 < b1.value < 200e6 and ball.value > 600 * b1.value
        out[variant] = b1.value
    # transposed orientation needs the same space
    Gt = _t(ops, batch=648, rows=7168, cols=2048)
    bt = ctypes.c_size_t()
    assert L.mns_workspace_bytes(ops.GRAM, ctypes.byref(Gt), ctypes.byref(p), 1, ctypes.byref(bt)) == 0
    assert bt.value == out[ops.GRAM]


def test_matrices_beyond_the_32_bit_operand_range_are_rejected_up_front(L):
    """One n x m iterate may span at most 2^31 bytes (the products' 32-bit operand offsets):
    the limit is reported by the workspace query and by the call itself, before any HIP call
    (the pointers here are not device memory)."""
    from newton_schulz_matrix_muon_amd import ops
    p = ops.ns_params(io_dtype=ops.BF16)
    b = ctypes.c_size_t()
    ok = _t(ops, batch=1, rows=32768, cols=32768)                  # exactly 2^31 bytes
    big = _t(ops, batch=1, rows=32768, cols=32776)                 # 2^31 + 512 KiB
    tall = _t(ops, batch=1, rows=32776, cols=32768)                # same, transposed orientation
    assert L.mns_workspace_bytes(ops.GRAM, ctypes.byref(ok), ctypes.byref(p), 0, ctypes.byref(b)) == 0
    for t in (big, tall):
        assert L.mns_workspace_bytes(ops.GRAM, ctypes.byref(t), ctypes.byref(p), 0, ctypes.byref(b)) == -3
        o = _t(ops, ptr=0x7e0000000000, batch=1, rows=t.rows, cols=t.cols)
        assert L.gram_ns_batched(ctypes.byref(t), ctypes.byref(o), ctypes.byref(p),
                                 ctypes.c_void_p(0x7f0000000000), 1 << 40, None, None) == -3
    # a grouped query with one oversized group fails as a whole
    G = (ops.MnsTensor * 2)(_t(ops, batch=1, rows=64, cols=64), big)
    assert L.mns_workspace_bytes_grouped(ops.GRAM, 2, G, ctypes.byref(p), ctypes.byref(b)) == -3


def test_argument_errors_return_before_any_hip_call(L):
    from newton_schulz_matrix_muon_amd import ops
    p = ops.ns_params(io_dtype=ops.BF16)
    G = _t(ops, ptr=0x10000)
    O = _t(ops, ptr=0x90000000)
    ws = ctypes.c_void_p(0x7f0000000000)
    call = lambda g, o, pp=p, w=ws, nb=1 << 40: L.gram_ns_batched(
        ctypes.byref(g), ctypes.byref(o), ctypes.byref(pp), w, nb, None, None)
    assert call(G, O, w=None) == -4                                    # no workspace
    assert call(G, O, nb=16) == -4                                     # too small
    assert call(_t(ops, ptr=0), O) == -1                               # null input
    assert call(_t(ops, rows=0), O) == -3                              # empty
    assert call(_t(ops, ld=4), O) == -3                                # ld < cols
    assert call(_t(ops, stride=10), O) == -3                           # stride too small
    assert call(_t(ops, dtype=7), O) == -2                             # unknown dtype
    assert call(G, _t(ops, ptr=0x90000000, dtype=2)) == -2             # out dtype differs
    assert call(G, _t(ops, ptr=0x90000000, cols=15)) == -3             # shape mismatch
    assert call(G, _t(ops, ptr=0x10000 + 64)) == -1                    # overlap
    bad = ops.ns_params(steps=0, io_dtype=ops.BF16)
    assert call(G, O, pp=bad) == -1
    bad = ops.ns_params(io_dtype=ops.BF16, iter_dtype=ops.F32)        # fp32 iterates need fp32 input
    assert call(G, O, pp=bad) == -2
    bad = ops.ns_params(coeffs=[[float("nan"), 0, 0]] * 5, io_dtype=ops.BF16)
    assert call(G, O, pp=bad) == -1
    assert L.mns_last_hip_error() == 0


def test_muon_step_argument_errors(L):
    from newton_schulz_matrix_muon_amd import ops
    p = ops.ns_params(io_dtype=ops.BF16)
    sp = ops.MnsStepParams(0.02, 0.95, 0.01, 0.2, 1, ops.GRAM)
    W = _t(ops, ptr=0x100000)
    G = _t(ops, ptr=0x200000)
    M = _t(ops, ptr=0x300000, dtype=0)
    ws = ctypes.c_void_p(0x7f0000000000)
    f = lambda w=W, g=G, m=M, s=sp, wsp=ws: L.muon_step(
        ctypes.byref(w), ctypes.byref(g), ctypes.byref(m), None, ctypes.byref(s),
        ctypes.byref(p), wsp, 1 << 40, None, None)
    assert f(wsp=None) == -4
    assert f(m=_t(ops, ptr=0x300000, dtype=1)) == -2                  # momentum must be fp32
    assert f(w=_t(ops, ptr=0x100000, rows=9)) == -3
    assert f(g=_t(ops, ptr=0x100000 + 32)) == -1                      # W and G overlap
    assert f(s=ops.MnsStepParams(float("inf"), 0.95, 0.01, 0.2, 1, ops.GRAM)) == -1
    assert f(s=ops.MnsStepParams(0.02, 0.95, 0.01, 0.2, 1, 5)) == -1


def test_gram_trace_argument_errors(L):
    from newton_schulz_matrix_muon_amd import ops
    p = ops.ns_params(io_dtype=ops.F16)
    G = _t(ops, ptr=0x10000, dtype=2)
    O = _t(ops, ptr=0x90000000, dtype=2)
    ws = ctypes.c_void_p(0x7f0000000000)
    tr = ctypes.c_void_p(0x7e0000000000)
    f = lambda g=G, pp=p, t=tr, wsp=ws, nb=1 << 40: L.gram_ns_trace(
        ctypes.byref(g), ctypes.byref(O), ctypes.byref(pp), wsp, nb, t, None)
    assert f(t=None) == -1                                             # no trace buffer
    assert f(pp=ops.ns_params(steps=1, io_dtype=ops.F16)) == -1       # nothing to trace
    assert f(wsp=None) == -4
    assert f(nb=16) == -4
    assert f(g=_t(ops, ptr=0x10000, dtype=1)) == -2                    # O dtype differs
    assert L.mns_last_hip_error() == 0


def test_timing_api_without_launches(L):
    from newton_schulz_matrix_muon_amd import ops
    names = [L.mns_kernel_kind_name(k).decode() for k in range(L.mns_timing_kinds())]
    assert {"gemm_rect", "gemm_symprod", "gemm_syrk", "prep_norm"} <= set(names)
    assert L.mns_kernel_kind_name(99) is None
    ops.timing_reset()
    assert all(v == (0.0, 0) for v in ops.timing_query().values())


def test_grouped_argument_errors(L):
    from newton_schulz_matrix_muon_amd import ops
    p = ops.ns_params(io_dtype=ops.BF16)
    sp = ops.MnsStepParams(0.02, 0.95, 0.01, 0.2, 1, ops.GRAM)
    Ws = ops._tensor_array([_t(ops, ptr=0x100000), _t(ops, ptr=0x400000, rows=16, cols=8)])
    Gs = ops._tensor_array([_t(ops, ptr=0x200000), _t(ops, ptr=0x500000, rows=16, cols=8)])
    Ms = ops._tensor_array([_t(ops, ptr=0x300000, dtype=0), _t(ops, ptr=0x600000, dtype=0, rows=16, cols=8)])
    ws = ctypes.c_void_p(0x7f0000000000)
    f = lambda n=2, w=Ws, g=Gs, m=Ms, wsp=ws: L.muon_step_grouped(
        n, w, g, m, None, ctypes.byref(sp), ctypes.byref(p), wsp, 1 << 40, None, None)
    assert f(n=0) == -1 and f(n=5) == -1                               # 1 .. 4 groups
    assert f(wsp=None) == -4
    W_ov = ops._tensor_array([_t(ops, ptr=0x100000), _t(ops, ptr=0x100000 + 64, rows=16, cols=8)])
    assert f(w=W_ov) == -1                                             # outputs overlap across groups
    G_dt = ops._tensor_array([_t(ops, ptr=0x200000), _t(ops, ptr=0x500000, rows=16, cols=8, dtype=2)])
    W_dt = ops._tensor_array([_t(ops, ptr=0x100000), _t(ops, ptr=0x400000, rows=16, cols=8, dtype=2)])
    assert f(w=W_dt, g=G_dt) == -2                                     # one input dtype for all groups
    Os = ops._tensor_array([_t(ops, ptr=0x900000), _t(ops, ptr=0x200000 + 32, rows=16, cols=8)])
    assert L.gram_ns_grouped(2, Gs, Os, ctypes.byref(p), ws, 1 << 40, None, None) == -1   # output over an input
    assert L.mns_last_hip_error() == 0


def test_grouped_workspace_is_the_sum_of_the_groups(L):
    from newton_schulz_matrix_muon_amd import ops
    p = ops.ns_params(io_dtype=ops.BF16)
    groups = [_t(ops, batch=432, rows=2048, cols=7168), _t(ops, batch=216, rows=7168, cols=2048),
              _t(ops, batch=3, rows=7168, cols=18432)]
    for variant in (ops.STANDARD, ops.GRAM):
        singles = []
        for g in groups:
            b = ctypes.c_size_t()
            assert L.mns_workspace_bytes(variant, ctypes.byref(g), ctypes.byref(p), 0, ctypes.byref(b)) == 0
            singles.append(b.value)
        tot = ctypes.c_size_t()
        assert L.mns_workspace_bytes_grouped(variant, 3, ops._tensor_array(groups), ctypes.byref(p),
                                             ctypes.byref(tot)) == 0
        assert sum(singles) <= tot.value <= sum(singles) + 3 * 256


def test_adamw_argument_errors(L):
    from newton_schulz_matrix_muon_amd import ops
    P = lambda *xs: (ctypes.c_void_p * len(xs))(*xs)
    n = (ctypes.c_int64 * 2)(100, 50)
    ok = ops.MnsAdamwParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1, 0)
    args = [P(0x1000, 0x9000), P(0x2000, 0xa000), P(0x3000, 0xb000), P(0x4000, 0xc000)]
    f = lambda a=args, nn=n, dt=1, ap=ok, nt=2: L.adamw_step(nt, *a, nn, dt, ctypes.byref(ap), None)
    assert f(nt=0) == -1
    assert f(dt=7) == -2
    assert f(ap=ops.MnsAdamwParams(1e-3, 1.0, 0.95, 1e-8, 0.1, 1, 0)) == -1       # beta1 = 1
    assert f(ap=ops.MnsAdamwParams(float("nan"), 0.9, 0.95, 1e-8, 0.1, 1, 0)) == -1
    assert f(ap=ops.MnsAdamwParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 0, 1)) == -1       # step 0 with bias correction
    assert f(a=[P(0x1000, 0x9000), P(0x1000 + 8, 0xa000), P(0x3000, 0xb000), P(0x4000, 0xc000)]) == -1  # p/g overlap
    assert f(a=[P(0x1000, 0), P(0x2000, 0xa000), P(0x3000, 0xb000), P(0x4000, 0xc000)]) == -1            # null
    assert f(nn=(ctypes.c_int64 * 2)(100, -1)) == -1
    assert L.mns_last_hip_error() == 0


def test_noalloc_step_rejects_a_matrix_larger_than_its_scratch(L):
    """muon_step_noalloc checks that one matrix fits the static scratch before any HIP call
    (the pointers here are not device memory): a 7168 x 18432 matrix needs ~1 GB of scratch
    with stabilized Gram NS and is refused; argument errors come first as in muon_step."""
    from newton_schulz_matrix_muon_amd import ops
    p = ops.ns_params(io_dtype=ops.BF16)
    sp = ops.MnsStepParams(0.02, 0.95, 0.01, 0.2, 1, ops.GRAM)
    big = dict(batch=1, rows=7168, cols=18432)
    W = _t(ops, ptr=0x10000000000, **big)
    G = _t(ops, ptr=0x20000000000, **big)
    M = _t(ops, ptr=0x30000000000, dtype=0, **big)
    call = lambda w, g, m, s=sp: L.muon_step_noalloc(ctypes.byref(w), ctypes.byref(g), ctypes.byref(m),
                                                     None, ctypes.byref(s), ctypes.byref(p), None, None)
    assert call(W, G, M) == -4
    assert call(W, G, _t(ops, ptr=0x30000000000, **big)) == -2        # M not fp32
    assert call(W, _t(ops, ptr=0, **big), M) == -1                     # null input
    bad = ops.MnsStepParams(float("inf"), 0.95, 0.01, 0.2, 1, ops.GRAM)
    assert call(W, G, M, bad) == -1
    assert L.mns_last_hip_error() == 0


def test_binding_and_torch_share_one_hip_runtime():
    """Loading the library through the binding, even before the caller imports torch, leaves
    exactly one HIP runtime in the process (torch's), so the library's calls see the device and
    the streams torch uses."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from newton_schulz_matrix_muon_amd import ops\n"
            "ops.lib()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         check=True).stdout
    assert out.strip().splitlines()[-1] == "1"
