"""The C-ABI library without a GPU: it loads, exports every function the header
declares, and rejects bad arguments on the host before any launch.

Every call below fails validation, so nothing reaches the HIP runtime; the
pointers are never dereferenced (fake, but aligned unless the test is about
alignment)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

OK, ENULL, ESHAPE, EDTYPE, EVALUE, EWS, EALIGN, EHIP = range(8)
FAKE = 0x7F0000000000          # 256-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    import draft_verification_vocab_amd as sv
    if not os.path.exists(sv.library_path()):
        from draft_verification_vocab_amd import _build
        _build.build()
    return sv.require_library()


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"SV_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("spec_verify_greedy", "spec_verify_sample", "peagle_build_draft_batch",
              "spec_draft_sample", "spec_verify_mixed", "spec_verify_workspace_bytes",
              "sv_status_string", "spec_accept_metrics", "spec_accept_metrics_words",
              "sv_step_graph_create", "sv_step_graph_launch", "sv_step_graph_destroy",
              "spec_verify_tree", "spec_verify_sample_lq", "spec_verify_sample_noalloc",
              "spec_verify_tree_lq", "spec_verify_mixed_lq",
              "spec_verify_noalloc_scratch_bytes", "spec_verify_greedy_early_exit",
              "spec_verify_sample_early_exit", "spec_verify_mixed_early_exit",
              "spec_verify_sample_lq_early_exit", "spec_verify_mixed_lq_early_exit",
              "spec_verify_tree_early_exit", "spec_verify_tree_lq_early_exit",
              "spec_verify_tree_mixed", "spec_verify_tree_mixed_early_exit"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    import draft_verification_vocab_amd as sv
    out = subprocess.run(["nm", "-D", "--defined-only", sv.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None
    # nothing else leaks out of the C ABI
    assert all(not e.startswith("_ZN2sv") for e in exported)


def test_status_strings(lib):
    for code in range(9):
        s = lib.sv_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.sv_status_string(OK) == b"ok"
    assert lib.sv_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    assert lib.spec_verify_workspace_bytes(0, 7, 100) == 0
    assert lib.spec_verify_workspace_bytes(1, -1, 100) == 0
    assert lib.spec_verify_workspace_bytes(1, 64, 100) == 0
    assert lib.spec_verify_workspace_bytes(1, 3, 0) == 0
    assert lib.spec_verify_workspace_bytes(1, 3, (1 << 19) + 1) == 0
    small = lib.spec_verify_workspace_bytes(1, 3, 32)
    big = lib.spec_verify_workspace_bytes(1024, 7, 151936)
    assert 0 < small < big
    # grows with the batch
    assert lib.spec_verify_workspace_bytes(2048, 7, 151936) > big


def greedy(lib, logits=FAKE, dtype=1, d=FAKE, B=2, K=3, V=64, out=FAKE, acc=FAKE,
           ws=FAKE, wsb=None, err=None):
    if wsb is None:
        wsb = lib.spec_verify_workspace_bytes(max(B, 1), max(K, 0), max(V, 1))
    return lib.spec_verify_greedy(logits, dtype, d, B, K, V, out, acc, ws, wsb, err, None)


def sample(lib, logits=FAKE, dtype=0, q=FAKE, d=FAKE, u=FAKE, T=1.0, B=2, K=3, V=64, out=FAKE,
           acc=FAKE, pd=None, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.spec_verify_workspace_bytes(max(B, 1), max(K, 0), max(V, 1))
    return lib.spec_verify_sample(logits, dtype, q, d, u, T, B, K, V, out, acc, pd, ws, wsb,
                                  None, None)


def test_verify_validation(lib):
    # shapes
    assert greedy(lib, B=-1) == ESHAPE
    assert greedy(lib, K=-1) == ESHAPE
    assert greedy(lib, K=64) == ESHAPE
    assert greedy(lib, V=0) == ESHAPE
    assert greedy(lib, V=(1 << 19) + 1) == ESHAPE
    assert greedy(lib, B=(1 << 20) + 1) == ESHAPE
    # dtype
    assert greedy(lib, dtype=2) == EDTYPE
    assert greedy(lib, dtype=7) == EDTYPE
    # empty batch is a no-op that needs no pointers
    assert greedy(lib, B=0, logits=None, d=None, out=None, acc=None, ws=None, wsb=0) == OK
    # nulls
    assert greedy(lib, logits=None) == ENULL
    assert greedy(lib, d=None) == ENULL
    assert greedy(lib, out=None) == ENULL
    assert greedy(lib, acc=None) == ENULL
    # workspace
    assert greedy(lib, ws=None) == EWS
    assert greedy(lib, wsb=16) == EWS
    # alignment
    assert greedy(lib, logits=FAKE + 1) == EALIGN
    assert greedy(lib, out=FAKE + 2) == EALIGN
    assert greedy(lib, ws=FAKE + 8) == EALIGN
    assert greedy(lib, err=FAKE + 1) == EALIGN
    # sampling: temperature and its extra inputs
    assert sample(lib, T=0.0) == EVALUE
    assert sample(lib, T=-1.0) == EVALUE
    assert sample(lib, T=float("inf")) == EVALUE
    assert sample(lib, T=float("nan")) == EVALUE
    assert sample(lib, T=1e-45) == EVALUE           # log2(e)/T overflows fp32
    # the boundary of that rule: log2(e)/3.5e-39 = 4.1e38 overflows (1/T = 2.9e38
    # would not); log2(e)/4.5e-39 = 3.2e38 is finite (accepted: B = 0 is a no-op)
    assert sample(lib, T=3.5e-39) == EVALUE
    assert sample(lib, B=0, T=4.5e-39, logits=None, q=None, d=None, u=None, out=None, acc=None,
                  ws=None, wsb=0) == OK
    assert sample(lib, q=None) == ENULL
    assert sample(lib, u=None) == ENULL
    assert sample(lib, u=FAKE + 2) == EALIGN
    assert sample(lib, pd=FAKE + 1) == EALIGN
    assert sample(lib, dtype=0, logits=FAKE + 2) == EALIGN      # fp32 needs 4-byte alignment
    assert sample(lib, B=0, T=0.5, logits=None, q=None, d=None, u=None, out=None, acc=None,
                  ws=None, wsb=0) == OK


def build(lib, **kw):
    a = dict(vo=FAKE, acc=FAKE, d=FAKE, L=FAKE, bt=FAKE, maxb=4, bs=16, th=FAKE, hs=FAKE,
             hdt=1, mask=99, B=2, K=3, H=64, ids=FAKE, pos=FAKE, slots=FAKE, hid=FAKE,
             sr=None, err=None)
    a.update(kw)
    return lib.peagle_build_draft_batch(a["vo"], a["acc"], a["d"], a["L"], a["bt"], a["maxb"],
                                        a["bs"], a["th"], a["hs"], a["hdt"], a["mask"], a["B"],
                                        a["K"], a["H"], a["ids"], a["pos"], a["slots"], a["hid"],
                                        a["sr"], a["err"], None)


def test_build_validation(lib):
    assert build(lib, K=0) == ESHAPE
    assert build(lib, K=64) == ESHAPE
    assert build(lib, H=0) == ESHAPE
    assert build(lib, bs=0) == ESHAPE
    assert build(lib, maxb=0) == ESHAPE
    assert build(lib, B=-3) == ESHAPE
    assert build(lib, hdt=5) == EDTYPE
    assert build(lib, B=0, vo=None, acc=None) == OK
    for k in ("vo", "acc", "d", "L", "bt", "th", "hs", "ids", "pos", "slots", "hid"):
        assert build(lib, **{k: None}) == ENULL, k
    assert build(lib, L=FAKE + 4) == EALIGN            # int64 needs 8 bytes
    assert build(lib, pos=FAKE + 4) == EALIGN
    assert build(lib, slots=FAKE + 4) == EALIGN
    assert build(lib, th=FAKE + 1) == EALIGN
    assert build(lib, hdt=0, hid=FAKE + 2) == EALIGN   # fp32 hidden needs 4 bytes
    assert build(lib, sr=FAKE + 2) == EALIGN


def test_binding_refuses_cpu_tensors(lib):
    import torch
    import draft_verification_vocab_amd as sv
    z = torch.zeros(1, 4, 32)
    d = torch.zeros(1, 3, dtype=torch.int32)
    with pytest.raises(ValueError):
        sv.spec_verify_greedy(z, d)


def test_tracer_host_paths(lib):
    import ctypes
    assert lib.sv_trace_begin(0, 0xFFFFFFFF) == EVALUE      # rejected before any HIP call
    assert lib.sv_trace_begin(-4, 1) == EVALUE
    assert lib.sv_trace_count() == 0
    kid, ms = ctypes.c_int(), ctypes.c_float()
    assert lib.sv_trace_read(0, ctypes.byref(kid), ctypes.byref(ms)) == EVALUE
    assert lib.sv_trace_read(0, None, None) == ENULL
    import draft_verification_vocab_amd as sv
    assert all(lib.sv_kernel_name(i).decode() == n for n, i in sv.KERNEL_IDS.items())
    names = [lib.sv_kernel_name(i) for i in range(11)]
    assert names == [b"verify_greedy_rows", b"verify_sample_rows", b"verify_sample_draw",
                     b"peagle_build", b"verify_greedy_accept", b"verify_sample_locate",
                     b"draft_sample", b"verify_mixed_rows", b"accept_metrics", b"tree_rows",
                     b"tree_walk"]
    assert lib.sv_kernel_name(11) == b"unknown"
    assert lib.sv_kernel_name(17) == b"unknown"
    lib.sv_trace_enable(1)                          # no trace active: nothing happens
    lib.sv_trace_enable(0)
    assert lib.sv_trace_count() == 0
    lib.sv_trace_end()                              # harmless when tracing is off


def draft(lib, logits=FAKE, dtype=1, n_rows=6, ri=None, u=FAKE, T=0.7, temps=None, B=2, K=3,
          V=64, tok=FAKE, probs=FAKE, desc=None, err=None):
    return lib.spec_draft_sample(logits, dtype, n_rows, ri, u, T, temps, B, K, V, tok, probs,
                                 desc, err, None)


def test_draft_validation(lib):
    assert draft(lib, K=0) == ESHAPE
    assert draft(lib, K=64) == ESHAPE
    assert draft(lib, V=0) == ESHAPE
    assert draft(lib, V=(1 << 19) + 1) == ESHAPE
    assert draft(lib, B=-1) == ESHAPE
    assert draft(lib, n_rows=5) == ESHAPE             # fewer than B*K rows and no row index
    assert draft(lib, n_rows=-1, ri=FAKE) == ESHAPE
    assert draft(lib, dtype=2) == EDTYPE
    for T in (-0.5, float("inf"), float("nan"), 1e-45):
        assert draft(lib, T=T) == EVALUE, T
    assert draft(lib, B=0, logits=None, u=None, tok=None, probs=None) == OK
    assert draft(lib, logits=None) == ENULL
    assert draft(lib, tok=None) == ENULL
    assert draft(lib, u=None) == ENULL                 # sampled rows need uniforms
    assert draft(lib, u=None, T=0.0, temps=FAKE) == ENULL
    assert draft(lib, logits=FAKE + 1) == EALIGN
    assert draft(lib, dtype=0, logits=FAKE + 2) == EALIGN
    assert draft(lib, ri=FAKE + 2) == EALIGN
    assert draft(lib, u=FAKE + 1) == EALIGN
    assert draft(lib, temps=FAKE + 2) == EALIGN
    assert draft(lib, probs=FAKE + 2) == EALIGN
    assert draft(lib, tok=FAKE + 1) == EALIGN
    assert draft(lib, err=FAKE + 1) == EALIGN
    assert draft(lib, desc=FAKE + 8) == EALIGN        # descriptors are 16-byte records


def mixed(lib, logits=FAKE, dtype=1, q=FAKE, d=FAKE, u=FAKE, temps=FAKE, B=2, K=3, V=64,
          out=FAKE, acc=FAKE, pd=None, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.spec_verify_workspace_bytes(max(B, 1), max(K, 0), max(V, 1))
    return lib.spec_verify_mixed(logits, dtype, q, d, u, temps, B, K, V, out, acc, pd, ws, wsb,
                                 None, None)


def test_mixed_validation(lib):
    assert mixed(lib, K=64) == ESHAPE
    assert mixed(lib, V=0) == ESHAPE
    assert mixed(lib, dtype=2) == EDTYPE
    assert mixed(lib, B=0, logits=None, q=None, d=None, u=None, temps=None, out=None, acc=None,
                 ws=None, wsb=0) == OK
    assert mixed(lib, temps=None) == ENULL
    assert mixed(lib, q=None) == ENULL
    assert mixed(lib, u=None) == ENULL
    assert mixed(lib, temps=FAKE + 2) == EALIGN
    assert mixed(lib, ws=None) == EWS
    assert mixed(lib, wsb=8) == EWS


def test_metrics_and_graph_validation(lib):
    assert lib.spec_accept_metrics_words(0) == 0
    assert lib.spec_accept_metrics_words(64) == 0
    assert lib.spec_accept_metrics_words(7) == 5 + 8
    am = lambda na=FAKE, B=4, K=7, m=FAKE, err=None: lib.spec_accept_metrics(na, B, K, m, err, None)
    assert am(B=-1) == ESHAPE
    assert am(K=0) == ESHAPE
    assert am(K=64) == ESHAPE
    assert am(B=0, na=None, m=None) == OK
    assert am(na=None) == ENULL
    assert am(m=None) == ENULL
    assert am(m=FAKE + 4) == EALIGN
    assert am(na=FAKE + 2) == EALIGN
    # graph: argument checks that come before any HIP call
    import draft_verification_vocab_amd as sv
    g = ctypes.c_void_p()
    assert lib.sv_step_graph_create(None, ctypes.byref(g)) == ENULL
    d = sv._StepDesc()
    assert lib.sv_step_graph_create(ctypes.byref(d), None) == ENULL
    d.mode = 7
    assert lib.sv_step_graph_create(ctypes.byref(d), ctypes.byref(g)) == EVALUE
    d.mode, d.metrics, d.K = 1, FAKE, 0
    assert lib.sv_step_graph_create(ctypes.byref(d), ctypes.byref(g)) == ESHAPE
    # q from drafter logits: sampling only, and never beside a dense q
    d.metrics, d.K, d.drafter_logits = None, 3, FAKE
    d.mode, d.draft_probs = 0, None
    assert lib.sv_step_graph_create(ctypes.byref(d), ctypes.byref(g)) == EVALUE
    d.mode, d.draft_probs = 2, FAKE
    assert lib.sv_step_graph_create(ctypes.byref(d), ctypes.byref(g)) == EVALUE
    assert lib.sv_step_graph_launch(None, None) == ENULL
    lib.sv_step_graph_destroy(None)


def test_step_desc_layout_matches_header():
    """The ctypes mirror of sv_step_desc has the C struct's size and offsets:
    compile a probe with the host compiler that prints them."""
    import shutil
    import tempfile
    import draft_verification_vocab_amd as sv
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = [f for f, _ in sv._StepDesc._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"spec_verify.h\"\nint main(void){\n"
    src += 'printf("%zu\\n", sizeof(sv_step_desc));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof(sv_step_desc, {f}));\n'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as t:
        c = os.path.join(t, "probe.c")
        exe = os.path.join(t, "probe")
        open(c, "w").write(src)
        subprocess.run([cc, "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        out = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                              check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(sv._StepDesc)
    assert out[1:] == [getattr(sv._StepDesc, f).offset for f in fields]


def tree(lib, logits=FAKE, dtype=1, q=FAKE, par=FAKE, tok=FAKE, u=FAKE, T=0.7, B=2, N=6, V=64,
         out=FAKE, path=FAKE, acc=FAKE, ws=FAKE, wsb=None, fn="spec_verify_tree"):
    if wsb is None:
        wsb = lib.spec_verify_workspace_bytes(max(B, 1), max(N, 0), max(V, 1))
    return getattr(lib, fn)(logits, dtype, q, par, tok, u, T, B, N, V, out, path, acc, ws, wsb,
                            None, None)


@pytest.mark.parametrize("fn", ["spec_verify_tree", "spec_verify_tree_early_exit"])
def test_tree_validation(lib, fn):
    import functools
    _tree_cases(lib, functools.partial(tree, fn=fn))


def _tree_cases(lib, tree):
    assert tree(lib, N=64) == ESHAPE
    assert tree(lib, N=-1) == ESHAPE
    assert tree(lib, V=0) == ESHAPE
    assert tree(lib, dtype=2) == EDTYPE
    for T in (-1.0, float("nan"), float("inf"), 1e-45):
        assert tree(lib, T=T) == EVALUE, T
    assert tree(lib, B=0, logits=None, q=None, par=None, tok=None, u=None, out=None, path=None,
                acc=None, ws=None, wsb=0) == OK
    assert tree(lib, par=None) == ENULL
    assert tree(lib, path=None) == ENULL
    assert tree(lib, q=None) == ENULL              # sampled trees need draft probs
    assert tree(lib, u=None) == ENULL
    assert tree(lib, ws=None) == EWS
    assert tree(lib, wsb=8) == EWS
    assert tree(lib, par=FAKE + 2) == EALIGN
    assert tree(lib, dtype=0, logits=FAKE + 2) == EALIGN


def lq(lib, logits=FAKE, dtype=1, dl=FAKE, n_rows=6, rows=None, desc=FAKE, d=FAKE, u=FAKE, T=0.7,
       B=2, K=3, V=64, out=FAKE, acc=FAKE, pd=None, ws=FAKE, wsb=None,
       fn="spec_verify_sample_lq"):
    if wsb is None:
        wsb = lib.spec_verify_workspace_bytes(max(B, 1), max(K, 0), max(V, 1))
    return getattr(lib, fn)(logits, dtype, dl, n_rows, rows, desc, d, u, T, B, K, V, out, acc, pd,
                            ws, wsb, None, None)


@pytest.mark.parametrize("fn", ["spec_verify_sample_lq", "spec_verify_sample_lq_early_exit"])
def test_sample_lq_validation(lib, fn):
    import functools
    lq_ = functools.partial(lq, fn=fn)
    _sample_lq_cases(lib, lq_)


def _sample_lq_cases(lib, lq):
    assert lq(lib, K=64) == ESHAPE
    assert lq(lib, n_rows=5) == ESHAPE                 # fewer than B*K rows, no row index
    assert lq(lib, n_rows=-1, rows=FAKE) == ESHAPE
    assert lq(lib, dtype=2) == EDTYPE
    for T in (0.0, -1.0, float("nan"), 1e-45):
        assert lq(lib, T=T) == EVALUE, T
    assert lq(lib, B=0, logits=None, dl=None, desc=None, d=None, u=None, out=None, acc=None,
              ws=None, wsb=0) == OK
    assert lq(lib, dl=None) == ENULL
    assert lq(lib, desc=None) == ENULL
    assert lq(lib, u=None) == ENULL
    assert lq(lib, ws=None) == EWS
    assert lq(lib, desc=FAKE + 8) == EALIGN
    assert lq(lib, dl=FAKE + 1) == EALIGN
    assert lq(lib, rows=FAKE + 2) == EALIGN


def mixed_lq(lib, logits=FAKE, dtype=1, dl=FAKE, n_rows=6, rows=None, desc=FAKE, d=FAKE, u=FAKE,
             temps=FAKE, B=2, K=3, V=64, out=FAKE, acc=FAKE, pd=None, ws=FAKE, wsb=None,
             fn="spec_verify_mixed_lq"):
    if wsb is None:
        wsb = lib.spec_verify_workspace_bytes(max(B, 1), max(K, 0), max(V, 1))
    return getattr(lib, fn)(logits, dtype, dl, n_rows, rows, desc, d, u, temps, B, K, V, out, acc,
                            pd, ws, wsb, None, None)


@pytest.mark.parametrize("fn", ["spec_verify_mixed_lq", "spec_verify_mixed_lq_early_exit"])
def test_mixed_lq_validation(lib, fn):
    import functools
    _mixed_lq_cases(lib, functools.partial(mixed_lq, fn=fn))


def _mixed_lq_cases(lib, mixed_lq):
    assert mixed_lq(lib, K=64) == ESHAPE
    assert mixed_lq(lib, n_rows=5) == ESHAPE             # fewer than B*K rows, no row index
    assert mixed_lq(lib, dtype=2) == EDTYPE
    assert mixed_lq(lib, temps=None) == ENULL            # per-sequence temperatures required
    assert mixed_lq(lib, B=0, logits=None, dl=None, desc=None, d=None, u=None, temps=None,
                    out=None, acc=None, ws=None, wsb=0) == OK
    assert mixed_lq(lib, dl=None) == ENULL
    assert mixed_lq(lib, desc=None) == ENULL
    assert mixed_lq(lib, ws=None) == EWS
    assert mixed_lq(lib, temps=FAKE + 2) == EALIGN
    assert mixed_lq(lib, desc=FAKE + 8) == EALIGN


def tree_lq(lib, logits=FAKE, dtype=1, dl=FAKE, n_rows=14, rows=None, desc=FAKE, par=FAKE,
            tok=FAKE, u=FAKE, T=0.7, B=2, N=6, V=64, out=FAKE, path=FAKE, acc=FAKE, ws=FAKE,
            wsb=None, fn="spec_verify_tree_lq"):
    if wsb is None:
        wsb = lib.spec_verify_workspace_bytes(max(B, 1), max(N, 0), max(V, 1))
    return getattr(lib, fn)(logits, dtype, dl, n_rows, rows, desc, par, tok, u, T, B, N, V, out,
                            path, acc, ws, wsb, None, None)


@pytest.mark.parametrize("fn", ["spec_verify_tree_lq", "spec_verify_tree_lq_early_exit"])
def test_tree_lq_validation(lib, fn):
    import functools
    _tree_lq_cases(lib, functools.partial(tree_lq, fn=fn))


def _tree_lq_cases(lib, tree_lq):
    assert tree_lq(lib, N=64) == ESHAPE
    assert tree_lq(lib, n_rows=13) == ESHAPE            # fewer than B*(N+1) rows, no row index
    assert tree_lq(lib, n_rows=-1, rows=FAKE) == ESHAPE
    # a row index may name any row count (the call then stops at the workspace)
    assert tree_lq(lib, n_rows=3, rows=FAKE, ws=None) == EWS
    assert tree_lq(lib, dtype=2) == EDTYPE
    for T in (0.0, -1.0, float("nan"), 1e-45):          # sampling only
        assert tree_lq(lib, T=T) == EVALUE, T
    assert tree_lq(lib, B=0, logits=None, dl=None, desc=None, par=None, tok=None, u=None,
                   out=None, path=None, acc=None, ws=None, wsb=0) == OK
    assert tree_lq(lib, dl=None) == ENULL
    assert tree_lq(lib, desc=None) == ENULL
    assert tree_lq(lib, u=None) == ENULL
    assert tree_lq(lib, par=None) == ENULL
    assert tree_lq(lib, N=0, par=None, tok=None, ws=None) == EWS   # a root alone needs no nodes
    assert tree_lq(lib, ws=None) == EWS
    assert tree_lq(lib, desc=FAKE + 8) == EALIGN
    assert tree_lq(lib, dl=FAKE + 1) == EALIGN
    assert tree_lq(lib, rows=FAKE + 2) == EALIGN


ESCRATCH = 8


def noalloc(lib, logits=FAKE, dtype=1, q=FAKE, d=FAKE, u=FAKE, T=1.0, B=2, K=3, V=64, out=FAKE,
            acc=FAKE, pd=None, err=None):
    return lib.spec_verify_sample_noalloc(logits, dtype, q, d, u, T, B, K, V, out, acc, pd, err,
                                          None)


def test_noalloc_validation(lib):
    """The no-allocation sampled verify checks its arguments as spec_verify_sample
    does, and rejects a call whose workspace would exceed its fixed scratch, all
    before any HIP call (none of these reach the GPU)."""
    assert lib.spec_verify_noalloc_scratch_bytes() == 8 << 20
    assert noalloc(lib, B=-1) == ESHAPE
    assert noalloc(lib, V=0) == ESHAPE
    assert noalloc(lib, dtype=2) == EDTYPE
    assert noalloc(lib, logits=None) == ENULL
    assert noalloc(lib, q=None) == ENULL
    assert noalloc(lib, u=None) == ENULL
    assert noalloc(lib, out=None) == ENULL
    assert noalloc(lib, T=0.0) == EVALUE
    assert noalloc(lib, T=3.5e-39) == EVALUE
    assert noalloc(lib, logits=FAKE + 1) == EALIGN
    assert noalloc(lib, pd=FAKE + 2) == EALIGN
    assert noalloc(lib, B=0, logits=None, q=None, d=None, u=None, out=None, acc=None) == OK
    # the largest batch at K=7, V=151936 whose workspace fits, and the next one
    cap = lib.spec_verify_noalloc_scratch_bytes()
    lo, hi = 1, 1 << 20
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if lib.spec_verify_workspace_bytes(mid, 7, 151936) <= cap:
            lo = mid
        else:
            hi = mid
    assert lib.spec_verify_workspace_bytes(lo, 7, 151936) <= cap
    assert lo >= 4096                     # far above the 1024-sequence serving batch
    assert noalloc(lib, B=hi, K=7, V=151936) == ESCRATCH
    assert lib.sv_status_string(ESCRATCH).startswith(b"call needs more scratch")


def test_early_exit_validation(lib):
    """The early-exit forms validate exactly as the full calls, before any
    launch (every case here is an error or an empty batch)."""
    def g(**kw):
        a = dict(logits=FAKE, dtype=1, d=FAKE, B=2, K=3, V=64, out=FAKE, acc=FAKE, ws=FAKE,
                 wsb=None, err=None)
        a.update(kw)
        wsb = a["wsb"] if a["wsb"] is not None else lib.spec_verify_workspace_bytes(
            max(a["B"], 1), max(a["K"], 0), max(a["V"], 1))
        return lib.spec_verify_greedy_early_exit(a["logits"], a["dtype"], a["d"], a["B"], a["K"],
                                                 a["V"], a["out"], a["acc"], a["ws"], wsb,
                                                 a["err"], None)

    def s(fn, **kw):
        a = dict(logits=FAKE, dtype=0, q=FAKE, d=FAKE, u=FAKE, T=1.0, temps=FAKE, B=2, K=3, V=64,
                 out=FAKE, acc=FAKE, pd=None, ws=FAKE, wsb=None)
        a.update(kw)
        wsb = a["wsb"] if a["wsb"] is not None else lib.spec_verify_workspace_bytes(
            max(a["B"], 1), max(a["K"], 0), max(a["V"], 1))
        if fn == "sample":
            return lib.spec_verify_sample_early_exit(a["logits"], a["dtype"], a["q"], a["d"],
                                                     a["u"], a["T"], a["B"], a["K"], a["V"],
                                                     a["out"], a["acc"], a["pd"], a["ws"], wsb,
                                                     None, None)
        return lib.spec_verify_mixed_early_exit(a["logits"], a["dtype"], a["q"], a["d"], a["u"],
                                                a["temps"], a["B"], a["K"], a["V"], a["out"],
                                                a["acc"], a["pd"], a["ws"], wsb, None, None)

    assert g(B=-1) == ESHAPE and g(K=64) == ESHAPE and g(V=0) == ESHAPE
    assert g(dtype=2) == EDTYPE
    assert g(B=0, logits=None, d=None, out=None, acc=None, ws=None, wsb=0) == OK
    assert g(logits=None) == ENULL and g(d=None) == ENULL and g(acc=None) == ENULL
    assert g(ws=None) == EWS and g(wsb=16) == EWS
    assert g(logits=FAKE + 1) == EALIGN and g(err=FAKE + 1) == EALIGN
    for fn in ("sample", "mixed"):
        assert s(fn, B=-1) == ESHAPE and s(fn, K=64) == ESHAPE
        assert s(fn, dtype=5) == EDTYPE
        assert s(fn, q=None) == ENULL and s(fn, u=None) == ENULL
        assert s(fn, wsb=16) == EWS
        assert s(fn, q=FAKE + 2) == EALIGN and s(fn, pd=FAKE + 1) == EALIGN
    assert s("sample", T=0.0) == EVALUE and s("sample", T=float("nan")) == EVALUE
    assert s("mixed", temps=None) == ENULL and s("mixed", temps=FAKE + 2) == EALIGN


@pytest.mark.parametrize("fn", ["spec_verify_tree_mixed", "spec_verify_tree_mixed_early_exit"])
def test_tree_mixed_validation(lib, fn):
    def tm(logits=FAKE, dtype=1, q=FAKE, par=FAKE, tok=FAKE, u=FAKE, temps=FAKE, B=2, N=6, V=64,
           out=FAKE, path=FAKE, acc=FAKE, ws=FAKE, wsb=None):
        if wsb is None:
            wsb = lib.spec_verify_workspace_bytes(max(B, 1), max(N, 0), max(V, 1))
        return getattr(lib, fn)(logits, dtype, q, par, tok, u, temps, B, N, V, out, path, acc, ws,
                                wsb, None, None)
    assert tm(N=64) == ESHAPE and tm(V=0) == ESHAPE
    assert tm(dtype=2) == EDTYPE
    assert tm(temps=None) == ENULL                      # per-tree temperatures required
    assert tm(B=0, logits=None, q=None, par=None, tok=None, u=None, temps=None, out=None,
              path=None, acc=None, ws=None, wsb=0) == OK
    assert tm(q=None) == ENULL and tm(u=None) == ENULL and tm(par=None) == ENULL
    assert tm(ws=None) == EWS
    assert tm(temps=FAKE + 2) == EALIGN and tm(q=FAKE + 1) == EALIGN
