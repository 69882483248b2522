"""Host-side checks of the C ABI that need no GPU.

The library must load, export every function include/flce.h declares, and
reject bad arguments before touching a device.
"""
import ctypes
import os
import re

import pytest

import linear_cross_entropy_02_amd as flce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(flce.LIB_PATH):
        pytest.fail("libflce.so is not built (run __graft_entry__.build())")
    return flce.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("flce_create", "flce_fwd_bwd", "flce_destroy", "flce_query_error",
                     "flce_workspace_bytes", "flce_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(flce.EXPORTED) == set(declared_functions())


def test_status_strings(lib):
    for code, name in [(0, "FLCE_OK"), (1, "FLCE_ERR_INVALID_ARGUMENT"), (2, "FLCE_ERR_UNSUPPORTED"),
                       (3, "FLCE_ERR_HIP"), (4, "FLCE_ERR_OUT_OF_MEMORY"), (5, "FLCE_ERR_BAD_TARGET")]:
        assert flce.status_string(code) == name
    assert flce.status_string(99) == "FLCE_ERR_UNKNOWN"


@pytest.mark.parametrize("hidden,vocab,dtype,chunk,dw_chunks", [
    (0, 100, flce.FLCE_BF16, 0, 0),       # H <= 0
    (-8, 100, flce.FLCE_BF16, 0, 0),
    (64, 0, flce.FLCE_BF16, 0, 0),        # V <= 0
    (12, 100, flce.FLCE_BF16, 0, 0),      # H not a multiple of 8 (bf16)
    (6, 100, flce.FLCE_F32, 0, 0),        # H not a multiple of 4 (fp32)
    (64, 100, 7, 0, 0),                   # bad dtype
    (64, 100, flce.FLCE_BF16, -1, 0),     # negative chunk
    (64, 100, flce.FLCE_BF16, 0, -1),     # negative dW group
    (64, 100, flce.FLCE_BF16, 0, 9),      # dW group above 8
])
def test_create_rejects_bad_config_without_device(lib, hidden, vocab, dtype, chunk, dw_chunks):
    st, h = flce.flce_create(hidden, vocab, dtype, chunk, dw_chunks)
    assert st == flce.FLCE_ERR_INVALID_ARGUMENT
    assert not h.value


@pytest.mark.parametrize("hidden,vocab,chunk,dw_chunks", [
    ((1 << 20) + 8, 100, 0, 0),           # H above 2^20
    (64, (1 << 20) + 1, 0, 0),            # padded vocabulary above 2^20
    (64, 100, 1 << 19, 3),                # G x C above 2^20
])
def test_create_reports_unsupported_sizes_without_device(lib, hidden, vocab, chunk, dw_chunks):
    st, h = flce.flce_create(hidden, vocab, flce.FLCE_BF16, chunk, dw_chunks)
    assert st == flce.FLCE_ERR_UNSUPPORTED
    assert not h.value


@pytest.mark.parametrize("hidden,vocab,dtype,flags,status", [
    (64, 100, flce.FLCE_BF16, 8, flce.FLCE_ERR_INVALID_ARGUMENT),          # unknown flag bit
    (64, 100, flce.FLCE_BF16, -1, flce.FLCE_ERR_INVALID_ARGUMENT),
    (64, 100, flce.FLCE_F32, flce.FLCE_FLAG_NO_WEIGHT_COPY, flce.FLCE_ERR_UNSUPPORTED),  # fp32
    # W of 2^31 bytes or more: one buffer descriptor no longer spans it below
    # the out-of-range offset
    (8192, 131072, flce.FLCE_BF16, flce.FLCE_FLAG_NO_WEIGHT_COPY, flce.FLCE_ERR_UNSUPPORTED),
])
def test_create_checks_flags_without_device(lib, hidden, vocab, dtype, flags, status):
    st, h = flce.flce_create(hidden, vocab, dtype, 0, 0, flags)
    assert st == status
    assert not h.value


def test_config_layout_matches_header():
    # the ctypes mirror of flce_config_t: field offsets as C lays them out
    c = flce.flce_config_t
    assert [(n, getattr(c, n).offset) for n, _ in c._fields_] == [
        ("hidden", 0), ("vocab", 8), ("dtype", 16), ("dw_chunks", 20), ("chunk_tokens", 24),
        ("flags", 32)]
    assert ctypes.sizeof(c) == 40


def test_create_null_arguments(lib):
    assert lib.flce_create(None, None) == flce.FLCE_ERR_INVALID_ARGUMENT
    h = ctypes.c_void_p()
    assert lib.flce_create(None, ctypes.byref(h)) == flce.FLCE_ERR_INVALID_ARGUMENT


def test_fwd_bwd_null_handle(lib):
    st = lib.flce_fwd_bwd(None, 16, 16, 16, 4, -100, flce.FLCE_MEAN, 16, 16, 16, None, None,
                          None, None)
    assert st == flce.FLCE_ERR_INVALID_ARGUMENT


def test_misc_null_handle_calls(lib):
    assert lib.flce_destroy(None) == flce.FLCE_OK
    assert lib.flce_workspace_bytes(None) == 0
    assert lib.flce_chunk_tokens(None) == 0
    assert lib.flce_dw_chunks(None) == 0
    assert lib.flce_query_error(None, None, None) == flce.FLCE_ERR_INVALID_ARGUMENT
    assert lib.flce_timing_enable(None, 1) == flce.FLCE_ERR_INVALID_ARGUMENT


def test_timing_kinds(lib):
    kinds = flce.flce_timing_kinds()
    assert "logits_gemm" in kinds and "dx_gemm" in kinds and "dw_gemm" in kinds
    assert lib.flce_timing_kind_name(-1) == b""


def test_library_has_no_undefined_internal_symbols(lib):
    """Every kernel launch stub must be defined in the library itself (a
    kernel template that fails to instantiate in the host pass leaves an
    undefined stub that only shows up when the library is loaded on a GPU)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", flce.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    bad = [l for l in out.splitlines() if "flce" in l]
    assert not bad, bad


def test_autograd_wrapper_refuses_host_tensors():
    """The wrapper has no CPU path: without a HIP device (or given host
    tensors) it raises instead of computing anything on the host."""
    import torch
    from linear_cross_entropy_02_amd.autograd import linear_cross_entropy
    X = torch.zeros(4, 8, dtype=torch.bfloat16, requires_grad=True)
    W = torch.zeros(16, 8, dtype=torch.bfloat16, requires_grad=True)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises((RuntimeError, ValueError, AssertionError)):
        linear_cross_entropy(X, W, y)


@pytest.mark.parametrize("teacher_hidden,status", [
    (0, flce.FLCE_ERR_INVALID_ARGUMENT),
    (-8, flce.FLCE_ERR_INVALID_ARGUMENT),
    (12, flce.FLCE_ERR_INVALID_ARGUMENT),          # not a multiple of 8 (bf16)
    ((1 << 20) + 8, flce.FLCE_ERR_UNSUPPORTED),
])
def test_distill_create_rejects_bad_teacher_without_device(lib, teacher_hidden, status):
    st, h = flce.flce_distill_create(64, 100, flce.FLCE_BF16, teacher_hidden)
    assert st == status and not h.value


def test_distill_null_handle(lib):
    st = lib.flce_distill_fwd_bwd(None, 16, 16, 16, 16, 16, 4, -100, 1.0, flce.FLCE_MEAN, 16, 16,
                                  16, None, None)
    assert st == flce.FLCE_ERR_INVALID_ARGUMENT


def _bare_op(hidden=16, vocab=40):
    """A FusedLinearCrossEntropy without a handle: enough to exercise the
    binding's argument checks, which run before any library call."""
    import torch
    op = object.__new__(flce.FusedLinearCrossEntropy)
    op.hidden, op.vocab, op.torch_dtype, op.handle = hidden, vocab, torch.float32, None
    return op


def test_binding_checks_inputs_before_any_call():
    import torch
    op = _bare_op()
    X, W = torch.zeros(5, 16), torch.zeros(40, 16)
    y = torch.zeros(5, dtype=torch.int64)
    op._check(X, W, y, 5)  # well-formed
    with pytest.raises(ValueError, match="targets"):
        op._check(X, W, torch.zeros(10, dtype=torch.int64)[::2], 5)  # strided view
    with pytest.raises(ValueError, match="targets"):
        op._check(X, W, torch.zeros(5, dtype=torch.int32), 5)
    with pytest.raises(ValueError, match="X must"):
        op._check(torch.zeros(16, 5).t(), W, y, 5)  # not contiguous
    with pytest.raises(ValueError, match="W must"):
        op._check(X, torch.zeros(41, 16), y, 5)
    with pytest.raises(ValueError, match="W must"):
        op._check(X, W.to(torch.float64), y, 5)


def test_binding_checks_output_buffers():
    """A wrongly shaped, typed or strided `out` buffer is refused before the
    library would write its full extent."""
    import torch
    op = _bare_op()
    spec, dev = op._out_spec(5), torch.device("cpu")
    good = dict(loss=torch.zeros(()), dX=torch.zeros(5, 16), dW=torch.zeros(40, 16),
                lse=torch.zeros(5), argmax=torch.zeros(5, dtype=torch.int32),
                n_valid=torch.zeros((), dtype=torch.int64))
    op._check_out(good, spec, dev)
    op._check_out({"loss": good["loss"], "dX": good["dX"], "dW": good["dW"]}, spec, dev)
    for name, bad in (("dW", torch.zeros(39, 16)), ("dX", torch.zeros(5, 16, dtype=torch.float64)),
                      ("lse", torch.zeros(10)[::2]), ("argmax", torch.zeros(5)),
                      ("n_valid", torch.zeros(1, dtype=torch.int64))):
        with pytest.raises(ValueError, match=name):
            op._check_out(dict(good, **{name: bad}), spec, dev)
    with pytest.raises(ValueError, match="on meta"):  # buffers on another device
        op._check_out(good, spec, torch.device("meta"))


def test_noalloc_rejects_without_device(lib):
    # argument and size errors come before any device call
    big = flce.flce_fwd_bwd_noalloc(4096, 128256, flce.FLCE_BF16, 16, 16, 16, 4, -100,
                                    flce.FLCE_MEAN, 16, 16, 16, chunk_tokens=2048, stream=0)
    assert big == flce.FLCE_ERR_UNSUPPORTED
    assert "static scratch" in flce.last_error()
    assert flce.flce_fwd_bwd_noalloc(12, 100, flce.FLCE_BF16, 16, 16, 16, 4, -100,
                                     flce.FLCE_MEAN, 16, 16, 16, stream=0) == \
        flce.FLCE_ERR_INVALID_ARGUMENT                                    # H % 8 != 0
    assert flce.flce_fwd_bwd_noalloc(64, 100, flce.FLCE_BF16, 16, None, 16, 4, -100,
                                     flce.FLCE_MEAN, 16, 16, 16, stream=0) == \
        flce.FLCE_ERR_INVALID_ARGUMENT                                    # W null
    assert flce.flce_fwd_bwd_noalloc(64, 100, flce.FLCE_BF16, 16, 16, 16, 4, -100, 3, 16, 16,
                                     16, stream=0) == flce.FLCE_ERR_INVALID_ARGUMENT
    assert flce.flce_fwd_bwd_noalloc(64, 100, flce.FLCE_BF16, 24, 16, 16, 4, -100,
                                     flce.FLCE_MEAN, 16, 16, 16, stream=0) == \
        flce.FLCE_ERR_INVALID_ARGUMENT                                    # X misaligned
    assert load_null_cfg(lib) == flce.FLCE_ERR_INVALID_ARGUMENT


def load_null_cfg(lib):
    return lib.flce_fwd_bwd_noalloc(None, 16, 16, 16, 4, -100, flce.FLCE_MEAN, 16, 16, 16, None,
                                    None, None, None)


def test_forward_only_flag_is_refused_by_the_soft_target_handle(lib):
    # the soft-target call has no forward-only form: refused before any device call
    st, h = flce.flce_distill_create(64, 100, flce.FLCE_BF16, 64,
                                     flags=flce.FLCE_FLAG_FORWARD_ONLY)
    assert st == flce.FLCE_ERR_INVALID_ARGUMENT and not h.value


def test_noalloc_refuses_a_forward_only_config(lib):
    # the allocation-free call is the fused forward+backward: a forward-only
    # configuration is an argument error, returned before any device call
    dt = flce.FLCE_BF16
    st = flce.flce_fwd_bwd_noalloc(64, 100, dt, 16, 16, 16, 4, -100, flce.FLCE_MEAN, 16, 16, 16,
                                   flags=flce.FLCE_FLAG_FORWARD_ONLY, stream=0)
    assert st == flce.FLCE_ERR_INVALID_ARGUMENT
