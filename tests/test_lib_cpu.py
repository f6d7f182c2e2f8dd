"""libfa on the CPU: the shared library loads, exports every symbol of include/fa.h, and rejects
bad arguments before touching the GPU (no kernel is launched in this file)."""

import ctypes
import os
import re

import pytest

import io_aware_exact_23_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

needs_lib = pytest.mark.skipif(not os.path.exists(fa.library_path()),
                               reason="libfa.so not built (run python -m io_aware_exact_23_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == ["fa_build_info", "fa_bwd", "fa_fp8_vt_cols", "fa_fwd", "fa_fwd_f32", "fa_fwd_fp8",
                                    "fa_fwd_noalloc", "fa_fwd_varlen", "fa_fwd_window", "fa_last_error",
                                    "fa_quantize_fp8", "fa_status_string", "fa_std_fwd",
                                    "fa_std_workspace_bytes"]


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


@needs_lib
def test_build_info_names_compiler_and_target():
    info = fa.fa_build_info()
    assert "clang" in info and "gfx950" in info and "HIP headers" in info


@needs_lib
def test_status_strings():
    for st in (0, -1, -2, -3):
        assert fa.fa_status_string(st).startswith(("FA_OK", "FA_ERR"))
    assert fa.fa_status_string(7) == "unknown fa status"


# Fake device addresses: argument checks must reject these calls before any HIP call.
A = 0x10000000
BAD = 0x10000001
INT_MAX = 2 ** 31 - 1

# The host-sanitizer test (test_host_sanitizers.py) reruns this file against a build of the library
# whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer checks (FA_TEST_LIBRARY,
# applied in conftest.py).


def _std(**kw):
    """fa_std_fwd with the fa_fwd keyword set plus a (fake) large enough workspace."""
    ws = kw.pop("workspace", A)
    wb = kw.pop("workspace_bytes", 1 << 40)
    fa.fa_std_fwd(workspace=ws, workspace_bytes=wb, **kw)


def _win(**kw):
    """fa_fwd_window with the fa_fwd keyword set: causal=1 becomes the window (-1, 0)."""
    causal = kw.pop("causal")
    if causal not in (0, 1):
        pytest.skip("the window entry point has no causal flag")
    fa.fa_fwd_window(window_left=-1, window_right=0 if causal else -1, **kw)


ENTRY = {"fa_fwd": lambda **kw: fa.fa_fwd(**kw), "fa_fwd_f32": lambda **kw: fa.fa_fwd_f32(**kw),
         "fa_fwd_noalloc": lambda **kw: fa.fa_fwd_noalloc(**kw),
         "fa_std_fwd": _std, "fa_fwd_window": _win}


@needs_lib
@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32", "fa_std_fwd", "fa_fwd_window", "fa_fwd_noalloc"])
@pytest.mark.parametrize("args,status,needle", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED, "64 or 128"),
    (dict(d=0), fa.FA_ERR_UNSUPPORTED, "64 or 128"),
    (dict(B=-1), fa.FA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(Nk=-3), fa.FA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARGUMENT, "finite"),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARGUMENT, "finite"),
    (dict(causal=2), fa.FA_ERR_INVALID_ARGUMENT, "causal"),
    (dict(causal=1, Nq=4, Nk=5), fa.FA_ERR_UNSUPPORTED, "Nq == Nk"),
    (dict(q=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(lse=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(k=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(q=BAD), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(v=A + 8), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(lse=A + 2), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(kv_seqlens=A + 1), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(B=70000, H=70000), fa.FA_ERR_UNSUPPORTED, "int32"),
    (dict(Nk=1 << 23, d=128), fa.FA_ERR_UNSUPPORTED, "2^31 bytes"),
    (dict(Nq=1 << 23, Nk=1 << 23, d=128, causal=1), fa.FA_ERR_UNSUPPORTED, "2^31 bytes"),
    (dict(Nq=INT_MAX, Nk=INT_MAX), fa.FA_ERR_UNSUPPORTED, "2^31 bytes"),
    (dict(B=INT_MAX, H=INT_MAX), fa.FA_ERR_UNSUPPORTED, "int32"),
    (dict(B=-INT_MAX - 1), fa.FA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(scale=-float("inf")), fa.FA_ERR_INVALID_ARGUMENT, "finite"),
])
def test_argument_errors(fn, args, status, needle):
    call = dict(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, Nq=8, Nk=8, d=64, scale=0.125, causal=0,
                kv_seqlens=None, stream=0)
    call.update(args)
    with pytest.raises(fa.FaError) as ei:
        ENTRY[fn](**call)
    assert ei.value.status == status
    assert needle in ei.value.message


@needs_lib
@pytest.mark.parametrize("args,needle", [
    (dict(workspace=None), "non-null"),
    (dict(workspace=A + 128), "256-byte aligned"),
    (dict(workspace_bytes=2 * 3 * 8 * 128 * 6 - 1), "smaller"),
])
def test_standard_workspace_errors(args, needle):
    # B=2, H=3, Nq=8, Nk=8: S and P rows are padded to 128 keys, 6 bytes per entry.
    call = dict(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, Nq=8, Nk=8, d=64, scale=0.125, causal=0,
                kv_seqlens=None, stream=0)
    call.update(args)
    with pytest.raises(fa.FaError) as ei:
        _std(**call)
    assert ei.value.status == fa.FA_ERR_INVALID_ARGUMENT
    assert needle in ei.value.message


@needs_lib
def test_standard_workspace_size():
    assert fa.fa_std_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, INT_MAX) == 0  # would not fit in size_t
    assert fa.fa_std_workspace_bytes(2, 3, 8, 8) == 2 * 3 * 8 * 128 * 6
    assert fa.fa_std_workspace_bytes(1, 1, 1, 129) == 256 * 6
    assert fa.fa_std_workspace_bytes(2, 16, 16384, 16384) == 2 * 16 * 16384 * 16384 * 6
    for args in [(0, 1, 1, 1), (1, 0, 1, 1), (1, 1, 0, 1), (1, 1, 1, 0), (-1, 1, 1, 1)]:
        assert fa.fa_std_workspace_bytes(*args) == 0


@needs_lib
def test_standard_rejects_a_head_too_large():
    with pytest.raises(fa.FaError) as ei:
        _std(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, Nq=32768, Nk=32768, d=64, scale=0.1, causal=0,
             kv_seqlens=None, stream=0)
    assert ei.value.status == fa.FA_ERR_UNSUPPORTED


@needs_lib
@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32", "fa_std_fwd", "fa_fwd_window"])
@pytest.mark.parametrize("args", [dict(B=0), dict(H=0), dict(Nq=0), dict(B=0, q=None, o=None, lse=None)])
def test_empty_batch_is_a_no_op(fn, args):
    call = dict(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, Nq=8, Nk=8, d=128, scale=0.1, causal=0,
                kv_seqlens=None, stream=0)
    call.update(args)
    ENTRY[fn](**call)  # returns FA_OK without launching anything
    assert fa.fa_last_error() == ""


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(fa.FaError):
        fa.fa_status_string(0)


@needs_lib
@pytest.mark.parametrize("args,status,needle", [
    (dict(window_left=-2), fa.FA_ERR_INVALID_ARGUMENT, ">= -1"),
    (dict(window_right=-5), fa.FA_ERR_INVALID_ARGUMENT, ">= -1"),
    (dict(window_left=3, Nq=4, Nk=6), fa.FA_ERR_UNSUPPORTED, "Nq == Nk"),
    (dict(window_right=0, Nq=4, Nk=6), fa.FA_ERR_UNSUPPORTED, "Nq == Nk"),
])
def test_window_argument_errors(args, status, needle):
    call = dict(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, Nq=8, Nk=8, d=64, scale=0.125, window_left=-1,
                window_right=-1, kv_seqlens=None, stream=0)
    call.update(args)
    with pytest.raises(fa.FaError) as ei:
        fa.fa_fwd_window(**call)
    assert ei.value.status == status
    assert needle in ei.value.message


VARLEN = dict(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, total_q=40, total_k=50, max_seqlen_q=30, d=128,
              scale=0.1, window_left=-1, window_right=0, cu_seqlens_q=A, cu_seqlens_k=A, stream=0)


@needs_lib
@pytest.mark.parametrize("args,status,needle", [
    (dict(d=80), fa.FA_ERR_UNSUPPORTED, "64 or 128"),
    (dict(B=-1), fa.FA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(total_k=-1), fa.FA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(window_left=-3), fa.FA_ERR_INVALID_ARGUMENT, ">= -1"),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARGUMENT, "finite"),
    (dict(cu_seqlens_q=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(cu_seqlens_k=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(lse=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(v=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(q=A + 8), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(cu_seqlens_k=A + 2), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(total_q=1 << 24), fa.FA_ERR_UNSUPPORTED, "2^31"),
    (dict(max_seqlen_q=INT_MAX, B=INT_MAX, H=2), fa.FA_ERR_UNSUPPORTED, "grid too large"),
    (dict(max_seqlen_q=INT_MAX, B=1, H=INT_MAX), fa.FA_ERR_UNSUPPORTED, "grid too large"),
])
def test_varlen_argument_errors(args, status, needle):
    call = dict(VARLEN)
    call.update(args)
    with pytest.raises(fa.FaError) as ei:
        fa.fa_fwd_varlen(**call)
    assert ei.value.status == status
    assert needle in ei.value.message


@needs_lib
@pytest.mark.parametrize("args", [dict(B=0), dict(H=0), dict(total_q=0), dict(max_seqlen_q=0),
                                  dict(B=0, q=None, o=None, lse=None, cu_seqlens_q=None)])
def test_varlen_empty_is_a_no_op(args):
    call = dict(VARLEN)
    call.update(args)
    fa.fa_fwd_varlen(**call)
    assert fa.fa_last_error() == ""


BWD = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, B=2, H=3, Nq=8, Nk=8, d=64,
           scale=0.125, causal=0, kv_seqlens=None, stream=0)


@needs_lib
@pytest.mark.parametrize("args,status,needle", [
    (dict(d=32), fa.FA_ERR_UNSUPPORTED, "64 or 128"),
    (dict(Nk=-1), fa.FA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(causal=1, Nq=4, Nk=5), fa.FA_ERR_UNSUPPORTED, "Nq == Nk"),
    (dict(dout=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(dq=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(dk=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(dv=A + 4), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(dout=A + 8), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARGUMENT, "finite"),
    (dict(Nq=0, dk=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(Nq=0, k=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(Nq=0, v=A + 8), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(Nq=0, kv_seqlens=A + 2), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(Nq=1 << 24, d=64), fa.FA_ERR_UNSUPPORTED, "2^31 bytes"),
    (dict(B=INT_MAX, H=INT_MAX), fa.FA_ERR_UNSUPPORTED, "int32"),
    (dict(Nq=INT_MAX, Nk=1), fa.FA_ERR_UNSUPPORTED, "2^31 bytes"),
])
def test_backward_argument_errors(args, status, needle):
    call = dict(BWD)
    call.update(args)
    with pytest.raises(fa.FaError) as ei:
        fa.fa_bwd(**call)
    assert ei.value.status == status
    assert needle in ei.value.message


@needs_lib
@pytest.mark.parametrize("args", [dict(B=0), dict(H=0), dict(Nq=0, Nk=0)])
def test_backward_empty_is_a_no_op(args):
    call = dict(BWD)
    call.update(args)
    fa.fa_bwd(**call)
    assert fa.fa_last_error() == ""


FP8 = dict(q8=A, k8=A, vt8=A, descale_q=A, descale_k=A, descale_v=A, o=A, lse=A, B=2, H=3, Nq=8,
           Nk=8, d=64, scale=0.125, causal=0, kv_seqlens=None, stream=0)


@needs_lib
@pytest.mark.parametrize("args,status,needle", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED, "64 or 128"),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(causal=1, Nq=4, Nk=5), fa.FA_ERR_UNSUPPORTED, "Nq == Nk"),
    (dict(causal=2), fa.FA_ERR_INVALID_ARGUMENT, "0 or 1"),
    (dict(q8=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(vt8=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(vt8=A + 8), fa.FA_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(descale_k=A + 2), fa.FA_ERR_INVALID_ARGUMENT, "4-byte aligned"),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARGUMENT, "finite"),
    (dict(Nk=1 << 24, d=128), fa.FA_ERR_UNSUPPORTED, "2^31 bytes"),
])
def test_fp8_forward_argument_errors(args, status, needle):
    call = dict(FP8)
    call.update(args)
    with pytest.raises(fa.FaError) as ei:
        fa.fa_fwd_fp8(**call)
    assert ei.value.status == status
    assert needle in ei.value.message


@needs_lib
@pytest.mark.parametrize("args", [dict(B=0), dict(H=0), dict(Nq=0), dict(Nq=0, Nk=0)])
def test_fp8_forward_empty_is_a_no_op(args):
    call = dict(FP8)
    call.update(args)
    fa.fa_fwd_fp8(**call)
    assert fa.fa_last_error() == ""


QUANT = dict(x=A, y=A, descale=A, B=2, H=3, N=100, d=128, lens=None, transpose=0, stream=0)


@needs_lib
@pytest.mark.parametrize("args,status,needle", [
    (dict(d=32), fa.FA_ERR_UNSUPPORTED, "64 or 128"),
    (dict(N=-5), fa.FA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(transpose=2), fa.FA_ERR_INVALID_ARGUMENT, "0 or 1"),
    (dict(x=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(descale=None), fa.FA_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(y=A + 8), fa.FA_ERR_INVALID_ARGUMENT, "16-byte aligned"),
    (dict(descale=A + 2), fa.FA_ERR_INVALID_ARGUMENT, "4-byte aligned"),
    (dict(N=5000000, transpose=1), fa.FA_ERR_UNSUPPORTED, "transposed"),
    (dict(N=INT_MAX), fa.FA_ERR_UNSUPPORTED, "2^31"),
    (dict(B=INT_MAX, H=INT_MAX), fa.FA_ERR_UNSUPPORTED, "int32"),
])
def test_quantize_argument_errors(args, status, needle):
    call = dict(QUANT)
    call.update(args)
    with pytest.raises(fa.FaError) as ei:
        fa.fa_quantize_fp8(**call)
    assert ei.value.status == status
    assert needle in ei.value.message


@needs_lib
def test_quantize_empty_batch_and_vt_cols():
    call = dict(QUANT)
    call.update(B=0)
    fa.fa_quantize_fp8(**call)
    assert fa.fa_last_error() == ""
    assert [fa.fa_fp8_vt_cols(n) for n in (0, 1, 63, 64, 65, 16384)] == [0, 64, 64, 64, 128, 16384]


@needs_lib
@pytest.mark.parametrize("value", ["100", "512", "abc"])
def test_decode_chunk_override_rejects_other_values(value):
    """FA_DECODE_CHUNK is read once per process, so each value runs in a fresh interpreter; a value
    other than 64, 128 or 256 makes a decode call (Nq == 1) fail before anything is launched, while
    prefill calls are unaffected by it."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import io_aware_exact_23_amd as fa\n"
        "A = 0x10000000\n"
        "try:\n"
        "    fa.fa_fwd(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, Nq=1, Nk=8, d=64, scale=0.1, causal=0,\n"
        "              kv_seqlens=None, stream=0)\n"
        "except fa.FaError as e:\n"
        "    print(e.status, e.message)\n"
        "try:\n"
        "    fa.fa_fwd(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, Nq=4, Nk=8, d=96, scale=0.1, causal=0,\n"
        "              kv_seqlens=None, stream=0)\n"
        "except fa.FaError as e:\n"
        "    print(e.status, e.message)\n" % ROOT)
    env = dict(os.environ, FA_DECODE_CHUNK=value)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = r.stdout.strip().splitlines()
    assert lines[0].startswith(f"{fa.FA_ERR_INVALID_ARGUMENT} ") and "FA_DECODE_CHUNK" in lines[0]
    assert lines[1].startswith(f"{fa.FA_ERR_UNSUPPORTED} ") and "64 or 128" in lines[1]


@needs_lib
def test_noalloc_rejects_decode_beyond_its_scratch():
    """fa_fwd_noalloc keeps decode partials in a 72 MiB static array: a call needing more is
    rejected before any HIP call (fake addresses are never touched)."""
    # 64 x 32 heads x ceil(16384 / 128) partials x 129 floats = 135 MB > 72 MiB.
    with pytest.raises(fa.FaError) as ei:
        fa.fa_fwd_noalloc(q=A, k=A, v=A, o=A, lse=A, B=64, H=32, Nq=1, Nk=16384, d=128, scale=0.1,
                          causal=0, kv_seqlens=None, stream=0)
    assert ei.value.status == fa.FA_ERR_UNSUPPORTED and "72 MiB" in ei.value.message
    # The same argument checks as fa_fwd.
    with pytest.raises(fa.FaError) as ei:
        fa.fa_fwd_noalloc(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, Nq=1, Nk=8, d=96, scale=0.1,
                          causal=0, kv_seqlens=None, stream=0)
    assert ei.value.status == fa.FA_ERR_UNSUPPORTED
