"""The C ABI library loads, exports every symbol include/kla.h declares, and
rejects bad arguments on the host before any HIP call (CPU only)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kla.h")

KLA_OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
KLA_OK_T0 = KLA_OK  # T = 0 without lambda_T: nothing to do, no HIP call


@pytest.fixture(scope="module")
def K():
    import bius_scan_sequence_amd as K
    return K


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kla_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kla_forward", "kla_forward_ou", "kla_forward_prologue", "kla_forward_vprec", "kla_forward_workspace_bytes", "kla_precision_scan",
              "kla_precision_scan_workspace_bytes", "kla_decode_step", "kla_backward",
              "kla_backward_workspace_bytes", "kla_workspace_init",
              "kla_workspace_error", "kla_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(K):
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(K.lib, n)


def test_status_strings(K):
    for code in (0, 1, 2, 3, 4, 99):
        assert isinstance(K.kla_status_string(code), str) and K.kla_status_string(code)


def test_workspace_sizes(K):
    assert K.kla_forward_workspace_bytes(8, 8, 2048, 64, 64) > 256
    assert K.kla_forward_workspace_bytes(1, 1, 0, 16, 16) >= 256
    assert K.kla_forward_workspace_bytes(1, 1, 256, 48, 16) == 0     # unsupported width
    assert K.kla_forward_workspace_bytes(0, 1, 256, 16, 16) == 0     # empty batch
    assert K.kla_precision_scan_workspace_bytes(1, 1024, 65536, 64) >= 256
    assert K.kla_precision_scan_workspace_bytes(1, 1, 65536, 64) > 256  # few chains: T split
    assert K.kla_precision_scan_workspace_bytes(1, 1, 10, 0) == 0
    assert K.kla_backward_workspace_bytes(8, 8, 2048, 64, 64) > 256
    assert K.kla_backward_workspace_bytes(1, 1, 0, 16, 16) >= 256
    assert K.kla_backward_workspace_bytes(1, 1, 256, 128, 64) > K.kla_backward_workspace_bytes(1, 1, 256, 64, 64)
    assert K.kla_backward_workspace_bytes(1, 1, 256, 48, 16) == 0


A = 0x10000  # an aligned fake device address; validation never dereferences it


def fwd(K, **over):
    args = dict(q=A, k=A, v=A, log_decay=A, proc_noise=A, val_prec=A, lambda0=None, M0=None,
                y=A, lambda_T=A, M_T=A, lambda_path=None, B=1, H=1, T=64, dk=16, dv=16, dtype=1,
                workspace=A, workspace_bytes=1 << 30, stream=None)
    args.update(over)
    return K.kla_forward(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), INVALID), (dict(v=None), INVALID), (dict(y=None), INVALID),
    (dict(lambda_T=None), INVALID), (dict(M_T=None), INVALID),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(T=-5), INVALID),
    (dict(dk=48), UNSUPPORTED), (dict(dv=8), UNSUPPORTED), (dict(dk=256), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED),
    (dict(q=A + 2), INVALID), (dict(log_decay=A + 8), INVALID),
    (dict(lambda0=A + 2), INVALID),
    (dict(y=A + 2), INVALID), (dict(y=A + 8), INVALID),  # y is written in 16-byte units
    (dict(workspace=None), WORKSPACE), (dict(workspace=A + 64), WORKSPACE),
    (dict(workspace_bytes=16), WORKSPACE),
    (dict(B=1 << 16, H=1 << 16, T=1024), INVALID),
])
def test_forward_rejects(K, over, code):
    assert fwd(K, **over) == code


def pscan(K, **over):
    args = dict(log_decay=A, proc_noise=A, obs_prec=A, lambda0=None, lambda_path=A, lambda_T=None,
                B=1, H=4, T=128, D=64, workspace=A, workspace_bytes=1 << 30, stream=None)
    args.update(over)
    return K.kla_precision_scan(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(log_decay=None), INVALID), (dict(lambda_path=None), INVALID),
    (dict(T=0, lambda_path=None, log_decay=None), KLA_OK_T0),
    (dict(D=0), INVALID), (dict(T=-1), INVALID), (dict(obs_prec=A + 1), INVALID),
    (dict(workspace=None), WORKSPACE), (dict(workspace_bytes=8), WORKSPACE),
])
def test_precision_scan_rejects(K, over, code):
    assert pscan(K, **over) == code


def dec(K, **over):
    args = dict(q=A, k=A, v=A, log_decay=A, proc_noise=A, val_prec=A, lambda_in=None, M_in=None,
                lambda_out=A, M_out=A, y=A, B=2, H=3, dk=64, dv=64, dtype=1, stream=None)
    args.update(over)
    return K.kla_decode_step(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), INVALID), (dict(v=None), INVALID), (dict(y=None), INVALID),
    (dict(lambda_out=None), INVALID), (dict(M_out=None), INVALID),
    (dict(B=0), INVALID), (dict(H=-2), INVALID), (dict(B=1 << 16, H=1 << 15), INVALID),
    (dict(dk=48), UNSUPPORTED), (dict(dv=8), UNSUPPORTED), (dict(dtype=3), UNSUPPORTED),
    (dict(q=A + 1), INVALID), (dict(k=A + 2, dtype=0), INVALID), (dict(y=A + 1), INVALID),
    (dict(M_out=A + 4), INVALID), (dict(M_in=A + 8), INVALID), (dict(lambda_in=A + 2), INVALID),
    (dict(lambda_out=A + 1), INVALID),
])
def test_decode_step_rejects(K, over, code):
    assert dec(K, **over) == code


def test_workspace_init_rejects(K):
    assert K.kla_workspace_init(None, 1024, None) == WORKSPACE
    assert K.kla_workspace_init(A + 4, 1024, None) == WORKSPACE
    assert K.kla_workspace_init(A, 1022, None) == INVALID


def bwd(K, **over):
    args = dict(q=A, k=A, v=A, log_decay=A, proc_noise=A, val_prec=A, lambda0=None, M0=None,
                lambda_path=A, grad_y=A, grad_lambda_T=None, grad_M_T=None, grad_q=A, grad_k=A, grad_v=A,
                grad_log_decay=A, grad_proc_noise=A, grad_val_prec=A, grad_lambda0=A, grad_M0=A,
                B=1, H=2, T=100, dk=64, dv=32, dtype=1, workspace=A, workspace_bytes=1 << 30, stream=None)
    args.update(over)
    return K.kla_backward(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), INVALID), (dict(lambda_path=None), INVALID), (dict(grad_y=None), INVALID),
    (dict(grad_v=None), INVALID), (dict(grad_val_prec=None), INVALID), (dict(grad_lambda0=None), INVALID),
    (dict(grad_M0=None), INVALID), (dict(B=0), INVALID), (dict(T=-1), INVALID),
    (dict(dk=256), UNSUPPORTED), (dict(dv=8), UNSUPPORTED), (dict(dk=48), UNSUPPORTED),
    (dict(dtype=2), UNSUPPORTED),
    (dict(q=A + 1), INVALID), (dict(q=A + 8), INVALID), (dict(lambda_path=A + 4), INVALID),
    (dict(grad_y=A + 8), INVALID), (dict(grad_q=A + 8), INVALID),
    (dict(grad_M0=A + 4), INVALID),
    (dict(M0=A + 8), INVALID), (dict(grad_M_T=A + 4), INVALID), (dict(grad_lambda_T=A + 2), INVALID),
    (dict(grad_k=A + 2, dtype=0), INVALID),
    (dict(workspace=None), WORKSPACE), (dict(workspace=A + 16), WORKSPACE),
    (dict(workspace_bytes=1024), WORKSPACE),
    (dict(B=1 << 12, H=1 << 12, T=1 << 10), INVALID),
])
def test_backward_rejects(K, over, code):
    assert bwd(K, **over) == code


def fwd_ou(K, **over):
    args = dict(q=A, k=A, v=A, dt=A, theta=A, sigma2=A, val_prec=A, lambda0=None, M0=None,
                y=A, lambda_T=A, M_T=A, lambda_path=None, B=1, H=1, T=64, dk=16, dv=16, dtype=1,
                workspace=A, workspace_bytes=1 << 30, stream=None)
    args.update(over)
    return K.kla_forward_ou(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(theta=None), INVALID), (dict(sigma2=None), INVALID), (dict(dt=None), INVALID),
    (dict(q=None), INVALID), (dict(theta=A + 2), INVALID), (dict(sigma2=A + 1), INVALID),
    (dict(dt=A + 8), INVALID), (dict(dk=48), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED),
    (dict(workspace_bytes=16), WORKSPACE), (dict(B=0), INVALID),
])
def test_forward_ou_rejects(K, over, code):
    assert fwd_ou(K, **over) == code


def fwd_pro(K, **over):
    args = dict(xq=A, xk=A, xv=A, dt_raw=A, theta=A, sigma2=A, vp_raw=A, conv_wq=A, conv_wk=A, conv_wv=A,
                conv_bq=None, conv_bk=None, conv_bv=None, conv_width=4, lambda0=None, M0=None,
                y=A, lambda_T=A, M_T=A, lambda_path=None, B=1, H=1, T=64, dk=16, dv=16, dtype=1,
                workspace=A, workspace_bytes=1 << 30, stream=None)
    args.update(over)
    return K.kla_forward_prologue(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(conv_wq=None), INVALID), (dict(conv_wk=None), INVALID), (dict(conv_wv=None), INVALID),
    (dict(conv_width=0), INVALID), (dict(conv_width=5), INVALID), (dict(conv_wv=A + 4), INVALID),
    (dict(conv_bk=A + 2), INVALID), (dict(theta=None), INVALID), (dict(xq=None), INVALID),
    (dict(dt_raw=A + 8), INVALID), (dict(dk=48), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED),
    (dict(workspace_bytes=16), WORKSPACE), (dict(B=0), INVALID),
])
def test_forward_prologue_rejects(K, over, code):
    assert fwd_pro(K, **over) == code


def fwd_vp(K, **over):
    args = dict(q=A, k=A, v=A, log_decay=A, proc_noise=A, val_prec=A, lambda0=None, M0=None,
                y=A, lambda_T=A, M_T=A, B=1, H=2, T=64, dk=64, dv=32, dtype=1, stream=None)
    args.update(over)
    return K.kla_forward_vprec(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), INVALID), (dict(val_prec=None), INVALID), (dict(y=None), INVALID),
    (dict(lambda_T=None), INVALID), (dict(M_T=None), INVALID), (dict(B=0), INVALID),
    (dict(dk=48), UNSUPPORTED), (dict(dv=8), UNSUPPORTED), (dict(dtype=9), UNSUPPORTED),
    (dict(k=A + 1), INVALID), (dict(v=A + 2, dtype=0), INVALID), (dict(M0=A + 2), INVALID),
    (dict(T=-1), INVALID),
])
def test_forward_vprec_rejects(K, over, code):
    assert fwd_vp(K, **over) == code


def test_workspace_error_rejects(K):
    import ctypes
    out = ctypes.c_int(0)
    assert K.lib.kla_workspace_error(None, ctypes.byref(out), None) == INVALID
    assert K.lib.kla_workspace_error(A + 4, ctypes.byref(out), None) == INVALID
    assert K.lib.kla_workspace_error(A, None, None) == INVALID


def fwd_na(K, **over):
    args = dict(q=A, k=A, v=A, log_decay=A, proc_noise=A, val_prec=A, lambda0=None, M0=None,
                y=A, lambda_T=A, M_T=A, lambda_path=None, B=1, H=1, T=64, dk=16, dv=16, dtype=1,
                error_flag=None, stream=None)
    args.update(over)
    return K.kla_forward_noalloc(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), INVALID), (dict(y=None), INVALID), (dict(M_T=None), INVALID),
    (dict(B=0), INVALID), (dict(T=-1), INVALID), (dict(dk=48), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(q=A + 2), INVALID), (dict(y=A + 8), INVALID), (dict(lambda0=A + 2), INVALID),
    (dict(error_flag=A + 2), INVALID), (dict(B=1 << 16, H=1 << 16, T=1024), INVALID),
])
def test_forward_noalloc_rejects(K, over, code):
    assert fwd_na(K, **over) == code


def test_forward_noalloc_rejects_beyond_scratch(K):
    """2048 heads at T = 2048 (bf16, d64) need about 69 MB, more than the
    64 MiB scratch array: KLA_ERR_TOO_LARGE before any launch."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("fake device addresses: run where no GPU is visible (the GPU test uses real tensors)")
    m = re.search(r"#define KLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and K.KLA_NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    rc = fwd_na(K, B=32, H=64, T=2048, dk=64, dv=64)
    assert rc == 5
    assert "KLA_NOALLOC_SCRATCH_BYTES" in K.kla_status_string(rc)
