"""The binding checks caller-supplied output tensors (shape, dtype, device,
contiguity) before any call into the library, so a wrong `out` raises
ValueError instead of letting a kernel write out of bounds.  CPU only: the
checks run before any device work."""
import pytest
import torch

import bius_scan_sequence_amd as K

B, H, T, DK, DV = 1, 2, 8, 16, 16


def tok(d=DK, dtype=torch.float32):
    return torch.zeros((B, H, T, d), dtype=dtype)


def fwd_inputs(dtype=torch.float32):
    return (tok(DK, dtype), tok(DK, dtype), tok(DV, dtype), tok(DK, dtype), tok(DK, dtype), tok(DK, dtype))


def good_fwd_out(dtype=torch.float32):
    return [torch.empty((B, H, T, DV), dtype=dtype), torch.empty((B, H, DK)), torch.empty((B, H, DK, DV))]


def bad_variants(good):
    """(description, out) pairs, each with one defect."""
    out = []
    for i, t in enumerate(good):
        shp = list(t.shape)
        shp[-1] += 1
        o = list(good)
        o[i] = torch.empty(shp, dtype=t.dtype)
        out.append((f"shape of entry {i}", o))
        o = list(good)
        o[i] = torch.empty(t.shape, dtype=torch.float16)
        out.append((f"dtype of entry {i}", o))
        if t.dim() >= 2 and t.shape[-1] > 1 and t.shape[-2] > 1:
            o = list(good)
            o[i] = torch.empty(tuple(t.shape[:-2]) + (t.shape[-1], t.shape[-2]), dtype=t.dtype).transpose(-1, -2)
            out.append((f"contiguity of entry {i}", o))
    out.append(("too few tensors", list(good)[:-1]))
    return out


@pytest.mark.parametrize("case", range(len(bad_variants(good_fwd_out()))))
def test_forward_rejects_bad_out(case):
    desc, out = bad_variants(good_fwd_out())[case]
    with pytest.raises(ValueError):
        K.forward(*fwd_inputs(), out=out)


@pytest.mark.parametrize("case", range(len(bad_variants(good_fwd_out()))))
def test_forward_ou_rejects_bad_out(case):
    desc, out = bad_variants(good_fwd_out())[case]
    q, k, v, dt, _, vp = fwd_inputs()
    theta = torch.ones((H, DK))
    with pytest.raises(ValueError):
        K.forward_ou(q, k, v, dt, theta, theta.clone(), vp, out=out)


@pytest.mark.parametrize("case", range(len(bad_variants(good_fwd_out()))))
def test_forward_prologue_rejects_bad_out(case):
    desc, out = bad_variants(good_fwd_out())[case]
    xq, xk, xv, dt, _, vp = fwd_inputs()
    theta = torch.ones((H, DK))
    w = (torch.zeros((H, DK, 4)), torch.zeros((H, DK, 4)), torch.zeros((H, DV, 4)))
    with pytest.raises(ValueError):
        K.forward_prologue(xq, xk, xv, dt, theta, theta.clone(), vp, w, out=out)


def test_forward_vprec_rejects_bad_out():
    q, k, v, ld, pn, _ = fwd_inputs()
    vp = tok(DV)
    good = [torch.empty((B, H, T, DV)), torch.empty((B, H, DK, DV)), torch.empty((B, H, DK, DV))]
    for desc, out in bad_variants(good):
        with pytest.raises(ValueError):
            K.forward_vprec(q, k, v, ld, pn, vp, out=out)


def test_precision_scan_rejects_bad_out():
    x = torch.zeros((B, H, T, DK))
    good = [torch.empty((B, H, T, DK)), torch.empty((B, H, DK))]
    for desc, out in bad_variants(good):
        with pytest.raises(ValueError):
            K.precision_scan(x, x.clone(), x.clone(), out=out)


def test_decode_step_rejects_bad_out():
    one = lambda d: torch.zeros((B, H, d))
    args = (one(DK), one(DK), one(DV), one(DK), one(DK), one(DK))
    good = [torch.empty((B, H, DV)), torch.empty((B, H, DK)), torch.empty((B, H, DK, DV))]
    for desc, out in bad_variants(good):
        with pytest.raises(ValueError):
            K.decode_step(*args, out=out)


def test_backward_rejects_bad_out():
    q, k, v, ld, pn, vp = fwd_inputs()
    gy = tok(DV)
    lpath = tok(DK)
    good = [torch.empty_like(x) for x in (q, k, v, ld, pn, vp)] + [torch.empty((B, H, DK)),
                                                                   torch.empty((B, H, DK, DV))]
    for desc, out in bad_variants(good):
        if desc == "too few tensors":
            continue  # backward unpacks its eight outputs positionally
        with pytest.raises(ValueError):
            K.backward(q, k, v, ld, pn, vp, gy, lpath, out=out)
