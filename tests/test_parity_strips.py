"""GPU: the layer computed as horizontal strips (one device's share each in a
patch-parallel run), text rows merged exactly or by the patch average of Eq. 7
(pith.science review of CLEAR, "What carries the argument")."""

import math

import numpy as np
import pytest
import torch

import dit_circular_local_amd as ca
from dit_circular_local_amd.inputs import make_qkv
from oracle import attention, text_rows_patch_average

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _inputs(dtype, B, H, n_text, gh, gw, d, seed):
    return make_qkv(B, H, n_text, gh, gw, d, dtype, seed, rms_norm=(dtype == "bf16"),
                    scale=1.0 if dtype == "bf16" else 1.0 / math.sqrt(d), device="cuda")


def _run_strips(q, k, v, n_text, gh, gw, r2, P, text_keys_everywhere, window="circle"):
    B, H, N, d = q.shape
    out = torch.full_like(q, float("nan"))
    po = torch.zeros((P, B * H, max(n_text, 1), d), dtype=torch.float32, device="cuda")[:, :, :n_text]
    pml = torch.zeros((P, B * H, max(n_text, 1), 2), dtype=torch.float32, device="cuda")[:, :, :n_text]
    po, pml = po.contiguous(), pml.contiguous()
    for s, (y0, y1) in enumerate(ca.strip_rows(gh, P)):
        ca.fwd_strip(q, k, v, n_text, gh, gw, y0, y1, out, po[s], pml[s], r2=r2,
                     with_text_keys=text_keys_everywhere or s == 0, window=window)
    return out, po, pml


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("P", [1, 2, 3, 5])
def test_strips_reproduce_the_layer(dtype, P):
    n_text, gh, gw, d, r2 = 130, 45, 24, 128, 49
    q, k, v = _inputs(dtype, 1, 2, n_text, gh, gw, d, seed=P)
    full = ca.fwd(q, k, v, n_text, gh, gw, r2=r2)
    out, po, pml = _run_strips(q, k, v, n_text, gh, gw, r2, P, text_keys_everywhere=False)
    ca.text_merge(po, pml, out, n_text, gh, gw, mode="exact")
    torch.cuda.synchronize()
    # image rows: the same tiles and chunk order as the whole-layer launch
    assert torch.equal(out[:, :, n_text:], full[:, :, n_text:])
    ref, _ = attention(_np(q), _np(k), _np(v), n_text, gh, gw, r2, workers=4)
    err = np.abs(_np(out) - ref).max()
    assert err <= TOL[dtype], f"{dtype} P={P}: max-abs {err:.3e}"


@pytest.mark.parametrize("dtype,P", [("fp32", 2), ("fp32", 4), ("bf16", 3), ("bf16", 8)])
def test_patch_average_text_rows_match_eq7(dtype, P):
    n_text, gh, gw, d, r2 = 64, 32, 16, 128, 16
    q, k, v = _inputs(dtype, 1, 2, n_text, gh, gw, d, seed=10 + P)
    out, po, pml = _run_strips(q, k, v, n_text, gh, gw, r2, P, text_keys_everywhere=True)
    ca.text_merge(po, pml, out, n_text, gh, gw, mode="patch_average")
    torch.cuda.synchronize()
    for h in range(2):
        ref = text_rows_patch_average(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), n_text, gh, gw, P)
        err = np.abs(_np(out[0, h, :n_text]) - ref).max()
        assert err <= TOL[dtype], f"{dtype} P={P} head {h}: max-abs {err:.3e}"


def test_exact_merge_lse_and_one_strip_with_text_keys_only_once():
    n_text, gh, gw, d, r2 = 40, 20, 20, 64, 25
    q, k, v = _inputs("fp32", 2, 1, n_text, gh, gw, d, seed=21)
    out, po, pml = _run_strips(q, k, v, n_text, gh, gw, r2, 4, text_keys_everywhere=False)
    _, lse = ca.text_merge(po, pml, out, n_text, gh, gw, mode="exact", return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = attention(_np(q), _np(k), _np(v), n_text, gh, gw, r2)
    assert np.abs(_np(lse[:, :, :n_text]) - ref_lse[:, :, :n_text]).max() <= 1e-5


@pytest.mark.parametrize("window", ["circle", "square"])
def test_strip_reads_only_its_halo(window):
    """Keys more than isqrt(r2) rows away from the strip do not change its rows:
    poisoning them (large finite values) leaves the strip's outputs bit-identical."""
    n_text, gh, gw, d, r2 = 16, 48, 24, 128, 36
    q, k, v = _inputs("bf16", 1, 2, n_text, gh, gw, d, seed=31)
    y0, y1 = 16, 29
    w = math.isqrt(r2)
    out_a, po_a, pml_a = (torch.zeros_like(q), torch.zeros((2, n_text, d), device="cuda"),
                          torch.zeros((2, n_text, 2), device="cuda"))
    ca.fwd_strip(q, k, v, n_text, gh, gw, y0, y1, out_a, po_a, pml_a, r2=r2, window=window)
    k2, v2 = k.clone(), v.clone()
    far = [y for y in range(gh) if y < y0 - w or y >= y1 + w]
    for y in far:
        s = n_text + y * gw
        k2[:, :, s:s + gw] = 300.0
        v2[:, :, s:s + gw] = -500.0
    out_b, po_b, pml_b = torch.zeros_like(q), torch.zeros_like(po_a), torch.zeros_like(pml_a)
    ca.fwd_strip(q, k2, v2, n_text, gh, gw, y0, y1, out_b, po_b, pml_b, r2=r2, window=window)
    torch.cuda.synchronize()
    rows = slice(n_text + y0 * gw, n_text + y1 * gw)
    assert torch.equal(out_a[:, :, rows], out_b[:, :, rows])
    # the text partial covers only the strip's own rows: unaffected as well
    assert torch.equal(po_a, po_b) and torch.equal(pml_a, pml_b)


def test_strip_and_merge_reject_bad_arguments():
    n_text, gh, gw, d = 8, 8, 8, 64
    q, k, v = _inputs("bf16", 1, 1, n_text, gh, gw, d, seed=1)
    out = torch.zeros_like(q)
    po, pml = torch.zeros((1, n_text, d), device="cuda"), torch.zeros((1, n_text, 2), device="cuda")
    for y0, y1 in [(3, 3), (-1, 4), (2, 9)]:
        with pytest.raises(ca.ClearError) as e:
            ca.fwd_strip(q, k, v, n_text, gh, gw, y0, y1, out, po, pml, radius=2)
        assert e.value.code == ca.CLEAR_EINVAL
    L = ca.lib()
    rc = L.clear_text_merge(po.data_ptr(), pml.data_ptr(), 1, ca.CLEAR_MERGE_PATCH_AVERAGE, out.data_ptr(),
                            po.data_ptr(), 1, 1, d, n_text, gh, gw, ca.CLEAR_BF16, None)
    assert rc == ca.CLEAR_EINVAL and "lse" in ca.last_error()
    rc = L.clear_text_merge(po.data_ptr(), pml.data_ptr(), 0, ca.CLEAR_MERGE_EXACT, out.data_ptr(),
                            None, 1, 1, d, n_text, gh, gw, ca.CLEAR_BF16, None)
    assert rc == ca.CLEAR_EINVAL


def _slab(t, n_text, gw, lo, hi):
    """Text tokens plus image rows [lo, hi) of [B, H, N, d] t, as a contiguous
    buffer: what one device of a patch-parallel run holds."""
    idx = torch.cat([torch.arange(n_text), n_text + torch.arange(lo * gw, hi * gw)]).to(t.device)
    return t.index_select(2, idx).contiguous()


@pytest.mark.parametrize("gh,gw,H,r,P", [(128, 128, 2, 16, 4), (128, 64, 2, 8, 8), (512, 512, 1, 32, 8),
                                         (80, 24, 3, 5, 5)])
def test_slab_local_strips_equal_the_layer(gh, gw, H, r, P):
    """Each strip computed on a buffer holding only the text tokens, its own rows
    and halos of h rows above and below (h = isqrt(r2) rounded up to the
    16-row query-tile height, clipped at the grid's edges): the O(r x W) slab of
    one device in the pages' patch-parallel inference (pith.science review of
    CLEAR, "What carries the argument").  With the strip's local grid and row
    range, its image rows equal the whole layer's bit for bit, its text-row
    partial equals the one computed on the full-size tensors, and the exact
    merge of the slabs' partials gives the text rows of the layer."""
    n_text, d, r2 = 512, 128, r * r
    q, k, v = _inputs("bf16", 1, H, n_text, gh, gw, d, seed=gh + r)
    full = ca.fwd(q, k, v, n_text, gh, gw, r2=r2)
    h = -(-math.isqrt(r2) // 16) * 16
    rows = [(y0, y1) for y0, y1 in ca.strip_rows(gh, P)]
    assert all(y0 % 16 == 0 for y0, _ in rows) or gh == 80
    po = torch.zeros((P, H, n_text, d), dtype=torch.float32, device="cuda")
    pml = torch.zeros((P, H, n_text, 2), dtype=torch.float32, device="cuda")
    po_full, pml_full = torch.zeros_like(po), torch.zeros_like(pml)
    out_full = torch.zeros_like(q)
    merged = torch.zeros_like(q)
    for s, (y0, y1) in enumerate(rows):
        lo, hi = max(0, y0 - h), min(gh, y1 + h)
        ql, kl, vl = (_slab(t, n_text, gw, lo, hi) for t in (q, k, v))
        outl = torch.zeros_like(ql)
        ca.fwd_strip(ql, kl, vl, n_text, hi - lo, gw, y0 - lo, y1 - lo, outl, po[s], pml[s], r2=r2,
                     with_text_keys=(s == 0))
        ca.fwd_strip(q, k, v, n_text, gh, gw, y0, y1, out_full, po_full[s], pml_full[s], r2=r2,
                     with_text_keys=(s == 0))
        torch.cuda.synchronize()
        mine = outl[:, :, n_text + (y0 - lo) * gw:n_text + (y1 - lo) * gw]
        if (y0 - lo) % 16 == 0 and lo % 16 == 0:
            # the slab's query tiles are the layer's: same chunk lists, same order
            assert torch.equal(mine, full[:, :, n_text + y0 * gw:n_text + y1 * gw]), f"strip {s}"
        else:
            # a slab cut off the 16-row tiling groups the queries differently
            err = (mine.float() - full[:, :, n_text + y0 * gw:n_text + y1 * gw].float()).abs().max().item()
            assert err <= 2e-2, f"strip {s}: max-abs {err:.3e}"
        assert torch.equal(po[s], po_full[s]) and torch.equal(pml[s], pml_full[s]), f"strip {s} partial"
    ca.text_merge(po, pml, merged, n_text, gh, gw, mode="exact")
    torch.cuda.synchronize()
    ref, _ = attention(_np(q[:, :, :]), _np(k), _np(v), n_text, gh, gw, r2, workers=8) if gh * gw <= 16384 \
        else (None, None)
    if ref is not None:
        err = np.abs(_np(merged[:, :, :n_text]) - ref[:, :, :n_text]).max()
        assert err <= TOL["bf16"], f"text rows: max-abs {err:.3e}"
    else:
        err = (merged[:, :, :n_text].float() - full[:, :, :n_text].float()).abs().max().item()
        assert err <= TOL["bf16"], f"text rows vs the layer: max-abs {err:.3e}"
