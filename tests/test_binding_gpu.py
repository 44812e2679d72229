"""The binding checks caller-supplied `out` and `sinks` tensors before anything is
enqueued: the kernels write B*Hq*Lq*Dv contiguous elements through out's address and
read Hq sinks, so a tensor of another shape, dtype, device or layout is refused."""
import pytest

import scaled_dot_product_06_amd as sd

pytestmark = pytest.mark.gpu


def _inputs(Lq=70, Lk=90):
    import torch
    g = torch.Generator(device="cpu").manual_seed(5)
    q = torch.randn(1, 8, Lq, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, 2, Lk, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, Lk, 128, generator=g).to(torch.bfloat16).cuda()
    s = torch.randn(8, generator=g).to(torch.bfloat16).cuda()
    return q, k, v, s


@pytest.mark.parametrize("bad", ["shape", "dtype", "strided", "cpu"])
def test_bad_out_is_refused_before_any_launch(bad):
    import torch
    q, k, v, s = _inputs()
    if bad == "shape":
        out = torch.full((1, 8, 69, 128), 2.0, dtype=torch.bfloat16, device="cuda")
    elif bad == "dtype":
        out = torch.full((1, 8, 70, 128), 2.0, dtype=torch.float16, device="cuda")
    elif bad == "strided":
        out = torch.full((1, 8, 128, 70), 2.0, dtype=torch.bfloat16, device="cuda").transpose(2, 3)
    else:
        out = torch.full((1, 8, 70, 128), 2.0, dtype=torch.bfloat16)
    with pytest.raises(sd.SdpaError) as err:
        sd.attention(q, k, v, 0.1, 1, None, s, out=out)
    assert err.value.code == sd.SDPA_ERR_INVALID and "out" in err.value.message
    torch.cuda.synchronize()
    assert torch.all(out == 2.0)


def test_non_contiguous_sinks_are_refused():
    import torch
    q, k, v, _ = _inputs()
    s = torch.randn(16).to(torch.bfloat16).cuda()[::2]
    with pytest.raises(sd.SdpaError) as err:
        sd.attention(q, k, v, 0.1, 1, None, s)
    assert "sinks" in err.value.message


def test_good_out_is_written():
    import torch
    q, k, v, s = _inputs()
    out = torch.full((1, 8, 70, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = sd.attention(q, k, v, 0.1, 1, None, s, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.isfinite(out.float()).all()
