"""The allocation-free RMSNorm backward (static per-GPU scratch instead of a
caller workspace) against the entry that takes the workspace: bit for bit,
on two calls in a row, the second with a smaller input; shapes whose
partials exceed the static buffer are refused before any device work."""
import numpy as np
import pytest

from layer_streaming_amd import synth
from tests.gpu_util import dev_bits, dev_zeros_bits, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from layer_streaming_amd import mt  # noqa: E402


def _inputs(rng, T, d, x_f32):
    if x_f32:
        x = rng.standard_normal((T, d)).astype(np.float32)
        dx_ = torch.from_numpy(x).cuda()
    else:
        dx_ = dev_bits(synth.bf16_exact_normal(rng, (T, d)))
    g = dev_bits(synth.bf16_exact_normal(rng, (d,), std=0.2, mean=1.0))
    dn = dev_bits(synth.bf16_exact_normal(rng, (T, d)))
    res = dev_bits(synth.bf16_exact_normal(rng, (T, d)))
    rstd = torch.from_numpy((0.5 + rng.random(T)).astype(np.float32)).cuda()
    return dx_, g, dn, res, rstd


def _with_workspace(s, T, d, x_f32, dx_, g, dn, res, rstd):
    scratch = torch.zeros(int(mt.lib.mt_k_rmsnorm_bwd_scratch_elems(T, d)), dtype=torch.float32, device="cuda")
    out, dg = dev_zeros_bits((T, d)), dev_zeros_bits((d,))
    mt.check(mt.lib.mt_k_rmsnorm_bwd(dn.data_ptr(), dx_.data_ptr(), x_f32, g.data_ptr(), rstd.data_ptr(),
                                     res.data_ptr(), out.data_ptr(), dg.data_ptr(), scratch.data_ptr(), T, d, s))
    return out, dg


def _no_alloc(s, T, d, x_f32, dx_, g, dn, res, rstd):
    out, dg = dev_zeros_bits((T, d)), dev_zeros_bits((d,))
    mt.check(mt.lib.mt_k_rmsnorm_bwd_noalloc(dn.data_ptr(), dx_.data_ptr(), x_f32, g.data_ptr(), rstd.data_ptr(),
                                             res.data_ptr(), out.data_ptr(), dg.data_ptr(), T, d, s))
    return out, dg


@pytest.mark.parametrize("shapes", [((8192, 3584, 0), (130, 256, 0)), ((2048, 8192, 1), (37, 3584, 1))],
                         ids=["7b-bf16-then-small", "70b-f32-then-small"])
def test_no_alloc_rmsnorm_bwd_matches_workspace_entry(shapes):
    rng = np.random.default_rng(5)
    s = torch.cuda.current_stream().cuda_stream
    for T, d, x_f32 in shapes:  # the second call is smaller: stale partials of the first must not leak in
        log(f"no-alloc rmsnorm bwd T={T} d={d} x_f32={x_f32}")
        args = _inputs(rng, T, d, x_f32)
        want_dx, want_dg = _with_workspace(s, T, d, x_f32, *args)
        got_dx, got_dg = _no_alloc(s, T, d, x_f32, *args)
        torch.cuda.synchronize()
        assert torch.equal(got_dx, want_dx)
        assert torch.equal(got_dg, want_dg)
        assert bool(torch.any(got_dg != 0))


def test_no_alloc_rmsnorm_bwd_refuses_oversized_shapes():
    """Every width the kernel supports (d <= 8192) fits the static buffer;
    a wider row is refused on the host, before any launch."""
    s = torch.cuda.current_stream().cuda_stream
    assert mt.lib.mt_k_rmsnorm_bwd_scratch_elems(1 << 20, 8192) <= 4 << 20
    T, d = 8192, 8200
    assert mt.lib.mt_k_rmsnorm_bwd_scratch_elems(T, d) > 4 << 20
    p = dev_zeros_bits((16,))
    r = mt.lib.mt_k_rmsnorm_bwd_noalloc(p.data_ptr(), p.data_ptr(), 0, p.data_ptr(), p.data_ptr(), None,
                                        p.data_ptr(), p.data_ptr(), T, d, s)
    assert r == mt.MT_E_INVAL
    assert b"static buffer" in mt.lib.mt_last_error()
