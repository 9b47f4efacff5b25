"""gtr_gla_fwd_noalloc (static per-GPU scratch, allocates nothing) against
gtr_gla_fwd (library-allocated workspace) through the C ABI: two calls in a
row, the second with a smaller input, each bit for bit equal to the existing
entry point (the same kernels and plan) and within the fp16 bar of the
oracle; the scratch re-initialises itself across the layout change. Then the
same small shape at d_k = 32 and again at d_k = 64 (the span kernels, equal
spans and sequences per launch, exchange slots of different sizes), in other
scan orders, so that the scratch's layout follows the key width too."""
import ctypes

import numpy as np
import pytest

import gla_synth
import oracle

torch = pytest.importorskip("torch")
import chunkwise_gated_recurrence_amd as gla  # noqa: E402

pytestmark = pytest.mark.gpu

BIG = gla_synth.WORKLOADS["img640"].with_(name="noalloc_big", seed=97)        # 6 heads, 40x40
SMALL = gla_synth.WORKLOADS["img640"].with_(name="noalloc_small", H=2, grid_h=24, grid_w=20,
                                            seed=98)
SMALL32 = SMALL.with_(name="noalloc_small32", d_k=32, seed=99)


def _call(fn, x, w, d, o, s):
    lib = gla.load_library()
    st = torch.cuda.current_stream().cuda_stream or None
    r = getattr(lib, fn)(*[t.data_ptr() for t in x], w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v,
                         d, 64, o.data_ptr(), s.data_ptr(), ctypes.c_void_p(st))
    assert r == gla.OK, (fn, r, gla.gtr_gla_status_str(r))


def test_noalloc_matches_the_allocating_entry_point():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    for w, d in ((BIG, 2), (SMALL, 1), (SMALL32, 3), (SMALL, 0)):
        arrays = gla_synth.generate(w)
        x = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]
        o_ref = torch.empty((w.B, w.L, w.H, w.d_v), dtype=torch.float16, device="cuda")
        s_ref = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
        o = torch.full_like(o_ref, 7.0)
        s = torch.full_like(s_ref, 7.0)
        print(f"[case] noalloc {w.name} dir={d}", flush=True)
        _call("gtr_gla_fwd", x, w, d, o_ref, s_ref)
        _call("gtr_gla_fwd_noalloc", x, w, d, o, s)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref), w.name
        oo, so = oracle.recurrent(*arrays, w.grid_h, w.grid_w, d)
        assert oracle.rel_err(o.cpu().numpy().astype(np.float64), oo) <= 5e-3
        assert oracle.rel_err(s.cpu().numpy(), so) <= 5e-3
    assert gla.gtr_gla_workspace_status() == gla.OK
