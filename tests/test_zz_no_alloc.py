"""The allocation-free binning call (gs_bin_sort_noalloc), through the C ABI,
against gs_bin_sort with a caller workspace: two calls in a row, the second on a
smaller scene, give bit-identical lists, ranges, K and status; a request larger
than the library's scratch is refused on the host."""
import ctypes as C

import numpy as np
import pytest

from gpu_cases import log, to_dev
from differentiable_gaussian_splatting_dgs_amd import scenes

pytestmark = pytest.mark.gpu


def _vp(t):
    return C.c_void_p(t.data_ptr())


def test_noalloc_bin_sort_matches_workspace_call():
    import torch
    from differentiable_gaussian_splatting_dgs_amd import gs
    lib = gs.load_library()
    big = scenes.random_small(91, n=30000, width=640, height=480, f=400.0, sh_degree=1, scale_mu=-2.8)
    small = scenes.random_small(92, n=3000, width=200, height=152, f=150.0, sh_degree=1, scale_mu=-2.6)
    for sc in (big, small):
        p = to_dev(sc.params())
        r = gs.Rasterizer(sc.cam, sc.n, sc.sh_degree)
        r.preprocess(p)
        torch.cuda.synchronize()
        cap = int(r.tiles_touched.sum().item()) + 77
        r._alloc_lists(cap)
        r.bin()  # the workspace call
        torch.cuda.synchronize()
        K = int(r.num_keys.item())
        assert int(r.overflow.item()) == 0 and K > 1000
        pl = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
        rg = torch.full_like(r.tile_ranges, -7)
        nk = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        ov = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        cam = gs.camera_struct(sc.cam)
        log(f"[noalloc] n={sc.n} K={K} cap={cap}")
        rc = lib.gs_bin_sort_noalloc(C.byref(cam), sc.n, _vp(r.depth), _vp(r.rect), _vp(r.tiles_touched), cap,
                                     _vp(pl), _vp(rg), _vp(nk), _vp(ov),
                                     C.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, lib.gs_error_string(rc)
        torch.cuda.synchronize()
        assert int(nk.item()) == K and int(ov.item()) == 0
        assert torch.equal(rg, r.tile_ranges)
        assert torch.equal(pl[:K], r.point_list[:K])
    # larger than the scratch: refused before any work, nothing written
    cam = gs.camera_struct(big.cam)
    need = C.c_size_t()
    assert lib.gs_bin_workspace_size(1 << 22, C.byref(cam), 1 << 24, C.byref(need)) == 0
    assert need.value > lib.gs_bin_scratch_bytes()
    fake = C.c_void_p(1 << 20)
    assert lib.gs_bin_sort_noalloc(C.byref(cam), 1 << 22, fake, fake, fake, 1 << 24, fake, fake, fake, fake,
                                   None) == -3
