"""dspark_schedule_noalloc, the schedule call that allocates nothing (its
sorted keys live in the library's own device array), against
dspark_schedule with a caller workspace: identical outputs on two calls in a
row, the second with a smaller input, for every mode; sizes past the array
are refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import __graft_entry__
    __graft_entry__._ensure_built()
    import draft_verify_schedule_amd.binding as b
    return b.load_library()


def _outputs(R, K):
    return {"a": torch.full((R, K), -7.0, dtype=torch.float32, device=DEV),
            "ell": torch.full((R,), -7, dtype=torch.int32, device=DEV),
            "cu_seqlens": torch.full((R + 1,), -7, dtype=torch.int32, device=DEV),
            "n_admitted": torch.full((1,), -7, dtype=torch.int32, device=DEV),
            "theta": torch.full((1,), -7.0, dtype=torch.float64, device=DEV)}


def _compare(got, ref):
    for k in ("ell", "cu_seqlens", "n_admitted"):
        assert torch.equal(got[k], ref[k]), k
    assert torch.equal(got["a"].view(torch.int32), ref["a"].view(torch.int32))
    assert torch.equal(got["theta"].view(torch.int64), ref["theta"].view(torch.int64))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_noalloc_matches_workspace_schedule(lib, mode):
    from draft_verify_schedule_amd import binding as b
    from draft_verify_schedule_amd import workloads as wl
    big = wl.make("sched_stress", device="cpu", V=64)          # 1024 x 7 = 7168 candidates
    small = wl.make("full_step", device="cpu", V=64)           # 512 x 7 = 3584 candidates
    for w in (big, small):                                     # the second call is smaller
        c, sps = w.c.to(DEV), w.sps.to(DEV)
        R, K = c.shape
        cap = (R * K) // 3
        ref = b.dspark_schedule(c, sps, mode, cap)
        got = _outputs(R, K)
        st = lib.dspark_schedule_noalloc(R, K, ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(sps.data_ptr()),
                                         sps.numel(), mode, cap, ctypes.c_void_p(got["a"].data_ptr()),
                                         ctypes.c_void_p(got["ell"].data_ptr()),
                                         ctypes.c_void_p(got["cu_seqlens"].data_ptr()),
                                         ctypes.c_void_p(got["n_admitted"].data_ptr()),
                                         ctypes.c_void_p(got["theta"].data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        torch.cuda.synchronize()
        _compare(got, ref)
        print("noalloc mode %d R=%d: n_admitted %d" % (mode, R, int(got["n_admitted"].item())), flush=True)


def test_noalloc_binding_and_empty_batch(lib):
    from draft_verify_schedule_amd import binding as b
    rng = np.random.default_rng(12)
    c = torch.from_numpy(rng.uniform(0.2, 1.0, size=(300, 5)).astype(np.float32)).to(DEV)
    sps = torch.from_numpy(1000.0 / (1.0 + np.arange(300 * 6 + 1) / 64.0)).to(DEV)
    _compare(b.dspark_schedule_noalloc(c, sps, 0), b.dspark_schedule(c, sps, 0))
    e = _outputs(0, 5)
    b.dspark_schedule_noalloc(torch.empty((0, 5), dtype=torch.float32, device=DEV), sps, 0, out=e)
    torch.cuda.synchronize()
    assert int(e["cu_seqlens"][0]) == 0 and int(e["n_admitted"][0]) == 0 and float(e["theta"][0]) == 0.0


def test_noalloc_refuses_sizes_past_the_array(lib):
    NULL = ctypes.c_void_p(0)
    FAKE = ctypes.c_void_p(0x100000)
    # 1025 x 16 = 16400 candidates: one more request than the array holds
    assert lib.dspark_schedule_noalloc(1025, 16, FAKE, FAKE, 1025 * 17 + 1, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       NULL) == -2
