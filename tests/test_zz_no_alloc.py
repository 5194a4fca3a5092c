"""The allocation-free routing entry point (bsg_route_noalloc, its counts in
the library's static device array) against bsg_route with a caller
workspace: the same kernels, so every output must match bit for bit, on two
calls in a row, the second smaller (the array keeps the first call's
contents)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _route_both(T, E, k, renorm, bin_rows, seed):
    from block_sparse_gemm_amd import bsg
    print(f"[no_alloc] T={T} E={E} k={k} renorm={renorm} bin_rows={bin_rows} seed={seed}",
          flush=True)
    rng = np.random.default_rng(seed)
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    outs = []
    for noalloc in (True, False):
        # poisoned outputs: stale values cannot pass for results
        o = dict(expert_idx=torch.full((T * k,), -7, **i32),
                 gate=torch.full((T * k,), float("nan"), device="cuda"),
                 dest_row=torch.full((T * k,), -7, **i32),
                 counts=torch.full((E,), -7, **i32),
                 bin_offsets=torch.full((E + 1,), -7, **i32))
        args = (logits, k, renorm, o["expert_idx"], o["gate"], o["dest_row"], o["counts"],
                o["bin_offsets"])
        if noalloc:
            bsg.route_noalloc(*args, bin_rows=bin_rows)
        else:
            ws = torch.zeros(bsg.route_workspace_bytes(T, k, E), dtype=torch.uint8, device="cuda")
            bsg.route(*args, ws, bin_rows=bin_rows)
        torch.cuda.synchronize()
        outs.append(o)
    return outs


def test_route_noalloc_matches_route_twice():
    from block_sparse_gemm_amd import bsg
    # the largest first, then a smaller one: fewer chunks and experts than the
    # counts the array still holds from the first call
    for T, E, k, renorm, bin_rows, seed in ((65536, 64, 2, False, 128, 1),
                                           (777, 40, 3, True, 256, 2)):
        assert bsg.route_workspace_bytes(T, k, E) <= bsg.ROUTE_SCRATCH_BYTES
        got, want = _route_both(T, E, k, renorm, bin_rows, seed)
        for key in ("expert_idx", "dest_row", "counts", "bin_offsets"):
            assert torch.equal(got[key], want[key]), key
        assert torch.equal(got["gate"].view(torch.int32), want["gate"].view(torch.int32)), "gate"
        assert int(got["counts"].sum()) == T * k


def test_route_noalloc_refuses_more_than_its_scratch():
    from block_sparse_gemm_amd import bsg
    T, E, k = 64 * 1025, 1024, 1          # 1025 chunks x 1024 experts x 4 bytes > 4 MiB
    assert bsg.route_workspace_bytes(T, k, E) > bsg.ROUTE_SCRATCH_BYTES
    logits = torch.zeros(T, E, device="cuda")
    out = torch.zeros(T * k, dtype=torch.int32, device="cuda")
    with pytest.raises(bsg.BsgError) as ei:
        bsg.route_noalloc(logits, k, False, out, out.float(), out, out[:E], out[:E + 1])
    assert ei.value.status == bsg.EUNSUPPORTED
