"""moe_permute_noalloc (the entry point for callers that cannot allocate:
graph capture, serving loops, harnesses that forbid hipMalloc) against
moe_permute with a caller workspace, through the C ABI: identical offsets,
perm_src, inv_perm and gathered rows (integer and byte work, so bit for
bit), on two calls in a row, the second with a smaller input; and a size
past the static scratch rejected with MOE_ERR_WORKSPACE before any launch."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_bias_amd as M
from fp8_block_scaled_bias_amd import _lib as L
from gpu_common import dev, host, log

pytestmark = pytest.mark.gpu


def _case(T, k, E, H, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    xq = rng.integers(0, 256, (T, H), dtype=np.uint8)
    xs = rng.standard_normal((T, H // 128)).astype(np.float32)
    return idx, counts, xq, xs


def _outputs(T, k, E, H, ns):
    R = T * k + ns * T
    i32 = dict(dtype=torch.int32, device="cuda")
    return (torch.full((E + ns + 1,), -7, **i32), torch.full((max(R, 1),), -7, **i32),
            torch.full((max(T * k, 1),), -7, **i32),
            torch.zeros((max(R, 1), H), dtype=torch.uint8, device="cuda"),
            torch.zeros((max(R, 1), H // 128), dtype=torch.float32, device="cuda"))


def _run(noalloc, idx, counts, xq, xs, E, H, ns):
    T, k = idx.shape
    off, ps, inv, a, sa = _outputs(T, k, E, H, ns)
    args = (dev(idx), dev(counts), T, k, E, ns, off, ps, inv, dev(xq), dev(xs), H, a, sa)
    if noalloc:
        M.moe_permute_noalloc(*args)
    else:
        wsb = max(16, M.moe_permute_workspace_bytes(T, k, E))
        ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
        M.moe_permute(*args, ws, wsb)
    return [host(t) for t in (off, ps, inv, a, sa)]


def test_permute_noalloc_equals_workspace_form():
    for T, k, E, ns, seed in ((16384, 8, 256, 1, 1), (777, 6, 64, 0, 2)):   # larger, then smaller
        idx, counts, xq, xs = _case(T, k, E, 256, seed)
        log(f"[noalloc] T={T} k={k} E={E} n_shared={ns}")
        ref = _run(False, idx, counts, xq, xs, E, 256, ns)
        got = _run(True, idx, counts, xq, xs, E, 256, ns)
        for name, a, b in zip(("offsets", "perm_src", "inv_perm", "rows", "scales"), got, ref):
            assert np.array_equal(a, b), f"T={T}: {name} differs"


def test_permute_noalloc_rejects_past_the_scratch():
    T, k, E = 65536 + 64, 8, 256          # ceil(T/64) * E = 262400 > 262144 int32
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    counts = torch.zeros((E,), dtype=torch.int32, device="cuda")
    off, ps, inv = (torch.empty((E + 2,), dtype=torch.int32, device="cuda"),
                    torch.empty((T * k + T,), dtype=torch.int32, device="cuda"),
                    torch.empty((T * k,), dtype=torch.int32, device="cuda"))
    with pytest.raises(M.MoEError) as ex:
        M.moe_permute_noalloc(idx, counts, T, k, E, 1, off, ps, inv, None, None, 128, None, None)
    assert ex.value.code == L.MOE_ERR_WORKSPACE
    log(f"[noalloc] rejected: {ex.value}")
