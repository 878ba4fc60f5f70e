"""Helpers shared by the GPU parity tests (host <-> device marshalling and
comparisons).  No method arithmetic lives here."""
import os
import sys
import time

import numpy as np
import torch

from oracle.formats import bf16_value_from_bits

NEAR_TIE = 1e-6   # routing margin below which a mismatch is logged, not failed


# Progress lines also go to a file in the repository's output folder, so that
# a long test shows signs of life even while pytest captures its output.
_PROGRESS = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                         "gpurun_out", "gpu_tests_progress.log")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()
    try:
        os.makedirs(os.path.dirname(_PROGRESS), exist_ok=True)
        with open(_PROGRESS, "a") as f:
            f.write(time.strftime("%H:%M:%S ") + " ".join(str(x) for x in a) + "\n")
    except OSError:
        pass


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_bits_host(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values_host(t):
    return bf16_value_from_bits(bf16_bits_host(t))


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (2^(e-7) in binade [2^e, 2^(e+1)))."""
    v = np.abs(np.asarray(v, np.float64))
    _, ex = np.frexp(np.maximum(v, 2.0 ** -126))
    return np.ldexp(1.0, ex - 1 - 7)


def assert_within_one_bf16_ulp(gpu, ref, what, acc_bound=None):
    """|gpu - ref| <= one bf16 ulp, plus `acc_bound` (per element) when the
    GPU's fp32 accumulation error must be added (cancelling sums)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(gpu - ref)
    tol = bf16_ulp(np.maximum(np.abs(gpu), np.abs(ref)))
    if acc_bound is not None:
        tol = tol + acc_bound
    bad = np.argwhere(d > tol)
    assert bad.size == 0, f"{what}: {len(bad)} elements differ by more than one bf16 ulp, first {bad[:5].tolist()}"
    n_diff = int((d > 0).sum())
    log(f"[{what}] elements differing by one bf16 ulp: {n_diff} of {d.size}")
    return n_diff


def compare_routes(gpu_idx, ora, label, thresh=NEAR_TIE):
    """Routing indices must be bit-equal except tokens whose FP64 margin is
    below `thresh`; those are logged.  Returns the mismatching tokens."""
    gpu_idx = np.asarray(gpu_idx)
    mism = np.where((gpu_idx != ora["idx"]).any(axis=1))[0]
    bad = []
    for t in mism:
        m = float(ora["margin"][t])
        log(f"[near-tie] {label} token {t}: margin {m:.3e} gpu {gpu_idx[t].tolist()} "
            f"oracle {ora['idx'][t].tolist()}")
        if m >= thresh:
            bad.append(t)
    assert not bad, f"{label}: routing differs on tokens with margin >= {thresh}: {bad[:10]}"
    log(f"[route] {label}: {len(mism)} near-tie tokens of {len(gpu_idx)}; "
        f"min margin {float(np.min(ora['margin'])):.3e}")
    return mism
