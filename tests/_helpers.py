"""Shared pieces of the GPU parity tests."""
import sys

import torch

import oracle

# Tolerances on the per-row max-norm relative error ||x - y||_inf / ||y||_inf
# against the fp64 oracle: fp32 inputs compute in fp32 throughout; bf16 inputs
# accumulate in fp32 but the output is rounded to bf16 (2^-9 relative) and the
# MLA P operand is rounded to bf16 before the MFMA.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def tol_for(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(t):
    return None if t is None else t.to("cuda")


def rows_sample(n_rows, k, seed=0):
    """Deterministic sample of k flat row ids, always including the first and last."""
    g = torch.Generator().manual_seed(seed)
    pick = torch.randperm(n_rows, generator=g)[: max(0, k - 2)].tolist()
    return sorted(set([0, n_rows - 1] + pick))


def assert_rows_close(got, want, tol, what=""):
    err = oracle.rel_err_rows(got, want)
    assert err <= tol, f"{what}: max row rel err {err:.3e} > {tol:.1e}"
    return err


def assert_lse_close(got, want, tol, what=""):
    got = got.double().cpu().reshape(-1)
    want = want.double().cpu().reshape(-1)
    inf_g, inf_w = torch.isinf(got), torch.isinf(want)
    assert torch.equal(inf_g, inf_w), f"{what}: -inf pattern differs"
    fin = ~inf_w
    if fin.any():
        d = (got[fin] - want[fin]).abs().max().item()
        assert d <= tol * max(1.0, want[fin].abs().max().item()), f"{what}: lse diff {d:.3e}"
