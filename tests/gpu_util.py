"""Helpers shared by the GPU parity tests: host<->device marshalling, the
tolerances, row sampling.  No method arithmetic lives here."""
import sys

import numpy as np
import torch

# spec tolerances: fp32 configs max-abs 1e-5; bf16 and int8-KV configs
# max-abs 2e-2 and mean-abs 2e-3.
TOL_F32_MAX = 1e-5
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_input(w, name):
    """Device tensor holding exactly the values the oracle receives."""
    if w["dtype"] == "bf16":
        bits = w[name + "_bits"]
        return torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(w[name], dtype=np.float32)).to("cuda")


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev_opt(a, dtype):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to("cuda")


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {err.size} values")
    if dtype == "f32":
        assert mx <= TOL_F32_MAX, f"{what}: max-abs {mx} > {TOL_F32_MAX}"
    else:
        assert mx <= TOL_BF16_MAX, f"{what}: max-abs {mx} > {TOL_BF16_MAX}"
        assert mean <= TOL_BF16_MEAN, f"{what}: mean-abs {mean} > {TOL_BF16_MEAN}"


def assert_lse_close(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{what}: -inf pattern differs"
    d = np.abs(got[~inf_ref] - ref[~inf_ref])
    tol = 2e-5 if dtype == "f32" else 2e-2
    mx = float(d.max(initial=0.0))
    say(f"  {what} lse: max-abs {mx:.3e}")
    assert mx <= tol, f"{what}: lse max-abs {mx} > {tol}"


def sample_rows(rng, B, H, T, n, extra_t=()):
    """Flat row indices ((b*H + h)*T + t): n random rows plus every (b, h) at the given t."""
    rows = set(int(x) for x in rng.integers(0, B * H * T, size=n))
    for b in range(B):
        for h in range(H):
            for t in extra_t:
                if 0 <= t < T:
                    rows.add((b * H + h) * T + t)
    return np.array(sorted(rows), dtype=np.int64)
