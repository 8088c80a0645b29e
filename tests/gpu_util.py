"""Shared helpers of the GPU parity tests: device upload of seeded inputs,
download as float64, the comparison metric and the tolerances."""
import numpy as np

import synthetic as syn

# Tolerances on max|gpu - oracle| / max|oracle| per output tensor.
TOL = {syn.BF16: 1e-2, syn.FP32: 1e-5}
TOL_CE = 1e-3


def dev(t, device="cuda"):
    """Upload a synthetic.Tensor (bf16 bit patterns or fp32) as a torch tensor."""
    import torch
    if t.dtype == syn.BF16:
        return torch.from_numpy(t.raw.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.raw)).to(device)


def host64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def assert_close(name, gpu, ref, tol):
    e = rel_err(gpu, ref)
    assert e <= tol, f"{name}: rel err {e:.3e} > {tol:.1e}"
    return e


def sample_idx(n, k, seed):
    """Sorted sample of row/column indices that always includes both ends and tile edges."""
    rng = np.random.default_rng(seed)
    fixed = [i for i in (0, 1, 127, 128, 255, 256, n - 2, n - 1) if 0 <= i < n]
    extra = rng.choice(n, size=min(n, k), replace=False)
    return np.unique(np.concatenate([np.array(fixed, dtype=np.int64), extra.astype(np.int64)]))


def tile_sample_idx(n, tile, seed, per_tile=1):
    """Sorted sample with `per_tile` random indices inside every `tile`-sized block of [0, n)
    (the last, partial block included) plus both ends, so that every tile of a tiled kernel's
    output is checked."""
    rng = np.random.default_rng(seed)
    idx = [0, n - 1]
    for t0 in range(0, n, tile):
        t1 = min(n, t0 + tile)
        idx += list(rng.integers(t0, t1, size=per_tile))
    return np.unique(np.array(idx, dtype=np.int64))


def rows(t, idx):
    """float64 copy of the selected rows of a device matrix."""
    import torch
    return host64(t[torch.as_tensor(idx, device=t.device)])


def cols(t, idx):
    """float64 copy of the selected columns of a device matrix."""
    import torch
    return host64(t[:, torch.as_tensor(idx, device=t.device)])
