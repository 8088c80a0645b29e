"""The allocation-free CE entry point against the workspace one, through the
C ABI: two calls in a row on the library's per-GPU scratch array, the second
with a smaller input, each compared bit for bit with tp_vocab_ce_partials on
the same inputs (the two share their kernels, so the results must be equal)."""
import numpy as np
import pytest

import synthetic as syn

from .gpu_util import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tp = pytest.importorskip("tensor_transformer_linear_tp_amd")


def _run_both(M, Vr, K, seed, v0):
    H = dev(syn.normal(seed, (M, K), 1.0, syn.BF16))
    W = dev(syn.normal(seed + 1, (Vr, K), 0.3, syn.BF16))
    target = np.random.default_rng(seed + 2).integers(v0 - 100, v0 + Vr + 100, size=M).astype(np.int32)
    td = torch.from_numpy(target).cuda()
    outs = []
    for noalloc in (True, False):
        m, s, t = (torch.full((M,), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3))
        if noalloc:
            tp.tp_vocab_ce_partials_noalloc(tp.TP_BF16, M, Vr, K, H, K, W, K, td, v0, m, s, t)
        else:
            n = tp.tp_vocab_ce_workspace_bytes(M, Vr)
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
            tp.tp_vocab_ce_partials(tp.TP_BF16, M, Vr, K, H, K, W, K, td, v0, m, s, t, ws, n)
        outs.append((m, s, t))
    torch.cuda.synchronize()
    return outs


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # First call: 2048 tokens x 4000 vocab rows (16 column tiles, a ragged last one;
    # the scratch holds 2*16 + 1 arrays of 2048 floats).  Second call: fewer tokens
    # and vocab rows, reading only what it writes of the same scratch.
    for (M, Vr, K, seed, v0) in ((2048, 4000, 136, 6100, 500), (300, 700, 72, 6200, 0)):
        (a, b) = _run_both(M, Vr, K, seed, v0)
        for name, x, y in zip(("max", "sumexp", "tgt"), a, b):
            xa, ya = x.cpu().numpy(), y.cpu().numpy()
            assert np.all(np.isfinite(xa)), name
            assert np.array_equal(xa.view(np.uint32), ya.view(np.uint32)), f"{name} differs at M={M}"


def test_noalloc_rejects_shapes_past_the_scratch():
    M, Vr, K = 8192, 65281, 8
    H = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(8, K, dtype=torch.bfloat16, device="cuda")   # never read: rejected before any launch
    td = torch.zeros(M, dtype=torch.int32, device="cuda")
    m, s, t = (torch.zeros(M, dtype=torch.float32, device="cuda") for _ in range(3))
    with pytest.raises(tp.TPError) as ei:
        tp.tp_vocab_ce_partials_noalloc(tp.TP_BF16, M, Vr, K, H, K, W, K, td, 0, m, s, t)
    assert ei.value.status == 6
    torch.cuda.synchronize()
    assert float(m.abs().sum()) == 0.0
