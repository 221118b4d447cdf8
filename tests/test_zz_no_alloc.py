"""The allocation-free backward (flash_attn_bwd_noalloc, workspace in the
library's fixed device array) against flash_attn_bwd with a caller workspace:
the same kernels, so the gradients must agree bit for bit.  Two calls in a
row, the second on a smaller problem, so the second finds the first's
contents in the shared array."""
import numpy as np
import pytest

from synth_inputs import normal_qkv, to_bf16

pytestmark = pytest.mark.gpu


def _case(B, H, N, d, causal, seed, dtype="bf16"):
    import torch
    import exact_attention_77_amd as fa
    print(f"noalloc case B{B} H{H} N{N} d{d} causal={causal} {dtype}", flush=True)
    xs = normal_qkv(B, H, N, d, seed, with_dout=True)
    q, k, v, do = ((to_bf16(x)[0] if dtype == "bf16" else torch.from_numpy(x)).cuda() for x in xs)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=causal)
    ref = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=causal)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.flash_attn_bwd_noalloc(q, k, v, o, lse, do, *got, causal=causal)
    torch.cuda.synchronize()
    for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(r, g), name
        assert torch.isfinite(g.float()).all(), name
    return [t.float().cpu().numpy() for t in got]


def test_noalloc_matches_workspace_backward_twice():
    a = _case(2, 8, 1000, 128, True, 91)     # 16000 rows
    b = _case(1, 3, 300, 64, False, 92)      # 900 rows: a smaller second call
    assert np.isfinite(a[0]).all() and np.isfinite(b[0]).all()


def test_noalloc_fp32_twice():
    a = _case(1, 4, 700, 128, True, 94, "f32")
    b = _case(1, 2, 130, 64, False, 95, "f32")
    assert np.isfinite(a[0]).all() and np.isfinite(b[0]).all()


def test_noalloc_at_the_row_limit():
    # B * H * N = 2^21 rows exactly: the whole scratch array
    _case(1, 32, 65536, 64, True, 93)
