"""Throughput over sequence length on one GPU, on the grid the
"FlashAttention-3" page benchmarks (実験設定): batch x seqlen = 16k tokens,
N = 512 .. 16k, with and without the causal mask, head_dim 64 and 128; the
head count (16 by default) is not given there.  bf16 forward and backward, and (d = 128) the fp8 forward on the
pre-pass outputs.  Seeded random inputs already in HBM; each point is the best
of three batches of 20 back-to-back launches after a settle phase of 200
headline-shaped launches.  Prints one JSON object per point.

    python -m exact_attention_77_amd.sweep [--heads 16] [--tokens 16384]
"""
from __future__ import annotations

import argparse
import json


def _timeit(step, n=20):
    import torch
    for _ in range(5):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        e0.record()
        for _ in range(n):
            step()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / n)
    return best


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--heads", type=int, default=16)
    ap.add_argument("--tokens", type=int, default=16384)
    args = ap.parse_args()

    import torch

    import exact_attention_77_amd as fa

    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    H = args.heads
    x = torch.randn(2, 16, 8192, 128, device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(200):   # settle the clock
        fa.flash_attn_fwd(x, x, x, causal=True)
    torch.cuda.synchronize()
    del x
    signs = (torch.randint(0, 2, (128,), device="cuda", dtype=torch.int8, generator=g) * 2 - 1).to(torch.int8)
    for d in (64, 128):
        for N in (512, 1024, 2048, 4096, 8192, 16384):
            B = max(1, args.tokens // N)
            for causal in (False, True):
                q, k, v, do = (torch.randn(B, H, N, d, device="cuda", dtype=torch.bfloat16, generator=g)
                               for _ in range(4))
                fl = 4.0 * B * H * N * N * d / (2 if causal else 1)
                ms = _timeit(lambda: fa.flash_attn_fwd(q, k, v, causal=causal))
                o, lse = fa.flash_attn_fwd(q, k, v, causal=causal)
                msb = _timeit(lambda: fa.flash_attn_bwd(q, k, v, o, lse, do, causal=causal))
                rec = {"B": B, "H": H, "N": N, "d": d, "causal": causal,
                       "bf16_fwd_tflops": round(fl / ms / 1e9, 1),
                       "bf16_bwd_tflops": round(2.5 * fl / msb / 1e9, 1)}
                if d == 128:
                    qf, kf, vf = (t.float() for t in (q, k, v))
                    q8, qs = fa.flash_attn_fp8_quantize(qf, fa.ROLE_Q, rotate=True, signs=signs)
                    k8, ks = fa.flash_attn_fp8_quantize(kf, fa.ROLE_K, rotate=True, signs=signs)
                    v8, vs = fa.flash_attn_fp8_quantize(vf, fa.ROLE_V)
                    del qf, kf, vf
                    ms8 = _timeit(lambda: fa.flash_attn_fwd_fp8(q8, k8, v8, qs, ks, vs, causal=causal))
                    rec["fp8_fwd_tflops"] = round(fl / ms8 / 1e9, 1)
                    del q8, k8, v8
                print(json.dumps(rec), flush=True)
                del q, k, v, do, o, lse


if __name__ == "__main__":
    main()
