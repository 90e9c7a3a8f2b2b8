"""The five workloads the library is checked and measured on (synthetic inputs).

Each is named by what it is; sizes follow the pages' shapes: the itwiki demo
(q, k of width 16 and v of width 32, chunk 16), the velog review's length
sweep 2^9 .. 2^16 (section 4.3), and pixel-by-pixel generation of 32x32x3
images, 3072 steps (velog review section 4.4).
"""
from __future__ import annotations

CAUSAL_FP32_DEMO = dict(name="causal_fwd_fp32_B2_H1_N64_dk16_dv32_C16",
                        B=2, H=1, N=64, dk=16, dv=32, C=16, dtype="f32")
NONCAUSAL_BF16 = dict(name="noncausal_fwd_bf16_B4_H8_N4096_d64",
                      B=4, H=8, N=4096, dk=64, dv=64, dtype="bf16")
CAUSAL_BF16_SWEEP = dict(name="causal_fwd_bf16_B8_H8_d64_C64", B=8, H=8, dk=64, dv=64, C=64, dtype="bf16",
                         Ns=[2 ** e for e in range(9, 17)])
DECODE_FP32 = dict(name="decode_fp32_T3072_B256_H8_d32", T=3072, B=256, H=8, dk=32, dv=32, dtype="f32")
CAUSAL_FWD_BWD_BF16 = dict(name="causal_fwd_bwd_bf16_B8_H16_N8192_d128_C64",
                           B=8, H=16, N=8192, dk=128, dv=128, C=64, dtype="bf16")
