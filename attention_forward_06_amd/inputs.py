"""Seeded synthetic inputs for the attention-forward workloads.

Holds shapes, seeds and the random draws only -- none of the attention
arithmetic -- so the HIP path and the CPU oracle can both be fed from it.

Recipe: one torch.Generator seeded with `seed` draws Q, K, V in that order as
float32 standard normals of shape [B, H, L, D], each scaled by `std`, then
rounded to nearest-even into the storage dtype.  The block-diagonal page's
quick check draws fp16 normals from seed 42; the fused-attention page's test
matrix draws N(0, 0.5) from seed 20.  When V is stored as fp8 e5m2 it is the
same float32 draw cast with torch's round-to-nearest-even conversion.
"""
import math

import torch

DTYPES = ("f16", "bf16", "bf16_v_e5m2", "f16_v_e5m2")

# Workloads shaped like the pages' (sizes, mask and dtype in the name).
WORKLOADS = {
    "blockdiag_b1_h2_n256_d128_bs64_f16":
        dict(mode="block_diag", B=1, H=2, L=256, D=128, dtype="f16", block_size=64),
    "dense_b4_h16_l2048_d64_f16":
        dict(mode="none", B=4, H=16, L=2048, D=64, dtype="f16", block_size=0),
    "causal_b4_h32_l4096_d128_bf16":
        dict(mode="causal", B=4, H=32, L=4096, D=128, dtype="bf16", block_size=0),
    "blockdiag_b8_h32_n16384_d128_bs64_f16":
        dict(mode="block_diag", B=8, H=32, L=16384, D=128, dtype="f16", block_size=64),
    "blockdiag_b8_h32_n16384_d128_bs128_f16":
        dict(mode="block_diag", B=8, H=32, L=16384, D=128, dtype="f16", block_size=128),
    "causal_b1_h16_l32768_d256_bf16_ve5m2":
        dict(mode="causal", B=1, H=16, L=32768, D=256, dtype="bf16_v_e5m2", block_size=0),
    # the small head dims the fused-attention page's wrapper also accepts
    "dense_b4_h16_l2048_d32_f16":
        dict(mode="none", B=4, H=16, L=2048, D=32, dtype="f16", block_size=0),
    "causal_b4_h32_l4096_d16_bf16":
        dict(mode="causal", B=4, H=32, L=4096, D=16, dtype="bf16", block_size=0),
    # the fp8-V variant with fp16 Q/K/O (the fp8 branch keys only on V's type)
    "causal_b1_h16_l32768_d256_f16_ve5m2":
        dict(mode="causal", B=1, H=16, L=32768, D=256, dtype="f16_v_e5m2", block_size=0),
}

# The non-causal test matrix of the fused-attention page: (Z, H, N_CTX, HEAD_DIM,
# dtype, BLOCK_M, BLOCK_N); seed 20, N(0, 0.5), sm_scale 0.5.
FUSED_PAGE_MATRIX = [
    (1, 1, 128, 128, "f16", 32, 128),
    (1, 1, 128, 128, "bf16", 64, 128),
    (1, 2, 256, 256, "bf16", 32, 256),
    (2, 2, 128, 256, "f16", 64, 128),
    (4, 32, 64, 64, "f16", 32, 64),
    (4, 32, 1024, 64, "bf16", 64, 128),
    (4, 32, 4096, 64, "f16", 128, 128),
]


def storage_dtypes(dtype):
    """torch dtypes of (q, k, v) for a dtype name."""
    if dtype == "f16":
        return torch.float16, torch.float16, torch.float16
    if dtype == "bf16":
        return torch.bfloat16, torch.bfloat16, torch.bfloat16
    if dtype == "bf16_v_e5m2":
        return torch.bfloat16, torch.bfloat16, torch.float8_e5m2
    if dtype == "f16_v_e5m2":
        return torch.float16, torch.float16, torch.float8_e5m2
    raise ValueError(f"unknown dtype {dtype!r}")


def default_scale(D):
    return 1.0 / math.sqrt(D)


def make_qkv(B, H, L, D, dtype, seed=42, std=1.0, device="cpu"):
    """Q, K, V as torch tensors [B, H, L, D] in their storage dtypes on `device`."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for dt in storage_dtypes(dtype):
        x = torch.randn((B, H, L, D), generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out.append(x.to(dt))
        del x
    return tuple(out)


def make_workload(name, seed=42, device="cpu"):
    w = WORKLOADS[name]
    q, k, v = make_qkv(w["B"], w["H"], w["L"], w["D"], w["dtype"], seed=seed, device=device)
    return q, k, v
