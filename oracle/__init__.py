"""CPU oracle for the FP4 rollout hot path -- TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct reference that the HIP path is
checked against. Only the test-suite, the smoke check and the benchmark's CPU
baseline may import it; the product library never does, and shares no code,
tables or helpers with it.

Sources (the method's pages):
  * "Sol-RL: FP4 Explore, BF16 Train" project page (nvlabs), section
    "Two-Stage Pipeline": N noises, an FP4-quantized solver, proxy rewards,
    top/bottom-K seed filter, per-iteration weight re-quantization.
  * aitrends.kr summary of the same paper, paragraphs on Stage 1 / Stage 2:
    6 FP4 solver steps, top K/2 and bottom K/2 seeds, weights re-quantized to
    FP4 after every update.
  * VeRL-Omni "DiffusionNFT" docs, section "Algorithm": the clipped reward
    normalisation r = 1/2 + 1/2 clip((r_raw - E r_raw)/Z, -1, 1), and the
    implicit positive / negative branch loss of the policy update.

The pages do not define the FP4 block formats; the two formats implemented
here (MXFP4: E2M1 + E8M0 per 32; NVFP4-style: E2M1 + E4M3 per 16 + fp32 tensor
scale) and every other reading of a silent passage are listed in the
repository's design notes.

Arithmetic is numpy float64 (exact where the result is exactly representable)
except where the format itself fixes fp32 steps (the NVFP4-style scale chain).

Parity status per function:
  e2m1.encode / decode ........ pinned (hand grid, midpoints, threshold table)
  mxfp4.quantize / dequant .... pinned (hand-worked blocks, round trip,
                                idempotence, sign and power-of-two symmetry)
  nvfp4.quantize / dequant .... pinned (hand-worked blocks, torch float8 cast,
                                brute-force code search)
  gemm.gemm_mx / gemm_nv ...... pinned (exact rationals, exact-integer case,
                                one-hot, identity)
  euler ....................... pinned (constant-field closed form, dt=0)
  reward / select ............. pinned (hand cases, brute-force sort,
                                permutation equivariance)
  rollout.gelu / rmsnorm ...... pinned (normal-CDF table values, the identity
                                GELU(z) - GELU(-z) = z, Mills-ratio tail series;
                                hand row, constant rows, mean-square identity)
  lora.merge .................. pinned (exact rationals on small non-square
                                shapes, all-ones and rank-one closed forms,
                                s = 0 and B = 0 identities)
  nft.noise / loss_terms ...... pinned (exact rationals, beta = 0 and equal-
                                velocity identities, r = 0 / 1 branch
                                selection, noising end points and slope)
  rollout (composite) ......... pinned (one token through one and two
                                velocity blocks, an Euler step and the
                                reward, in exact rationals, with plausible
                                mis-compositions shown to miss; the bf16
                                reading of the hidden activation by a block
                                where the two readings differ, and its
                                rounding against torch's casts)
"""
from . import e2m1, mxfp4, nvfp4, gemm, euler, reward, rollout, lora, nft  # noqa: F401
