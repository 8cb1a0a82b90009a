"""The synthetic workloads: shapes, distributions and seeds.

Recipes only -- no arithmetic of the method.  The pages measure on real LLM
serving (Qwen3 models, GSM8K, MBPP, Civil Comments); none of those models or
datasets is used or reproduced.  Seeded Gaussian tensors at Llama-shaped
projection sizes stand in for the activations and weights such workloads
would produce.  ``std`` is the standard deviation.

  tiny      GEMM Y[M,1024] = X[M,1024] . W^T, W [1024,1024], and RMSNorm (w = 1,
            eps = 1e-6) on the same X; X, W ~ N(0, 1/1024); M in {1, 3, 16, 64}.
  rmsnorm   X[M,4096] ~ N(0,1), w ~ N(1, 0.1^2), eps = 1e-6; M in {1,7,128,2048,8192}.
  llama8b   K=4096 with N in {4096, 1024, 14336}, and K=14336 with N=4096;
            X ~ N(0,1), W ~ N(0, 0.02^2); M swept over 1..8192.
  lora      X[M,4096] ~ N(0,1), A[16,4096] ~ N(0, 0.01^2) -> fp32 [M,16];
            split-K 8 deterministic vs atomic vs unsplit; M in {1,8,64,512,4096};
            1000 identical-input replays.
  llama70b  K=8192, N=28672 under a dynamic-batch stream: 200 batches, M ~ U{1..4096},
            8 probe rows at random positions, other rows from a 4096-row pool.
"""
from __future__ import annotations

import numpy as np

from . import synth

EPS = float(np.float32(1e-6))

TINY = dict(name="tiny", K=1024, N=1024, Ms=(1, 3, 16, 64), std=1.0 / 32,
            x_seed=1001, w_seed=1002, perm_seed=1003)

RMSNORM = dict(name="rmsnorm_k4096", K=4096, Ms=(1, 7, 128, 2048, 8192),
               x_seed=2001, w_seed=2002, perm_seed=2003, w_mean=1.0, w_std=0.1)

LLAMA8B = dict(
    name="llama3_8b_projections",
    shapes=((4096, 4096), (4096, 1024), (4096, 14336), (14336, 4096)),   # (K, N)
    Ms=(1, 5, 33, 127, 1000, 4096, 8192),
    # real primes and awkward tails beside the listed sizes
    extra_Ms=(2, 3, 7, 17, 31, 64, 128, 257, 509, 2039, 2048, 4093, 8191),
    x_seeds={4096: 3001, 14336: 3002}, w_seeds=(3011, 3012, 3013, 3014), perm_seed=3020,
    w_std=0.02, pool_rows=8192)

LORA = dict(name="lora_shrink", K=4096, R=16, Ms=(1, 8, 64, 512, 4096), split_k=8,
            x_seed=4001, a_seed=4002, pos_seed=4003, a_std=0.01, replays=1000)

LLAMA70B = dict(name="llama3_70b_mlp_stream", K=8192, N=28672, n_batches=200, m_max=4096,
                pool_rows=4096, n_probes=8, x_seed=5001, w_seed=5002, m_seed=5003,
                probe_seed=5004, w_std=0.02)


def tiny_inputs():
    c = TINY
    x = synth.normal_bf16((max(c["Ms"]), c["K"]), c["x_seed"], std=c["std"])
    w = synth.normal_bf16((c["N"], c["K"]), c["w_seed"], std=c["std"])
    ones = np.full(c["K"], 0x3F80, dtype=np.uint16)
    return x, w, ones


def rmsnorm_inputs():
    c = RMSNORM
    x = synth.normal_bf16((max(c["Ms"]), c["K"]), c["x_seed"])
    w = synth.normal_bf16((c["K"],), c["w_seed"], mean=c["w_mean"], std=c["w_std"])
    return x, w


def llama8b_x(K: int, rows: int | None = None):
    c = LLAMA8B
    return synth.normal_bf16((rows or c["pool_rows"], K), c["x_seeds"][K])


def llama8b_w(shape_index: int):
    c = LLAMA8B
    K, N = c["shapes"][shape_index]
    return synth.normal_bf16((N, K), c["w_seeds"][shape_index], std=c["w_std"])


def lora_inputs(M: int | None = None):
    c = LORA
    x = synth.normal_bf16((M or max(c["Ms"]), c["K"]), c["x_seed"])
    a = synth.normal_bf16((c["R"], c["K"]), c["a_seed"], std=c["a_std"])
    return x, a


def llama70b_stream():
    c = LLAMA70B
    probes, batches = synth.batch_stream(c["n_batches"], c["m_max"], c["pool_rows"],
                                         c["n_probes"], c["m_seed"], c["probe_seed"])
    return probes, batches


def llama70b_x_pool():
    c = LLAMA70B
    return synth.normal_bf16((c["pool_rows"], c["K"]), c["x_seed"])


def llama70b_w():
    c = LLAMA70B
    return synth.normal_bf16((c["N"], c["K"]), c["w_seed"], std=c["w_std"])
