"""Seeded synthetic inputs for the W4A4 + LoRA linear layer.

This module only draws random numbers and casts them to the storage types
(fp16 for X, W, L_down, L_up; fp32 for the column scale a and bias b).  It
holds none of the layer's arithmetic, so both the HIP path and the CPU oracle
may take their inputs from it.

Workloads (shapes written M x K x N, LoRA rank R, quantization group 64):

* ``small``      16 x 256 x 256, R=16: X ~ N(0,1), W ~ N(0,0.02).
* ``mlp_up``     700 x 1024 x 3072, R=32: the MLP up-projection of a Qwen3-0.6B
                 class backbone at a 700-token batch (hidden 1024 -> 3072, the
                 shapes in "W4A4 CUDA Kernel for Voice Clone", section 3.1);
                 X ~ N(0,1) with 8 outlier channels scaled x20.
* ``mlp_down``   700 x 3072 x 1024, R=32: the matching down-projection;
                 X = SiLU(u) * v with u, v ~ N(0,1); W ~ N(0,0.015).
* ``decode``     M in {1, 4, 16} x 4096 x 14336, R=32: an 8B-class decode
                 layer; one W shared by all M, X drawn per M.
* ``prefill``    8192 x 4096 x 4096, R=32: Student-t (nu=3) X with 1% of the
                 channels (41 of 4096) scaled x30; a ~ U(0.5,2), b ~ N(0,0.05).

Everywhere: L_down, L_up ~ N(0,0.02); unless stated a ~ U(0.9,1.1) and
b ~ N(0,0.01).  N(0, s) means standard deviation s.  Draws are made in fp64
with numpy's PCG64 ``default_rng(seed)`` and then rounded to nearest-even into
the storage type.  Draw order: outlier channel indices, X, W, L_down, L_up,
a, b.  Outlier channels are columns of X (K indices), chosen without
replacement; the whole column is multiplied before the fp16 cast.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import numpy as np

BASE_SEED = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    R: int
    index: int                      # position in the workload list (seed offset)
    x_kind: str = "normal"          # normal | silu_mul | student_t3
    n_outliers: int = 0
    outlier_scale: float = 1.0
    w_std: float = 0.02
    lora_std: float = 0.02
    a_range: tuple = (0.9, 1.1)
    b_std: float = 0.01
    m_sweep: tuple = field(default=())   # decode: several M share one W

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index


WORKLOADS = {
    "small": Workload("small", 16, 256, 256, 16, 0),
    "mlp_up": Workload("mlp_up", 700, 1024, 3072, 32, 1, n_outliers=8, outlier_scale=20.0),
    "mlp_down": Workload("mlp_down", 700, 3072, 1024, 32, 2, x_kind="silu_mul", w_std=0.015),
    "decode": Workload("decode", 16, 4096, 14336, 32, 3, m_sweep=(1, 4, 16)),
    "prefill": Workload("prefill", 8192, 4096, 4096, 32, 4, x_kind="student_t3",
                        n_outliers=41, outlier_scale=30.0, a_range=(0.5, 2.0), b_std=0.05),
}


def _draw_x(rng: np.random.Generator, w: Workload, M: int, outlier_cols) -> np.ndarray:
    K = w.K
    if w.x_kind == "normal":
        x = rng.standard_normal((M, K))
    elif w.x_kind == "silu_mul":
        u = rng.standard_normal((M, K))
        v = rng.standard_normal((M, K))
        x = (u / (1.0 + np.exp(-u))) * v
    elif w.x_kind == "student_t3":
        x = rng.standard_t(3.0, size=(M, K))
    else:
        raise ValueError(w.x_kind)
    if len(outlier_cols):
        x[:, outlier_cols] *= w.outlier_scale
    return x.astype(np.float16)


def generate(name: str, M: int | None = None, seed: int | None = None,
             rows: int | None = None) -> dict:
    """Draw one workload's inputs.

    ``M`` overrides the row count (the decode workload uses M in {1,4,16}; X is
    then drawn from ``seed + M`` while W and the LoRA factors keep the
    workload's own seed).  ``rows`` truncates X after drawing (for cheap CPU
    timing samples of the same distribution).

    Returns a dict of numpy arrays: x fp16 [M,K], w fp16 [N,K],
    lora_down fp16 [K,R], lora_up fp16 [N,R], col_scale fp32 [N],
    bias fp32 [N], plus the shape ints.
    """
    w = WORKLOADS[name]
    M = w.M if M is None else int(M)
    base = w.seed if seed is None else int(seed)
    rng = np.random.default_rng(base)
    n_out = w.n_outliers
    outlier_cols = np.sort(rng.choice(w.K, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    if w.m_sweep:
        # weights come from the workload seed; X from seed + M
        x = _draw_x(np.random.default_rng(base + M), w, M, outlier_cols)
    else:
        x = _draw_x(rng, w, M, outlier_cols)
    wt = (rng.standard_normal((w.N, w.K)) * w.w_std).astype(np.float16)
    ld = (rng.standard_normal((w.K, w.R)) * w.lora_std).astype(np.float16)
    lu = (rng.standard_normal((w.N, w.R)) * w.lora_std).astype(np.float16)
    a = rng.uniform(w.a_range[0], w.a_range[1], size=w.N).astype(np.float32)
    b = (rng.standard_normal(w.N) * w.b_std).astype(np.float32)
    if rows is not None:
        x = x[:rows].copy()
    return dict(x=x, w=wt, lora_down=ld, lora_up=lu, col_scale=a, bias=b,
                M=x.shape[0], K=w.K, N=w.N, R=w.R, outlier_cols=outlier_cols)


def random_case(M: int, K: int, N: int, R: int, seed: int, x_scale: float = 1.0,
                w_std: float = 0.02) -> dict:
    """A generic seeded case of any shape (edge-case tests), same recipe as
    ``small``: X ~ N(0, x_scale), W ~ N(0, w_std), LoRA ~ N(0, 0.02),
    a ~ U(0.9, 1.1), b ~ N(0, 0.01)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * x_scale).astype(np.float16)
    wt = (rng.standard_normal((N, K)) * w_std).astype(np.float16)
    ld = (rng.standard_normal((K, R)) * 0.02).astype(np.float16)
    lu = (rng.standard_normal((N, R)) * 0.02).astype(np.float16)
    a = rng.uniform(0.9, 1.1, size=N).astype(np.float32)
    b = (rng.standard_normal(N) * 0.01).astype(np.float32)
    return dict(x=x, w=wt, lora_down=ld, lora_up=lu, col_scale=a, bias=b,
                M=M, K=K, N=N, R=R)
