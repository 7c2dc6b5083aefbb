"""Seeded synthetic inputs for the NF4 path.

This module only draws random numbers and shapes them into the workloads the
NF4 path is measured on; it contains none of the quantization arithmetic, so
that the CPU oracle and the HIP library can both be fed from it without
sharing any of the method's code.

Workloads (weights are row-major [out_features, in_features]):

  C1  one 1024x1024 fp32 weight ~ N(0, 0.02); x bf16 [1024] ~ N(0, 1); no
      double quantization.
  C2  one 4096x4096 weight ~ N(0, 0.02) with 0.1 % of entries scaled by 20,
      rounded once to bf16; x bf16 [4096] ~ N(0, 1); double quantization.
  C3  Llama-8B-shaped MLP: gate and up [14336, 4096], down [4096, 14336],
      bf16 ~ N(0, 0.02); X bf16 [M, K] ~ N(0, 1) for M in (1, 4, 16).
  C4  X bf16 [4096, 4096] ~ N(0, 1); W bf16 [14336, 4096] ~ N(0, 0.02);
      LoRA A bf16 [16, 4096], B bf16 [14336, 16] ~ N(0, 0.01); alpha 32.
      Its backward takes dY bf16 [4096, 14336] ~ N(0, 1).
  C5  70B-shaped layer: q, o [8192, 8192]; k, v [1024, 8192]; gate, up
      [28672, 8192]; down [8192, 28672]; bf16 ~ N(0, 0.02).

Recipe: numpy PCG64 (`default_rng(seed)`), float32 standard normals times the
standard deviation in float32, outliers multiplied by 20 in float32 at
round(0.001 n) distinct positions drawn without replacement, then one
round-to-nearest-even cast to bf16.  Seeds are 1000 * workload + tensor id
(0 weight, 1/2 further MLP weights, 5 activations, 6 LoRA A, 7 LoRA B,
8 output gradients, 9 outlier positions).  C5 is drawn on the device with torch generators seeded
5_000_000 + 10 * layer + matrix index (q, k, v, o, gate, up, down = 0..6).
"""

from __future__ import annotations

import numpy as np

SEED_W, SEED_W1, SEED_W2, SEED_X, SEED_A, SEED_B, SEED_DY, SEED_OUTLIER = 0, 1, 2, 5, 6, 7, 8, 9

C3_SHAPES = {"gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336)}
C5_SHAPES = {
    "q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
    "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672),
}
C5_ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def seed(workload: int, tensor_id: int) -> int:
    return 1000 * workload + tensor_id


def normal_f32(shape, std: float, seed_value: int) -> np.ndarray:
    """float32 N(0, std^2) samples (std is the standard deviation)."""
    rng = np.random.default_rng(seed_value)
    z = rng.standard_normal(size=shape, dtype=np.float32)
    return z * np.float32(std)


def add_outliers(w: np.ndarray, fraction: float, factor: float, seed_value: int) -> np.ndarray:
    """Scale round(fraction * n) distinct, uniformly drawn entries by `factor` in float32."""
    flat = w.reshape(-1).copy()
    k = int(round(fraction * flat.size))
    rng = np.random.default_rng(seed_value)
    pos = rng.choice(flat.size, size=k, replace=False)
    flat[pos] = flat[pos] * np.float32(factor)
    return flat.reshape(w.shape)


def to_bf16(a: np.ndarray):
    """One round-to-nearest-even cast to a torch bfloat16 CPU tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f32(t) -> np.ndarray:
    """Exact widening of a torch bfloat16 tensor to a float32 numpy array."""
    import torch
    return t.detach().to("cpu").to(torch.float32).numpy()


# ---------------------------------------------------------------- workloads

def c1_inputs():
    w = normal_f32((1024, 1024), 0.02, seed(1, SEED_W))
    x = to_bf16(normal_f32((1, 1024), 1.0, seed(1, SEED_X)))
    return {"w_f32": w, "x": x}


def c2_weight(rows: int = 4096, cols: int = 4096, pool_index: int = 0):
    """C2 weight; pool_index > 0 gives further distinct draws of the same recipe."""
    base = 100_000 * pool_index
    w = normal_f32((rows, cols), 0.02, seed(2, SEED_W) + base)
    w = add_outliers(w, 0.001, 20.0, seed(2, SEED_OUTLIER) + base)
    return to_bf16(w)


def c2_inputs():
    return {"w": c2_weight(), "x": to_bf16(normal_f32((1, 4096), 1.0, seed(2, SEED_X)))}


def c3_weight(name: str, scale_rows: int | None = None):
    rows, cols = C3_SHAPES[name]
    if scale_rows is not None:
        rows = scale_rows
    tid = {"gate": SEED_W, "up": SEED_W1, "down": SEED_W2}[name]
    return to_bf16(normal_f32((rows, cols), 0.02, seed(3, tid)))


def c3_x(m: int, k: int):
    return to_bf16(normal_f32((m, k), 1.0, seed(3, SEED_X) + 10 * m + (k % 7)))


def c4_inputs(m: int = 4096, n: int = 14336, k: int = 4096, r: int = 16):
    return {
        "x": to_bf16(normal_f32((m, k), 1.0, seed(4, SEED_X))),
        "w": to_bf16(normal_f32((n, k), 0.02, seed(4, SEED_W))),
        "a": to_bf16(normal_f32((r, k), 0.01, seed(4, SEED_A))),
        "b": to_bf16(normal_f32((n, r), 0.01, seed(4, SEED_B))),
        "alpha": 32.0,
        "r": r,
    }


def c4_grad(m: int = 4096, n: int = 14336):
    """The output gradient dY [m, n] of the C4 layer (bf16 ~ N(0, 1))."""
    return to_bf16(normal_f32((m, n), 1.0, seed(4, SEED_DY)))


def c5_weight_device(layer: int, name: str, device="cuda"):
    """One C5 weight drawn on the device (bf16)."""
    import torch
    rows, cols = C5_SHAPES[name]
    g = torch.Generator(device=device)
    g.manual_seed(5_000_000 + 10 * layer + C5_ORDER.index(name))
    w = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    w.mul_(0.02)
    return w.to(torch.bfloat16)


def random_blocks_f32(n: int, seed_value: int, kinds=("normal", "uniform", "wide")) -> np.ndarray:
    """Mixed-distribution float32 data for edge-case sweeps (not a workload)."""
    rng = np.random.default_rng(seed_value)
    parts = []
    per = -(-n // len(kinds))
    for kind in kinds:
        if kind == "normal":
            parts.append(rng.standard_normal(per, dtype=np.float32))
        elif kind == "uniform":
            parts.append(rng.uniform(-3, 3, per).astype(np.float32))
        elif kind == "wide":
            mant = rng.uniform(1, 2, per)
            sign = rng.choice([-1.0, 1.0], per)
            expo = rng.integers(-140, 120, per)
            parts.append((sign * np.ldexp(mant, expo)).astype(np.float32))
    return np.concatenate(parts)[:n]
