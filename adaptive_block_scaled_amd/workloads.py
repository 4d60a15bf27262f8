"""Seeded synthetic inputs for the IF4 path (shared by tests, the benchmark and
the oracle's callers).  Holds no quantization arithmetic: only random draws,
the bf16 cast and the per-tensor exponent rule, which is an input policy.

The pages measure on language-model weights, activations and gradients
(W4A4G4 training, W4A4 post-training quantization); none of those tensors
are available, so these draws stand in for them with the distributions
below.  Recipe (numpy PCG64 `default_rng`):
  * values are drawn in fp32 and cast once to bf16 with round-to-nearest-even;
  * an activation-like tensor is N(0,1) with round(0.001 * cols) outlier
    columns, chosen without replacement after the values are drawn, x50;
  * the gradient-like tensor is N(0, sigma=1e-3) passed through one seeded
    random-sign 16x16 orthonormal Hadamard rotation per group of 16 along
    dim 1 (the rotation the pages apply before quantizing weight gradients);
  * weights are N(0, 0.02) or 0.02 * Student-t(nu=4).
"""
from dataclasses import dataclass
import math

import numpy as np

GROUP = 16
# Largest decodable magnitude of one IF4 group at exponent 0: 6 * 448.
IF4_TOP = 6.0 * 448.0


def tensor_scale_exp(amax: float) -> int:
    """Per-tensor power-of-two exponent E so that the tensor's largest group
    uses the top of the E4M3 scale range: E = ceil(log2(amax / 2688)), 0 for
    an all-zero tensor, clamped to [-64, 64]."""
    if not (amax > 0.0) or not math.isfinite(amax):
        return 0
    e = math.ceil(math.log2(amax / IF4_TOP))
    return int(max(-64, min(64, e)))


def to_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 (RNE) and return the bf16 values widened to fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) &
         np.uint32(0xFFFF0000))
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, u | np.uint32(0x00400000), r) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def outlier_activations(rows: int, cols: int, seed: int, dtype=np.float32) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    n_out = int(round(0.001 * cols))
    if n_out:
        idx = rng.choice(cols, size=n_out, replace=False)
        x[:, idx] *= np.float32(50.0)
    return x


def hadamard16() -> np.ndarray:
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]], dtype=np.float64)
    h = h2
    for _ in range(3):
        h = np.kron(h, h2)
    return h / 4.0  # orthonormal


def rht16(x: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Per-group random-sign Hadamard rotation along dim 1: y_g = H (d * x_g)
    with H the orthonormal 16x16 Sylvester matrix and d a vector of 16 signs
    shared by all groups (fp32 numpy arithmetic)."""
    rows, cols = x.shape
    h = hadamard16().astype(np.float32)
    g = x.reshape(rows, cols // GROUP, GROUP) * d
    y = np.matmul(g, h.T)
    return np.ascontiguousarray(y.reshape(rows, cols), dtype=np.float32)


def random_signs(rng) -> np.ndarray:
    return rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=GROUP)


def rht_gradient(rows: int, cols: int, seed: int, sigma: float = 1e-3) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(sigma)
    return rht16(x, random_signs(rng))


def normal_weights(rows: int, cols: int, seed: int, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)


def student_t_weights(rows: int, cols: int, seed: int, nu: float = 4.0,
                      scale: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    out = np.empty((rows, cols), np.float32)
    step = max(1, (1 << 24) // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = (rng.standard_t(nu, (r1 - r0, cols)) * scale).astype(np.float32)
    return out


@dataclass
class Tensor:
    name: str
    values: np.ndarray  # fp32 values (bf16-exact when dtype == "bf16")
    dtype: str          # "f32" or "bf16"

    @property
    def scale_exp(self) -> int:
        return tensor_scale_exp(float(np.max(np.abs(self.values))) if self.values.size else 0.0)


def c1_mixed_fp32(seed: int = 0) -> Tensor:
    """fp32 256x256: rows 0-127 N(0,1), rows 128-255 U(-1,1), in that order."""
    rng = np.random.default_rng(seed)
    x = np.empty((256, 256), np.float32)
    x[:128] = rng.standard_normal((128, 256), dtype=np.float32)
    x[128:] = rng.uniform(-1.0, 1.0, (128, 256)).astype(np.float32)
    return Tensor("c1_mixed_fp32_256x256", x, "f32")


def c2_activations(seed: int = 0, rows: int = 8192, cols: int = 4096) -> Tensor:
    return Tensor(f"c2_act_outliers_bf16_{rows}x{cols}",
                  to_bf16_f32(outlier_activations(rows, cols, seed)), "bf16")


def c3_rht_gradient(seed: int = 0, rows: int = 16384, cols: int = 4096) -> Tensor:
    return Tensor(f"c3_rht_grad_bf16_{rows}x{cols}",
                  to_bf16_f32(rht_gradient(rows, cols, seed)), "bf16")


def sign_mask(d: np.ndarray) -> int:
    """16-bit mask of a +-1 vector: bit i set where d_i = -1."""
    return int(sum(1 << i for i in range(GROUP) if d[i] < 0))


def c3_raw_gradient(seed: int = 0, rows: int = 16384, cols: int = 4096):
    """The gradient before its rotation, as a bf16 tensor, and the rotation's
    sign mask: the input of the fused rotate-and-quantize.  Same draws, in the
    same order, as rht_gradient (values first, then the 16 signs)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(1e-3)
    d = random_signs(rng)
    return Tensor(f"c3_raw_grad_bf16_{rows}x{cols}", to_bf16_f32(x), "bf16"), sign_mask(d)


def c4_gemm(seed: int = 0, m: int = 4096, n: int = 4096, k: int = 4096):
    a = Tensor(f"c4_A_bf16_{m}x{k}", to_bf16_f32(outlier_activations(m, k, seed)), "bf16")
    w = Tensor(f"c4_W_bf16_{n}x{k}", to_bf16_f32(normal_weights(n, k, seed + 1)), "bf16")
    return a, w


def c5_ffn(seed: int = 0, m: int = 8192, n: int = 28672, k: int = 8192):
    a = Tensor(f"c5_A_bf16_{m}x{k}", to_bf16_f32(outlier_activations(m, k, seed)), "bf16")
    w = Tensor(f"c5_W_bf16_{n}x{k}", to_bf16_f32(student_t_weights(n, k, seed + 1)), "bf16")
    return a, w
