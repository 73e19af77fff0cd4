"""Seeded synthetic inputs standing in for the pages' calibration corpus and weights.

This module only draws random numbers in the shapes and distributions of the
workloads; it contains no step of the quantization method.  Both the HIP path
and the CPU oracle consume the exact tensors produced here (large inputs are
drawn on the GPU and copied to the host for the oracle).

Recipes:
* calibration inputs, "spectral" model: X = (Z diag(sigma)) Q^T with
  Z ~ N(0, 1), sigma_i^2 = 10^(-3 i / (n - 1)) (three decades) and Q a Haar
  orthogonal matrix (QR of a Gaussian with the sign of diag(R) fixed); then
  round(frac * n) channels chosen by the seed are multiplied by 20;
* "product" model (post-SwiGLU-like): a * b elementwise with a, b from the
  spectral model and b = rho a + sqrt(1 - rho^2) a', rho = 0.5;
* weights: Gaussian N(0, std^2) or Student-t with 5 degrees of freedom scaled
  to std 0.02 (0.015492 t_5), built as Z / sqrt(chi2_5 / 5);
* adapters: B (rows x r), A (r x n) ~ N(0, 0.01^2);
* rotation signs: +-1 with equal probability.
"""

import math

import torch


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def haar_orthogonal(n, seed, device="cpu"):
    g = _gen(seed, device)
    A = torch.randn(n, n, generator=g, device=device, dtype=torch.float64 if device == "cpu" else torch.float32)
    Q, R = torch.linalg.qr(A)
    Q = Q * torch.sign(torch.diagonal(R))[None, :]
    return Q.to(torch.float32)


def spectrum(n, device="cpu"):
    i = torch.arange(n, device=device, dtype=torch.float64)
    return torch.sqrt(10.0 ** (-3.0 * i / max(n - 1, 1))).to(torch.float32)


def outlier_channels(n, count, seed, device="cpu"):
    g = _gen(seed, "cpu")
    return torch.randperm(n, generator=g)[:count].to(device)


class SpectralSource:
    """Draws calibration rows chunk by chunk; chunk k is reproducible from (seed, k)."""

    def __init__(self, n, seed, device="cpu", outlier_frac=0.01, n_outliers=None, product=False, rho=0.5):
        self.n = n
        self.seed = int(seed)
        self.device = device
        self.Q = haar_orthogonal(n, self.seed * 7919 + 1, device)
        self.sigma = spectrum(n, device)
        count = n_outliers if n_outliers is not None else int(round(outlier_frac * n))
        self.outliers = outlier_channels(n, count, self.seed * 7919 + 2, device)
        self.product = product
        self.rho = rho

    def _spectral(self, rows, g):
        Z = torch.randn(rows, self.n, generator=g, device=self.device, dtype=torch.float32)
        X = (Z * self.sigma[None, :]) @ self.Q.T
        X[:, self.outliers] *= 20.0
        return X

    def chunk(self, k, rows, dtype=torch.bfloat16):
        g = _gen(self.seed * 1000003 + 17 * k + 3, self.device)
        if not self.product:
            return self._spectral(rows, g).to(dtype)
        a = self._spectral(rows, g)
        a2 = self._spectral(rows, g)
        b = self.rho * a + math.sqrt(1.0 - self.rho ** 2) * a2
        return (a * b).to(dtype)


def gaussian(shape, std, seed, device="cpu", dtype=torch.float32):
    g = _gen(seed, device)
    return (std * torch.randn(*shape, generator=g, device=device, dtype=torch.float32)).to(dtype)


def student_t(shape, seed, df=5, std=0.02, device="cpu", dtype=torch.float32):
    g = _gen(seed, device)
    z = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    chi2 = torch.zeros(*shape, device=device, dtype=torch.float32)
    for _ in range(df):
        chi2 += torch.randn(*shape, generator=g, device=device, dtype=torch.float32) ** 2
    t = z / torch.sqrt(chi2 / df)
    scale = std / math.sqrt(df / (df - 2))
    return (scale * t).to(dtype)


def signs(n, seed, device="cpu"):
    g = _gen(seed, "cpu")
    s = torch.randint(0, 2, (n,), generator=g, dtype=torch.int8) * 2 - 1
    return s.to(device)


def trellis8_values(device="cpu"):
    """The 8-state trellis of the trellis workload, 2 bits per weight (the Pingala-8 post names
    an 8-state set-partitioned trellis without giving it): eight levels -3.5 .. 3.5 in steps of
    1, split into four cosets D_j = {level j, level j + 4}; branch u of state s carries
    D_{(s & 1) + 2u}, so the two branches of a state use the cosets of one parent subset (even
    states the even levels, odd states the odd ones), as in the post's 2-state toy.
    Returns an 8 x 2 x 2 fp32 tensor."""
    levels = [-3.5 + i for i in range(8)]
    vals = [[[levels[(s & 1) + 2 * u], levels[(s & 1) + 2 * u + 4]] for u in range(2)] for s in range(8)]
    return torch.tensor(vals, dtype=torch.float32, device=device)
