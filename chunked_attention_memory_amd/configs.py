"""Workload shapes and the algorithmic FLOP count of the forward.

Shapes: the five workloads this library is measured and tested on (tiny fp32,
batched bf16 16K, the 128K-token headline, 1M and 4M tokens). The FLOP count
is what the throughput report divides by; it counts multiply-adds only (2 FLOP
each) and excludes exp, softmax, the affine derivations and masking.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    c: int
    d: int
    dv: int
    dtype: str  # "f32" or "bf16"

    @property
    def nchunks(self) -> int:
        return -(-self.n // self.c)

    @property
    def tokens(self) -> int:
        return self.B * self.n


WORKLOADS = {
    0: Workload("tiny_f32_n256_c64_d32", 1, 1, 256, 64, 32, 32, "f32"),
    1: Workload("bf16_B4_H8_n16k_c2048", 4, 8, 16384, 2048, 128, 256, "bf16"),
    2: Workload("bf16_B1_H8_n128k_c2048", 1, 8, 131072, 2048, 128, 256, "bf16"),
    3: Workload("bf16_B1_H8_n1m_c2048", 1, 8, 1048576, 2048, 128, 256, "bf16"),
    4: Workload("bf16_B1_H4_n4m_c2048", 1, 4, 4194304, 2048, 128, 256, "bf16"),
}


def chunk_sizes(n: int, c: int) -> list[int]:
    return [min(c, n - a) for a in range(0, n, c)]


def flop_count(n: int, c: int, d: int, dv: int) -> dict:
    """Multiply-add FLOPs of one head (one batch row, one head).

    * SCA: 2(d + dv) per unmasked (query, key) pair; chunk s has
      c_{s-1} c_s pairs with the previous chunk and c_s (c_s + 1)/2 causal
      pairs inside itself.
    * memory write E^T V for chunks 1..N-2 (2 c_t d dv each);
    * correction factor E^T psi(K) for chunks 2..N-2 (2 c_t d^2; chunk 1
      multiplies the zero state);
    * the state product (E^T psi(K)) M' for N-3 steps (2 d^2 dv each);
    * readout psi(Q_m) M' for chunks 3..N (2 c_s d dv each).
    """
    sizes = chunk_sizes(n, c)
    N = len(sizes)
    pairs = 0
    for s, cs in enumerate(sizes):
        prev = sizes[s - 1] if s else 0
        pairs += prev * cs + cs * (cs + 1) // 2
    sca = 2 * (d + dv) * pairs
    write = sum(2 * sizes[t] * d * dv for t in range(0, max(N - 2, 0)))
    corr = sum(2 * sizes[t] * d * d for t in range(1, max(N - 2, 0)))
    scan = max(N - 3, 0) * 2 * d * d * dv
    read = sum(2 * sizes[s] * d * dv for s in range(2, N))
    return {"pairs": pairs, "sca": sca, "awm_write": write, "awm_corr": corr,
            "awm_scan": scan, "awm_read": read,
            "total": sca + write + corr + scan + read}


def backward_flop_count(n: int, c: int, d: int, dv: int) -> dict:
    """Multiply-add FLOPs of the backward of one head, each product counted
    once (recomputation that an implementation chooses is not counted).

    * SCA: per unmasked pair the logits q.k (2d), dP = dO.v (2dv), the dV
      (2dv), dQ (2d) and dK (2d) contributions;
    * memory, chunks 3..N that read the state: psi(Q)^T dO into the state
      gradient and dO S^T into dpsi(Q) (2 c_s d dv each);
    * the reverse scan's transposed correction product, N-3 steps of 2 d^2 dv;
    * per chunk t entering the memory (1..N-2): Phi dS_t into dV and
      V dS_t^T into dPhi (2 c_t d dv each); for t >= 2, X_t = dS_t S_{t-1}^T
      (2 d^2 dv) and psi X^T, Phi X (2 c_t d^2 each).
    """
    sizes = chunk_sizes(n, c)
    N = len(sizes)
    pairs = flop_count(n, c, d, dv)["pairs"]
    sca = 2 * (3 * d + 2 * dv) * pairs
    read = sum(2 * 2 * sizes[s] * d * dv for s in range(2, N))
    scan = max(N - 3, 0) * 2 * d * d * dv
    keys = sum(2 * 2 * sizes[t] * d * dv for t in range(0, max(N - 2, 0)))
    corr = sum(2 * d * d * dv + 2 * 2 * sizes[t] * d * d for t in range(1, max(N - 2, 0)))
    return {"pairs": pairs, "sca": sca, "awm_read": read, "awm_scan": scan, "awm_keys": keys, "awm_corr": corr,
            "total": sca + read + scan + keys + corr}


def workload_flops(w: Workload) -> dict:
    per = flop_count(w.n, w.c, w.d, w.dv)
    return {k: v * w.B * w.H for k, v in per.items()}
