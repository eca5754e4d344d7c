"""The synthetic workloads the library is tested and measured on.

Each workload is named by what it is and its sizes.  Inputs come from
``inputs.make_inputs`` with the listed seed (i.i.d. N(0, 1), rounded to the
storage type).  The shapes follow the pages' own measurements: causal fp16
B=1 H=32 D=128 with N from 512 to 8192 is the benchmark of "CUDA
FlashAttention: from online softmax to the long-sequence IO limit" (§8); the
B=1 H=32 N=4096 D=64 shape is the validation workload of "FlashAttention
dataflow and engineering validation on MI50" (§5.2).  One head of N=16384
is the shape the first page's split along K is for (§7: long N, small B*H).
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    causal: bool
    dtype: str
    seed: int
    spiky_keys: bool = False
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)

    def fwd_flops(self) -> float:
        """Algorithmic forward FLOPs: 4BHN^2D non-causal, 2BHN^2D causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.D
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """Algorithmic backward FLOPs: five N x N x D products (S recompute,
        dP, dV, dQ, dK) at 2 FLOP per multiply-add, halved when causal."""
        f = 10.0 * self.B * self.H * self.N * self.N * self.D
        return f / 2 if self.causal else f

    def io_bytes_fwd(self) -> float:
        """Compulsory forward HBM bytes: read Q, K, V, write O (2 B each
        element) and the FP32 LSE."""
        e = self.B * self.H * self.N * self.D
        return 4 * e * 2 + self.B * self.H * self.N * 4

    def io_bytes_bwd(self) -> float:
        """Compulsory backward bytes: read Q, K, V, O, dO; write dQ, dK, dV;
        read LSE; write and read the FP32 row term Delta."""
        e = self.B * self.H * self.N * self.D
        r = self.B * self.H * self.N
        return 8 * e * 2 + 3 * r * 4


SMALL = Workload("fwd_b1h1n256d64_fp16", 1, 1, 256, 64, False, "fp16", seed=1)
NONCAUSAL_D64 = Workload("fwd_b1h32n4096d64_fp16", 1, 32, 4096, 64, False, "fp16", seed=2)
CAUSAL_D128 = {n: Workload("fwd_causal_b1h32n%dd128_fp16" % n, 1, 32, n, 128, True, "fp16", seed=3)
               for n in (512, 1024, 2048, 4096, 8192)}
LONG_BF16 = Workload("fwd_causal_b1h16n32768d128_bf16_spikyk", 1, 16, 32768, 128, True, "bf16",
                     seed=4, spiky_keys=True)
FWDBWD_D64 = Workload("fwdbwd_causal_b1h32n4096d64_fp16", 1, 32, 4096, 64, True, "fp16", seed=5,
                      backward=True)
FEW_HEADS_LONG = Workload("fwd_b1h1n16384d128_fp16", 1, 1, 16384, 128, False, "fp16", seed=6)
# the workload the headline metric is quoted on
HEADLINE = CAUSAL_D128[8192]

ALL = [SMALL, NONCAUSAL_D64, *CAUSAL_D128.values(), LONG_BF16, FWDBWD_D64, FEW_HEADS_LONG]
