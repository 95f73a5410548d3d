"""Seeded synthetic inputs for the GEMM workloads (shared by the tests, the smoke check and
the benchmark; holds no GEMM arithmetic).

Values are drawn in float64 with numpy's PCG64 and stored in the operand type with torch's
CPU casts. Seeds follow the pages' example harness (page 5, quack/dense_gemm_sm90.py, the
removed 0.1.10 run(): torch.manual_seed(1111)): seed = 1111 + 10 * workload_index + slot,
slot A = 0, B = 1, C = 2, group sizes = 3.

Every generator returns an `Inputs` with CPU tensors:
  store_*   the contiguous storage tensor in the operand type;
  A, B, C   logical views: A (L, M, K), B (L, N, K), C (L, M, N) (varlen-M: A (M, K) or,
            gathered, (rows, K), B (G, N, K), C (M, N); varlen-K: A (M, K), B (N, K),
            C (G, M, N)); an M-major A is a permuted view of a [L][K][M] store.
plus the scalars of the problem (alpha, beta, activation, cu_seqlens_m / cu_seqlens_k,
the gather index a_idx, output types).
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32,
            "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
CODE_DT = {"f16": torch.int16, "bf16": torch.int16, "f32": torch.int32,
           "e4m3": torch.uint8, "e5m2": torch.uint8}
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}
ELEM_BYTES = {"f16": 2, "bf16": 2, "f32": 4, "e4m3": 1, "e5m2": 1}


@dataclass
class Inputs:
    name: str
    M: int
    N: int
    K: int
    L: int
    a_dt: str
    b_dt: str
    A: torch.Tensor
    B: torch.Tensor
    C: Optional[torch.Tensor] = None
    c_dt: str = "none"
    d_dt: str = "none"
    post_dt: str = "none"
    alpha: float = 1.0
    beta: float = 1.0
    act: str = "none"
    cu_seqlens: Optional[np.ndarray] = None
    dact: bool = False  # activation backward: C is the pre-activation, D = (alpha A x B) * act'(C)
    extra: dict = field(default_factory=dict)
    cu_seqlens_k: Optional[np.ndarray] = None  # varlen-K: K ranges of the G groups (K = total extent)
    a_idx: Optional[np.ndarray] = None         # gathered A: the A row of each global output row

    @property
    def varlen(self) -> bool:
        return self.cu_seqlens is not None

    def flops(self) -> float:
        if self.varlen:
            return 2.0 * self.M * self.N * self.K
        if self.cu_seqlens_k is not None:
            return 2.0 * self.M * self.N * float(self.cu_seqlens_k[-1])
        return 2.0 * self.M * self.N * self.K * self.L


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_dtype(x: np.ndarray, dt: str) -> torch.Tensor:
    """Store float64 values in operand type `dt` (torch CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dt in ("e4m3", "e5m2"):
        t = t.clamp(-FP8_MAX[dt], FP8_MAX[dt]).to(torch.float32)
    return t.to(TORCH_DT[dt])


def uniform(seed, shape, dt):
    return to_dtype(rng(seed).uniform(-1.0, 1.0, size=shape), dt)


def normal(seed, shape, dt, std=1.0):
    return to_dtype(rng(seed).standard_normal(size=shape) * std, dt)


def quantize_fp8(seed, shape, dt):
    """Per-tensor scaled fp8: s = amax|X| / fmax, codes = X / s stored in fp8 (saturating).
    Returns (codes tensor, scale s as a Python float)."""
    x = rng(seed).standard_normal(size=shape)
    s = float(np.max(np.abs(x))) / FP8_MAX[dt]
    return to_dtype(x / s, dt), s


def codes_of(t: torch.Tensor) -> np.ndarray:
    """Raw stored codes of a tensor (its whole storage from its storage offset, flat)."""
    base = t
    while base._base is not None:
        base = base._base
    flat = base.reshape(-1)
    return flat.view(CODE_DT[_dt_name(flat.dtype)]).numpy().view(_np_code(flat.dtype))


def _dt_name(tdt):
    for k, v in TORCH_DT.items():
        if v == tdt:
            return k
    raise KeyError(tdt)


def _np_code(tdt):
    return {torch.float16: np.uint16, torch.bfloat16: np.uint16, torch.float32: np.uint32,
            torch.float8_e4m3fn: np.uint8, torch.float8_e5m2: np.uint8}[tdt]


# ---------------------------------------------------------------------------------------
# helpers to build operands in a given major mode
# ---------------------------------------------------------------------------------------

def make_a(gen, L, M, K, m_major, seed, dt, **kw):
    """Logical A (L, M, K); storage [L][M][K] (K-major) or [L][K][M] (M-major)."""
    if m_major:
        store = gen(seed, (L, K, M), dt, **kw)
        return store.permute(0, 2, 1)
    return gen(seed, (L, M, K), dt, **kw)


def make_b(gen, L, N, K, n_major, seed, dt, **kw):
    if n_major:
        store = gen(seed, (L, K, N), dt, **kw)
        return store.permute(0, 2, 1)
    return gen(seed, (L, N, K), dt, **kw)


# ---------------------------------------------------------------------------------------
# the five workloads (sizes as in the project's workload list)
# ---------------------------------------------------------------------------------------

def plain_256():
    """Plain GEMM 256^3, fp16 in, fp16 D, U[-1, 1), alpha = 1, no C, no activation."""
    s = 1111 + 10 * 0
    M = N = K = 256
    A = uniform(s + 0, (1, M, K), "f16")
    B = uniform(s + 1, (1, N, K), "f16")
    return Inputs("plain_256_f16", M, N, K, 1, "f16", "f16", A, B, d_dt="f16")


def act_4096(beta=0.5, act="gelu_tanh", c=True, gemm_scale=None):
    """4096^3 bf16, A/B ~ N(0,1)/sqrt(K), C ~ N(0,1), beta = 0.5, GELU-tanh, D and PostAct."""
    s = 1111 + 10 * 1
    M = N = K = 4096
    std = 1.0 / np.sqrt(K) if gemm_scale is None else gemm_scale
    A = normal(s + 0, (1, M, K), "bf16", std)
    B = normal(s + 1, (1, N, K), "bf16", std)
    C = normal(s + 2, (1, M, N), "bf16") if c else None
    return Inputs("act_4096_bf16_gelu", M, N, K, 1, "bf16", "bf16", A, B, C=C,
                  c_dt="bf16" if c else "none", d_dt="bf16", post_dt="bf16", alpha=1.0,
                  beta=beta, act=act)


def square_8192(dt="f16"):
    """8192^3, U[-1, 1), K-major A and B, D in the input type."""
    s = 1111 + 10 * 2
    M = N = K = 8192
    A = uniform(s + 0, (1, M, K), dt)
    B = uniform(s + 1, (1, N, K), dt)
    return Inputs(f"square_8192_{dt}", M, N, K, 1, dt, dt, A, B, d_dt=dt)


def batched_2048():
    """M = N = 2048, K = 4096, L = 16, fp16 U[-1,1), A M-major, B N-major, fp16 D."""
    s = 1111 + 10 * 2 + 5
    M = N = 2048
    K = 4096
    L = 16
    A = make_a(uniform, L, M, K, True, s + 0, "f16")
    B = make_b(uniform, L, N, K, True, s + 1, "f16")
    return Inputs("batched_2048x2048x4096x16_f16_mn", M, N, K, L, "f16", "f16", A, B, d_dt="f16")


def fp8_8192():
    """8192^3, A e4m3 and B e5m2 (K-major) quantised from N(0,1) with per-tensor scales
    amax/448 and amax/57344; alpha = s_a * s_b; bf16 D."""
    s = 1111 + 10 * 3
    M = N = K = 8192
    A, sa = quantize_fp8(s + 0, (1, M, K), "e4m3")
    B, sb = quantize_fp8(s + 1, (1, N, K), "e5m2")
    alpha = float(np.float32(sa) * np.float32(sb))
    return Inputs("fp8_8192_e4m3xe5m2", M, N, K, 1, "e4m3", "e5m2", A, B, d_dt="bf16",
                  alpha=alpha, extra={"scale_a": sa, "scale_b": sb})


def dact_4096(act="gelu_tanh"):
    """Activation backward at 4096^3 bf16 (page 6, gemm_dact_sm90): A = the incoming gradient
    and B = the weight, both ~ N(0,1)/sqrt(K); C = the saved pre-activation ~ N(0,1) (the
    forward workload's scale); D = dout * act'(C) and PostAct = act(C), bf16."""
    s = 1111 + 10 * 5
    M = N = K = 4096
    std = 1.0 / np.sqrt(K)
    A = normal(s + 0, (1, M, K), "bf16", std)
    B = normal(s + 1, (1, N, K), "bf16", std)
    C = normal(s + 2, (1, M, N), "bf16")
    return Inputs(f"dact_4096_bf16_{act}", M, N, K, 1, "bf16", "bf16", A, B, C=C, c_dt="bf16",
                  d_dt="bf16", post_dt="bf16", act=act, dact=True)


def group_sizes(seed, G, unit=128, max_units=32):
    return rng(seed).integers(1, max_units + 1, size=G) * unit


def varlen_moe(G=8, N=4096, K=4096, sizes=None, std=1.0 / 64.0, act="silu"):
    """Varlen-M: G groups, M_g = 128 * U{1..32}; A (sum M_g, K) bf16 ~ N(0,1)/64; B (G, N, K)
    bf16 ~ N(0,1)/64; SiLU; PostAct only (bf16)."""
    s = 1111 + 10 * 4
    if sizes is None:
        sizes = group_sizes(s + 3, G)
    sizes = np.asarray(sizes, dtype=np.int64)
    cu = np.zeros(G + 1, dtype=np.int32)
    cu[1:] = np.cumsum(sizes)
    M = int(cu[-1])
    A = normal(s + 0, (M, K), "bf16", std)
    B = normal(s + 1, (G, N, K), "bf16", std)
    return Inputs("varlen_m_8x4096x4096_bf16_silu", M, N, K, G, "bf16", "bf16", A, B,
                  post_dt="bf16", act=act, cu_seqlens=cu)


def varlen_k_moe(G=8, M=4096, N=4096, sizes=None, std=1.0, k_unit=128):
    """Varlen-K (grouped K, the weight gradient of a grouped MoE layer): G groups of
    K_g = 128 * U{1..32} tokens (the group-size law of the varlen-M workload), A = X^T with X
    (sum K_g, M) bf16 row-major, i.e. A (M, K) M-major; B = dY^T with dY (sum K_g, N) bf16
    row-major, i.e. B (N, K) N-major; A, B ~ N(0,1) * std; D (G, M, N) bf16."""
    s = 1111 + 10 * 6
    if sizes is None:
        sizes = group_sizes(s + 3, G, unit=k_unit)
    sizes = np.asarray(sizes, dtype=np.int64)
    cu = np.zeros(len(sizes) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(sizes)
    K = int(cu[-1])
    A = normal(s + 0, (K, M), "bf16", std).t()
    B = normal(s + 1, (K, N), "bf16", std).t()
    return Inputs(f"varlen_k_{len(sizes)}x{M}x{N}_bf16", M, N, K, len(sizes), "bf16", "bf16", A, B,
                  d_dt="bf16", cu_seqlens_k=cu)


def varlen_moe_gather(G=8, N=4096, K=4096, sizes=None, std=1.0 / 64.0, act="silu", topk=2):
    """The varlen-M workload with gathered A (MoE tokens read through the routing index):
    X has sum(M_g) / topk token rows ~ N(0,1)/64 and a_idx names, for every row of the
    expert-sorted problem, the token it reads (seeded, uniform over the tokens)."""
    s = 1111 + 10 * 7
    inp = varlen_moe(G, N, K, sizes, std, act)
    rows = max(1, inp.M // topk)
    X = normal(s + 0, (rows, K), "bf16", std)
    a_idx = rng(s + 4).integers(0, rows, size=inp.M).astype(np.int32)
    inp.name = f"varlen_m_gather_{G}x{N}x{K}_bf16_silu"
    inp.A = X
    inp.a_idx = a_idx
    return inp


def varlen_k_moe_gather(G=8, M=4096, N=4096, sizes=None, std=1.0, topk=2):
    """The varlen-K workload with gathered A columns (the weight gradient read straight from
    the unpermuted token matrix): X has sum(K_g) / topk token rows ~ N(0,1), stored
    (tokens, M) row-major, so A = X^T is (M, tokens) M-major; a_idx names, for every routed
    token of the expert-sorted problem, the token row it reads (seeded, uniform)."""
    s = 1111 + 10 * 8
    inp = varlen_k_moe(G, M, N, sizes, std)
    tokens = max(1, inp.K // topk)
    inp.A = normal(s + 0, (tokens, M), "bf16", std).t()
    inp.a_idx = rng(s + 4).integers(0, tokens, size=inp.K).astype(np.int32)
    inp.name = f"varlen_k_gather_{G}x{M}x{N}_bf16"
    return inp


WORKLOADS = {
    "plain_256": plain_256,
    "act_4096": act_4096,
    "square_8192_f16": lambda: square_8192("f16"),
    "square_8192_bf16": lambda: square_8192("bf16"),
    "batched_2048": batched_2048,
    "fp8_8192": fp8_8192,
    "varlen_moe": varlen_moe,
    "dact_4096": dact_4096,
    "varlen_k_moe": varlen_k_moe,
    "varlen_moe_gather": varlen_moe_gather,
    "varlen_k_moe_gather": varlen_k_moe_gather,
}


# ---------------------------------------------------------------------------------------
# device placement (layout-preserving copies and output buffers)
# ---------------------------------------------------------------------------------------

def to_dev(t):
    """Copy a (possibly permuted) CPU view to the GPU with the same strides."""
    if t is None:
        return None
    base = t
    while base._base is not None:
        base = base._base
    dbase = base.to("cuda")
    return torch.as_strided(dbase, t.size(), t.stride(), t.storage_offset())


def out_like(inp, dt, m_major=False, fill=float("nan"), device="cuda"):
    """Output (L, M, N) (varlen: (M, N)) of type dt on the GPU, N- or M-contiguous,
    pre-filled with `fill` so that unwritten elements show."""
    tdt = TORCH_DT[dt]
    if inp.varlen:
        t = torch.empty((inp.N, inp.M), dtype=tdt, device=device).t() if m_major else \
            torch.empty((inp.M, inp.N), dtype=tdt, device=device)
    else:
        t = torch.empty((inp.L, inp.N, inp.M), dtype=tdt, device=device).permute(0, 2, 1) if m_major \
            else torch.empty((inp.L, inp.M, inp.N), dtype=tdt, device=device)
    t.fill_(fill)
    return t
