"""Seeded synthetic inputs for block-scaled quantization.

This module only builds inputs: BF16 bit patterns, routing metadata and
tensor scales.  It holds none of the quantization arithmetic and serves both
the GPU library's tests/benchmark and the CPU oracle, which otherwise share
nothing.

The five workloads stand in for the MoE activations named on the Modular
grouped block-scaled matmul dispatch page ("NVFP4 routing": the Kimi K2.5
up-projection with K = 7168; the tuned-stages table also lists K = 2048) and
follow the pages' argument types (uint32 row_offsets / scales_offsets, int32
expert_ids and row_indices, fp32 per-expert tensor scale).  Every array comes
from numpy's PCG64 ``default_rng(seed)``: values are drawn in float32 and
rounded to nearest even into BF16.
"""
from dataclasses import dataclass, field

import numpy as np

MXFP4, MXFP8, NVFP4 = 0, 1, 2
FP8_E4M3_MAX_TIMES_FP4_MAX = np.float32(6.0 * 448.0)  # 2688: the tensor scale that maps
# a tensor's amax onto the largest NVFP4 code under the largest E4M3 block scale


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest even BF16; return the uint16 patterns.
    Inputs must be finite and below the BF16 overflow threshold."""
    f = np.ascontiguousarray(f32, dtype=np.float32)
    b = f.view(np.uint32)
    r = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact float32 value of BF16 patterns."""
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def amax_of(h: np.ndarray) -> np.float32:
    """Largest |value| over the finite BF16 patterns (NaN/Inf skipped), as
    float32 (exact)."""
    mag = np.asarray(h) & np.uint16(0x7FFF)
    mag = mag[mag < np.uint16(0x7F80)]
    if mag.size == 0:
        return np.float32(0.0)
    return np.float32(bf16_to_f32(mag).max())


def tensor_scale(h: np.ndarray) -> np.float32:
    """fl32(amax / 2688); 1.0 for an empty or all-zero tensor.  The NVFP4
    workloads' recipe for their input tensor scales: it sets an input and is
    never an expected value (the device tensor-scale producer is checked
    against the oracle's own definition, clamps included)."""
    a = amax_of(h)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / FP8_E4M3_MAX_TIMES_FP4_MAX)


@dataclass
class DenseCase:
    name: str
    fmt: int
    x: np.ndarray                      # uint16 [M, K] BF16 patterns
    tensor_sf: float = 1.0             # NVFP4 only

    @property
    def shape(self):
        return self.x.shape


@dataclass
class GroupedCase:
    name: str
    fmt: int
    x: np.ndarray                      # uint16 [num_src_rows, K]
    row_offsets: np.ndarray            # uint32 [G + 1]
    scales_offsets: np.ndarray         # uint32 [G + 1]
    expert_ids: np.ndarray             # int32 [G]
    tensor_sf: np.ndarray | None       # float32 [E] (NVFP4) or None
    row_indices: np.ndarray | None     # int32 [max_rows] or None
    max_rows: int = 0
    num_scale_rows: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def G(self):
        return int(self.expert_ids.shape[0])


def _roundup(a, m):
    return (a + m - 1) // m * m


def offsets_from_counts(counts, pad: int = 128):
    """row_offsets = [0, cumsum(counts)]; scales_offsets = [0,
    cumsum(roundup(counts, pad))], both uint32."""
    counts = np.asarray(counts, np.int64)
    ro = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    so = np.concatenate([[0], np.cumsum(_roundup(counts, pad))]).astype(np.uint32)
    return ro, so


# ------------------------------------------------------------------ workloads

def dense_mxfp4_small(seed: int = 1001, M: int = 128, K: int = 4096) -> DenseCase:
    """Dense MXFP4, [128, 4096], N(0, 1)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M, K), dtype=np.float32)
    return DenseCase("dense_mxfp4_128x4096", MXFP4, bf16_bits(z))


def dense_mxfp8_scaled_rows(seed: int = 1002, M: int = 8192, K: int = 7168) -> DenseCase:
    """Dense MXFP8, [8192, 7168]: N(0, 1) times a per-row 2^u, u ~ U(-8, 8),
    and 0.1% of elements (Bernoulli) multiplied by 100 as outliers."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M, K), dtype=np.float32)
    u = rng.uniform(-8.0, 8.0, (M, 1))
    z *= np.exp2(u).astype(np.float32)
    mask = rng.random((M, K), dtype=np.float32) < np.float32(0.001)
    z[mask] *= np.float32(100.0)
    return DenseCase("dense_mxfp8_8192x7168", MXFP8, bf16_bits(z))


def dense_nvfp4_scaled_rows(seed: int = 1003, M: int = 16384, K: int = 7168) -> DenseCase:
    """Dense NVFP4, [16384, 7168]: N(0, 1) times a per-row 2^u, u ~ U(-4, 4);
    tensor scale fl32(global amax / 2688)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M, K), dtype=np.float32)
    u = rng.uniform(-4.0, 4.0, (M, 1))
    z *= np.exp2(u).astype(np.float32)
    x = bf16_bits(z)
    return DenseCase("dense_nvfp4_16384x7168", NVFP4, x, float(tensor_scale(x)))


def grouped_nvfp4_prefill(seed: int = 1004, rows: int = 16384, K: int = 7168,
                          experts: int = 128, alpha: float = 0.3) -> GroupedCase:
    """Grouped NVFP4 prefill: 128 experts, 16384 routed rows x 7168, N(0, 1);
    per-expert counts multinomial over Dirichlet(0.3) (empty experts allowed);
    scale rows padded to multiples of 128 per expert; expert_ids = arange;
    per-expert tensor scale fl32(amax of its rows / 2688), 1.0 if empty; no
    gather (routed row r reads source row r)."""
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((rows, K), dtype=np.float32))
    p = rng.dirichlet([alpha] * experts)
    counts = rng.multinomial(rows, p)
    ro, so = offsets_from_counts(counts, 128)
    sf = np.ones(experts, np.float32)
    for e in range(experts):
        if counts[e] > 0:
            sf[e] = tensor_scale(x[ro[e]:ro[e + 1]])
    return GroupedCase("grouped_nvfp4_prefill_16384x7168_e128", NVFP4, x, ro, so,
                       np.arange(experts, dtype=np.int32), sf, None, max_rows=rows,
                       num_scale_rows=int(so[-1]), extra={"counts": counts})


def grouped_mx_prefill(fmt: int) -> GroupedCase:
    """The grouped NVFP4 prefill routing and activations, quantized to an MX
    format instead (no tensor scales)."""
    c = grouped_nvfp4_prefill()
    name = {MXFP4: "mxfp4", MXFP8: "mxfp8"}[fmt]
    return GroupedCase(f"grouped_{name}_prefill_16384x7168_e128", fmt, c.x, c.row_offsets,
                       c.scales_offsets, c.expert_ids, None, None, max_rows=c.max_rows,
                       num_scale_rows=c.num_scale_rows, extra=c.extra)


def grouped_mx_decode(fmt: int = MXFP4, seed: int = 1005, tokens: int = 64, K: int = 2048,
                      experts: int = 256, topk: int = 8) -> GroupedCase:
    """Grouped decode with gather: [64, 2048] N(0, 1) activations, top-8 of 256
    experts per token (uniform, no repeats), 512 routed rows ordered stably by
    expert; row_indices maps each routed row to its token; scale rows padded
    to 128 per expert."""
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((tokens, K), dtype=np.float32))
    choice = np.stack([rng.choice(experts, topk, replace=False) for _ in range(tokens)])
    pair_expert = choice.reshape(-1)
    pair_token = np.repeat(np.arange(tokens), topk)
    order = np.argsort(pair_expert, kind="stable")
    row_indices = pair_token[order].astype(np.int32)
    counts = np.bincount(pair_expert, minlength=experts)
    ro, so = offsets_from_counts(counts, 128)
    name = "grouped_%s_decode_gather_512x2048_e256" % ("mxfp4" if fmt == MXFP4 else "mxfp8")
    return GroupedCase(name, fmt, x, ro, so, np.arange(experts, dtype=np.int32), None,
                       row_indices, max_rows=tokens * topk, num_scale_rows=int(so[-1]),
                       extra={"counts": counts})


# ------------------------------------------------------------ sweep inputs

@dataclass
class DequantCase:
    """Block-scaled codes and scales to decode (random bytes: every code and
    scale pattern, NaN and overflow ones included, appears)."""
    name: str
    fmt: int
    codes: np.ndarray                  # uint8 [M, K/2] (FP4) or [M, K] (FP8)
    scales: np.ndarray                 # uint8 [M, K/block]
    K: int
    tensor_sf: float = 1.0


def dequant_random_bytes(fmt: int, M: int, K: int, seed: int,
                         tensor_sf: float = 1.0) -> DequantCase:
    rng = np.random.default_rng(seed)
    bs = 16 if fmt == NVFP4 else 32
    width = K if fmt == MXFP8 else K // 2
    codes = rng.integers(0, 256, (M, width), dtype=np.uint8)
    scales = rng.integers(0, 256, (M, K // bs), dtype=np.uint8)
    name = {MXFP4: "mxfp4", MXFP8: "mxfp8", NVFP4: "nvfp4"}[fmt]
    return DequantCase(f"dequant_{name}_{M}x{K}", fmt, codes, scales, K, tensor_sf)


@dataclass
class GemmCase:
    """Two MX operands for c = A B^T: codes row-major, scales already in the
    MFMA 16x16x128 layout (random bytes)."""
    name: str
    fmt: int
    a_codes: np.ndarray
    a_scales: np.ndarray               # uint8 [ceil(M/16), 256 * ceil(K/512)]
    b_codes: np.ndarray
    b_scales: np.ndarray
    K: int


def gemm_random_operands(fmt: int, M: int, N: int, K: int, seed: int) -> GemmCase:
    """Random codes (E4M3 NaN codes replaced by 1.0) and scale bytes in
    [120, 134] (2^-7 .. 2^7) for both operands."""
    rng = np.random.default_rng(seed)
    width = K if fmt == MXFP8 else K // 2

    def codes(rows):
        c = rng.integers(0, 256, (rows, width), dtype=np.uint8)
        if fmt == MXFP8:
            c[(c & 0x7F) == 0x7F] = 0x38
        return c

    def scales(rows):
        return rng.integers(120, 135, ((rows + 15) // 16, ((K // 32 + 15) // 16) * 256),
                            dtype=np.uint8)

    name = {MXFP4: "mxfp4", MXFP8: "mxfp8"}[fmt]
    return GemmCase(f"mfma_gemm_{name}_{M}x{N}x{K}", fmt, codes(M), scales(M), codes(N),
                    scales(N), K)


@dataclass
class GroupedGemmCase:
    """Routed MX activations (codes in routed order, MFMA-layout scales at
    padded scale rows) and per-expert MX weights [num_experts * N, K]."""
    name: str
    fmt: int
    a_codes: np.ndarray
    a_scales: np.ndarray
    row_offsets: np.ndarray
    scales_offsets: np.ndarray
    expert_ids: np.ndarray
    max_rows: int
    num_scale_rows: int
    b_codes: np.ndarray
    b_scales: np.ndarray
    num_experts: int
    K: int


def grouped_gemm_prefill(fmt: int = MXFP4, seed: int = 1203, rows: int = 16384, K: int = 7168,
                         N: int = 512, experts: int = 128, alpha: float = 0.3) -> GroupedGemmCase:
    """The prefill routing (multinomial over Dirichlet(alpha) per-expert
    counts, scale rows padded to 128 per expert) with random codes and scale
    bytes in [120, 134] for the activations and for E experts' [N, K] weights."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(rows, rng.dirichlet([alpha] * experts))
    ro, so = offsets_from_counts(counts, 128)
    width = K if fmt == MXFP8 else K // 2
    rec = ((K // 32 + 15) // 16) * 256

    def codes(n):
        c = rng.integers(0, 256, (n, width), dtype=np.uint8)
        if fmt == MXFP8:
            c[(c & 0x7F) == 0x7F] = 0x38
        return c

    nsr = int(so[-1])
    a_scales = rng.integers(120, 135, ((nsr + 15) // 16, rec), dtype=np.uint8)
    b_scales = rng.integers(120, 135, (experts * ((N + 15) // 16), rec), dtype=np.uint8)
    name = {MXFP4: "mxfp4", MXFP8: "mxfp8"}[fmt]
    return GroupedGemmCase(f"mfma_grouped_gemm_{name}_{rows}x{N}x{K}_e{experts}", fmt,
                           codes(rows), a_scales, ro, so, np.arange(experts, dtype=np.int32),
                           rows, nsr, codes(experts * N), b_scales, experts, K)


def grouped_gemm_decode(fmt: int = MXFP4, seed: int = 1204, tokens: int = 64, K: int = 2048,
                        N: int = 7168, experts: int = 256, topk: int = 8) -> GroupedGemmCase:
    """The decode routing of grouped_mx_decode (each of 64 tokens picks 8 of
    256 experts uniformly without repeats; 512 routed rows ordered stably by
    expert; scale rows padded to 128 per expert) with random codes and scale
    bytes in [120, 134] for the routed activations [512, K] and for the
    experts' [N, K] weights."""
    rng = np.random.default_rng(seed)
    choice = np.stack([rng.choice(experts, topk, replace=False) for _ in range(tokens)])
    counts = np.bincount(choice.reshape(-1), minlength=experts)
    ro, so = offsets_from_counts(counts, 128)
    width = K if fmt == MXFP8 else K // 2
    rec = ((K // 32 + 15) // 16) * 256
    rows = tokens * topk

    def codes(n):
        c = rng.integers(0, 256, (n, width), dtype=np.uint8)
        if fmt == MXFP8:
            c[(c & 0x7F) == 0x7F] = 0x38
        return c

    nsr = int(so[-1])
    a_scales = rng.integers(120, 135, ((nsr + 15) // 16, rec), dtype=np.uint8)
    b_scales = rng.integers(120, 135, (experts * ((N + 15) // 16), rec), dtype=np.uint8)
    name = {MXFP4: "mxfp4", MXFP8: "mxfp8"}[fmt]
    return GroupedGemmCase(f"mfma_grouped_gemm_{name}_decode_{rows}x{N}x{K}_e{experts}", fmt,
                           codes(rows), a_scales, ro, so, np.arange(experts, dtype=np.int32),
                           rows, nsr, codes(experts * N), b_scales, experts, K)


def sweep_matrix(bs: int, background: str = "zeros", anchor_bits: int = 0,
                 seed: int = 0) -> np.ndarray:
    """[bs * 65536, bs] BF16 patterns.  Row p * 65536 + h holds pattern h at
    position p (every BF16 bit pattern at every position).  The other
    positions hold the background: "zeros"; "anchor" (the pattern
    ``anchor_bits`` at position (p + 1) % bs, zeros elsewhere); or "normal"
    (seeded N(0, 1) values drawn per row)."""
    n = 65536
    out = np.zeros((bs * n, bs), np.uint16)
    if background == "normal":
        rng = np.random.default_rng(seed)
        out[:] = bf16_bits(rng.standard_normal((bs * n, bs), dtype=np.float32))
    pat = np.arange(n, dtype=np.uint32).astype(np.uint16)
    for p in range(bs):
        blk = out[p * n:(p + 1) * n]
        if background == "anchor" and bs > 1:
            blk[:, (p + 1) % bs] = np.uint16(anchor_bits)
        blk[:, p] = pat
    return out


def random_bf16(shape, seed: int, scale_log2_range=(-8, 8), special_frac: float = 0.0):
    """N(0, 1) times per-row 2^u plus, optionally, a fraction of NaN/Inf/zero/
    subnormal patterns sprinkled in (edge-case inputs)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(shape, dtype=np.float32)
    if len(shape) == 2 and shape[0] > 0:
        u = rng.uniform(scale_log2_range[0], scale_log2_range[1], (shape[0], 1))
        z *= np.exp2(u).astype(np.float32)
    x = bf16_bits(z)
    if special_frac > 0 and x.size:
        m = rng.random(shape) < special_frac
        specials = np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F,
                             0x7F7F, 0xFF7F, 0x0080], np.uint16)
        x[m] = specials[rng.integers(0, len(specials), int(m.sum()))]
    return x
