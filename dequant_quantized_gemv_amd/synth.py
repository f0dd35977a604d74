"""Seeded synthetic inputs for the quantized dequantize / GEMV / GEMM workloads.

This module only draws random numbers and lays bytes out in the ggml block
formats; it holds none of the dequantize or product arithmetic.  Both the GPU
tests and the CPU oracle's tests take their inputs from here.

Generator: SplitMix64 used as a counter-based generator: the i-th draw of a
stream with key ``s`` is ``mix(s + (i + 1) * 0x9E3779B97F4A7C15)``, where
``mix`` is SplitMix64's output function (Steele, Lea, Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014).  Every tensor field (scales
d, offsets m, quant bytes, activations) has its own stream key derived from
(workload seed, tensor id, field id), so a tensor never changes when another
one is resized.

Distributions:
  * fp16 fields: a double uniform in [lo, hi] (53-bit mantissa), then
    round-to-nearest-even to binary16 (numpy's double -> half conversion).
  * Q4 quant bytes: one uniform byte each, so both nibbles are uniform 0..15
    and independent.
  * Q8_0 codes: uniform integers in [-127, 127] as (u64 mod 255) - 127 (the
    modulo bias is below 2^-56).
  * Activations: N(0, 1) by Box-Muller in double from two uniform streams,
    then rounded to fp32 (or binary16 for the fp16-activation GEMM).

Block byte layouts (little-endian binary16 fields, blocks of 32 weights):
  Q4_0: d[2] qs[16]          (18 bytes)
  Q4_1: d[2] m[2] qs[16]     (20 bytes)
  Q8_0: d[2] qs[32] (int8)   (34 bytes)
  Q5_0: d[2] qh[4] qs[16]    (22 bytes; qh little-endian, bit t = bit 4 of code t)
  Q5_1: d[2] m[2] qh[4] qs[16] (24 bytes)
A matrix is ``rows`` rows of k/32 blocks each, rows back to back.
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

BLOCK_BYTES = {"q4_0": 18, "q4_1": 20, "q8_0": 34, "q5_0": 22, "q5_1": 24}
QS_OFFSET = {"q4_0": 2, "q4_1": 4, "q8_0": 2, "q5_0": 6, "q5_1": 8}
QH_OFFSET = {"q5_0": 2, "q5_1": 4}
HAS_M = ("q4_1", "q5_1")

FIELD_D, FIELD_M, FIELD_QS, FIELD_X, FIELD_X2, FIELD_IDS, FIELD_QH = 0, 1, 2, 3, 4, 5, 6


def _mix(z):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed, tensor_id, field_id):
    """Key of the stream for one field of one tensor."""
    v = np.uint64((int(seed) & 0xFFFFFFFF) << 32 | (int(tensor_id) & 0xFFFF) << 8
                  | (int(field_id) & 0xFF))
    return np.uint64(_mix(v))


def splitmix64(key, count, start=0):
    """Draws start .. start+count-1 of the stream with the given key."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + i * GAMMA
    return _mix(z)


def uniform01(key, count):
    """Doubles uniform in [0, 1) with 53 random bits."""
    return (splitmix64(key, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_half_bits(key, count, lo, hi):
    u = uniform01(key, count)
    v = lo + (hi - lo) * u
    return v.astype(np.float16).view(np.uint16)


def normal(key_a, key_b, count):
    u1 = uniform01(key_a, count)
    u2 = uniform01(key_b, count)
    return np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * np.pi * u2)


# ---------------------------------------------------------------------------
# Block packing (byte layout only)
# ---------------------------------------------------------------------------

def pack_blocks(fmt, d_bits, codes, m_bits=None):
    """Lay out blocks from fields.

    d_bits, m_bits: binary16 bit patterns, shape (nblocks,).
    codes: shape (nblocks, 32); 0..15 for Q4_x (element t < 16 goes to the low
    nibble of qs[t], t >= 16 to the high nibble of qs[t-16]); 0..31 for Q5_x
    (the low four bits as Q4_x, bit 4 of element t in bit t of qh);
    -128..127 for Q8_0.
    Returns a flat uint8 array of nblocks * block_bytes.
    """
    d_bits = np.asarray(d_bits, dtype=np.uint16).ravel()
    codes = np.asarray(codes).reshape(-1, 32)
    nb = d_bits.size
    if codes.shape[0] != nb:
        raise ValueError("codes and d disagree on the block count")
    bs = BLOCK_BYTES[fmt]
    out = np.zeros((nb, bs), dtype=np.uint8)
    out[:, 0:2] = d_bits.astype("<u2").view(np.uint8).reshape(nb, 2)
    if fmt in HAS_M:
        if m_bits is None:
            raise ValueError(f"{fmt} needs m")
        m_bits = np.asarray(m_bits, dtype=np.uint16).ravel()
        out[:, 2:4] = m_bits.astype("<u2").view(np.uint8).reshape(nb, 2)
    off = QS_OFFSET[fmt]
    if fmt in ("q4_0", "q4_1"):
        c = codes.astype(np.int64)
        if c.min(initial=0) < 0 or c.max(initial=0) > 15:
            raise ValueError("Q4 codes must be 0..15")
        out[:, off:off + 16] = (c[:, :16] | (c[:, 16:] << 4)).astype(np.uint8)
    elif fmt in ("q5_0", "q5_1"):
        c = codes.astype(np.int64)
        if c.min(initial=0) < 0 or c.max(initial=0) > 31:
            raise ValueError("Q5 codes must be 0..31")
        lo = c & 15
        out[:, off:off + 16] = (lo[:, :16] | (lo[:, 16:] << 4)).astype(np.uint8)
        qh = ((c >> 4) << np.arange(32, dtype=np.int64)).sum(axis=1).astype(np.uint32)
        hoff = QH_OFFSET[fmt]
        out[:, hoff:hoff + 4] = qh.astype("<u4").view(np.uint8).reshape(nb, 4)
    else:
        c = codes.astype(np.int64)
        if c.min(initial=0) < -128 or c.max(initial=0) > 127:
            raise ValueError("Q8 codes must be -128..127")
        out[:, off:off + 32] = c.astype(np.int8).view(np.uint8)
    return out.ravel()


def quant_matrix(fmt, rows, k, seed, tensor_id, d_range, m_range=(-0.1, 0.0)):
    """Random quantized matrix (rows x k) as flat block bytes."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    nb = rows * (k // 32)
    bs = BLOCK_BYTES[fmt]
    out = np.empty((nb, bs), dtype=np.uint8)
    d = uniform_half_bits(stream_key(seed, tensor_id, FIELD_D), nb, *d_range)
    out[:, 0:2] = d.astype("<u2").view(np.uint8).reshape(nb, 2)
    if fmt in HAS_M:
        m = uniform_half_bits(stream_key(seed, tensor_id, FIELD_M), nb, *m_range)
        out[:, 2:4] = m.astype("<u2").view(np.uint8).reshape(nb, 2)
    if fmt in QH_OFFSET:
        # one 32-bit draw (the low half of a 64-bit one) gives a block's qh
        z = splitmix64(stream_key(seed, tensor_id, FIELD_QH), nb) & np.uint64(0xFFFFFFFF)
        hoff = QH_OFFSET[fmt]
        out[:, hoff:hoff + 4] = z.astype("<u4").view(np.uint8).reshape(nb, 4)
    off = QS_OFFSET[fmt]
    key = stream_key(seed, tensor_id, FIELD_QS)
    if fmt in ("q4_0", "q4_1", "q5_0", "q5_1"):
        # two 64-bit draws give the 16 quant bytes of a block
        z = splitmix64(key, 2 * nb)
        out[:, off:off + 16] = z.view(np.uint8).reshape(nb, 16)
    else:
        z = splitmix64(key, 32 * nb)
        c = (z % np.uint64(255)).astype(np.int64) - 127
        out[:, off:off + 32] = c.astype(np.int8).view(np.uint8).reshape(nb, 32)
    return out.ravel()


def activations(k, n, seed, tensor_id, dtype=np.float32):
    """n activation columns of length k, N(0,1); returned as shape (n, k)."""
    a = stream_key(seed, tensor_id, FIELD_X)
    b = stream_key(seed, tensor_id, FIELD_X2)
    v = normal(a, b, n * k).reshape(n, k)
    return v.astype(dtype)


def expert_ids(n_tokens, n_used, n_experts, seed, tensor_id):
    """Expert choices: for each token, n_used distinct ids drawn uniformly from
    0..n_experts-1 (a partial Fisher-Yates shuffle driven by the stream);
    returned as int32 of shape (n_tokens, n_used)."""
    if n_used > n_experts:
        raise ValueError("more slots than experts")
    z = splitmix64(stream_key(seed, tensor_id, FIELD_IDS), n_tokens * n_used)
    out = np.empty((n_tokens, n_used), dtype=np.int32)
    for t in range(n_tokens):
        perm = np.arange(n_experts)
        for s in range(n_used):
            j = s + int(z[t * n_used + s] % np.uint64(n_experts - s))
            perm[s], perm[j] = perm[j], perm[s]
        out[t] = perm[:n_used]
    return out


# ---------------------------------------------------------------------------
# The workloads (shapes and value distributions)
# ---------------------------------------------------------------------------

SEED_BASE = 0x5EED0000
D_Q4 = (1e-3, 2e-2)
D_Q8 = (1e-3, 1e-2)
M_Q4_1 = (-0.1, 0.0)

# decode-layer sweep: a 7B-shaped transformer layer (q, k, v, o, gate, up, down)
LAYER_SHAPES = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
                ("o", 4096, 4096), ("gate", 11008, 4096), ("up", 11008, 4096),
                ("down", 4096, 11008)]

# one GPU's share of that layer under 8-way tensor parallelism: q, k, v, gate
# and up split by output rows, o and down by K (partial sums, to be added
# across the 8 GPUs); every shard boundary falls on a block
TP = 8
LAYER_SHARE_SHAPES = [("q", 512, 4096), ("k", 512, 4096), ("v", 512, 4096),
                      ("o", 4096, 512), ("gate", 1376, 4096), ("up", 1376, 4096),
                      ("down", 4096, 1376)]

# mixture-of-experts decode: expert matrices of intermediate width 768 (the
# Q4_0 expert model the PR's commit list names) over a hidden width of 2048,
# 128 experts, 8 used per token: gate and up 768 x 2048, down 2048 x 768
MOE_SHAPES = [("gate", 768, 2048), ("up", 768, 2048), ("down", 2048, 768)]

WORKLOADS = {
    "dequant_q4_0_4096x4096_f32": dict(id=0, fmt="q4_0", m=4096, k=4096, d=D_Q4),
    "gemv_q8_0_4096x4096_n1": dict(id=1, fmt="q8_0", m=4096, k=4096, n=1, d=D_Q8),
    "gemv_q4_1_11008x4096": dict(id=2, fmt="q4_1", m=11008, k=4096, n=(1, 2, 4, 8),
                                 d=D_Q4, mr=M_Q4_1),
    "gemv_q4_0_decode_layer": dict(id=3, fmt="q4_0", layer=LAYER_SHAPES, n=1, d=D_Q4),
    "gemm_q4_0_14336x4096_n512": dict(id=4, fmt="q4_0", m=14336, k=4096, n=512, d=D_Q4),
    "gemv_q4_0_decode_layer_tp8_share": dict(id=6, fmt="q4_0", layer=LAYER_SHARE_SHAPES, tp=TP, n=1,
                                             d=D_Q4),
    "gemv_q4_0_moe_experts": dict(id=5, fmt="q4_0", layer=MOE_SHAPES, n_experts=128, n_used=8,
                                  n_tokens=1, d=D_Q4),
}


def workload_seed(config_id):
    return SEED_BASE + int(config_id)
