"""CPU oracle for the fused mixed-precision MoE expert layer (test infrastructure).

This is a plain, slow, fp64 statement of what the layer computes.  It is test
infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline
leg may use it.  It shares no code with the HIP library and imports nothing
from it.

Sources (the pages are machine-written summaries of one paper, PagedWeight):

* [PW] "Technical summary: PagedWeight", gist.science (ja) and its Hindi twin.
  - Core components 1 ("Paged Weight representation"): the unit of precision
    is an expert linear block named by (layer, expert, gate_up | down); the
    weights are Any-Precision LLM overlaid bit planes with associated lookup
    tables; a Weight Page Table holds per block a desired bitwidth d_i and a
    committed bitwidth q_i.
  - Core components 3 ("Asynchronous execution and kernel optimization",
    second bullet): one fused kernel reads the bit planes and the tables
    directly and runs every linear block at its own bitwidth.
  - Core components 2 ("Online routing statistics"): routing mass is the
    selection frequency and weight of each expert, i.e. the router hands each
    token a set of experts with weights.

The pages print no formula, so the definitions below are the plainest reading:

* overlaid bit planes: the b-bit code of a weight is formed from the first b
  planes, plane 0 being the most significant bit; so a b-bit code is the top-b
  prefix of the 8-bit code.
* the table of bitwidth b for row n maps a b-bit code to the row's fp16 value.
* the layer is a routed SwiGLU FFN: h = SiLU(gate) * up, o = W_down h,
  y[t] = sum_j w[t, j] o_{ids[t, j]}(x[t]).

Edge readings (also listed in the design notes): a slot whose expert id is
outside [0, E) contributes nothing; a block whose committed bitwidth is outside
3..8 contributes nothing (its rows read as zero); duplicate ids within a token
are summed; experts nobody routes to are never read.

Parity pins: see tests/test_oracle_pins.py.  Every function here has at least
one pin that does not reuse its own code.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

MIN_BITS = 3
MAX_BITS = 8
LUT_ROW_ENTRIES_ALL = sum(2 ** b for b in range(MIN_BITS, MAX_BITS + 1))  # 504


def lut_offset(N: int, b: int) -> int:
    """Element offset of the bitwidth-b table inside the b-major concatenation
    (tables for b = 3, 4, ... laid one after another, each [N][2**b])."""
    return sum(N * 2 ** c for c in range(MIN_BITS, b))


def plane_bits(planes: np.ndarray, p: int) -> np.ndarray:
    """Bit of plane p for every weight: uint8 [N][K] in {0, 1}.

    Word c of a row holds weights 32c .. 32c+31, weight 32c+j in bit j (LSB
    first).  On a little-endian host the bytes of word c are, in memory order,
    bits 0-7, 8-15, 16-23, 24-31, so unpacking every byte LSB first lists the
    bits in weight order."""
    assert np.little_endian
    words = np.ascontiguousarray(planes[p], dtype=np.uint32)   # [N][K/32]
    N, W = words.shape
    return np.unpackbits(words.view(np.uint8).reshape(N, 4 * W), axis=1, bitorder="little")


def unpack_codes(planes: np.ndarray, b: int) -> np.ndarray:
    """b-bit codes int32 [N][K] from the first b planes ([PW] Core components 1):
    code = sum over p < b of bit_p * 2**(b - 1 - p)."""
    assert MIN_BITS <= b <= MAX_BITS and planes.shape[0] >= b
    N, W = planes.shape[1], planes.shape[2]
    code = np.zeros((N, 32 * W), dtype=np.int32)
    for p in range(b):
        code += plane_bits(planes, p).astype(np.int32) * (2 ** (b - 1 - p))
    return code


def lut_table(lut_all: np.ndarray, N: int, b: int) -> np.ndarray:
    """Per-row table of bitwidth b as fp16 bits: [N][2**b]."""
    off = lut_offset(N, b)
    return np.asarray(lut_all[off: off + N * 2 ** b]).reshape(N, 2 ** b)


def dequant_block(planes: np.ndarray, lut_all: np.ndarray, b: int) -> np.ndarray:
    """Weights of one linear block at bitwidth b as fp16 bit patterns [N][K]:
    W[n, kk] = table_b[n][code_b(n, kk)] (a table copy, no arithmetic)."""
    N = planes.shape[1]
    code = unpack_codes(planes, b)
    tab = lut_table(lut_all, N, b)
    out = np.empty(code.shape, dtype=np.uint16)
    for n in range(N):
        out[n] = tab[n][code[n]]
    return out


def fp16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) in fp64."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(xe: np.ndarray, Wgu: np.ndarray, Wd: np.ndarray, I: int) -> np.ndarray:
    """One expert on a batch of its tokens (fp64): rows [0, I) of gate_up are
    the gate, rows [I, 2I) the up projection; h = SiLU(gate) * up; o = W_down h."""
    gu = xe @ Wgu.T
    g, u = gu[:, :I], gu[:, I:]
    h = silu(g) * u
    return h @ Wd.T


def block_valid(b: int) -> bool:
    return MIN_BITS <= int(b) <= MAX_BITS


def _dequant_cached(planes, lut_all, b, cache):
    if cache is None:
        return dequant_block(planes, lut_all, b)
    key = (id(planes), id(lut_all), b)
    if key not in cache:
        cache[key] = (planes, lut_all, dequant_block(planes, lut_all, b))
    return cache[key][2]


def moe_forward(x: np.ndarray, ids: np.ndarray, w: np.ndarray,
                planes: Sequence[Sequence[np.ndarray]], luts: Sequence[Sequence[np.ndarray]],
                q: np.ndarray, H: int, I: int, E: int,
                tokens: Sequence[int] | None = None, cache: dict | None = None) -> np.ndarray:
    """Routed top-k SwiGLU MoE layer with every block at its committed bitwidth.

    x fp16 [T][H]; ids int [T][k]; w fp32 [T][k]; planes[e][m], luts[e][m] in
    the input format; q uint8 [E][2].  Returns y fp64 [len(tokens)][H] for the
    requested tokens (all tokens by default).  Experts are visited in ascending
    id; each expert's blocks are dequantized once ([PW] Core components 3: each
    block at its own bitwidth).  ``cache`` (optional dict) keeps dequantized
    blocks between calls, keyed by the storage arrays' identity and bitwidth."""
    T, k = ids.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = np.zeros((len(tok), H), dtype=np.float64)
    sel_ids = ids[tok]
    for e in sorted(set(int(v) for v in sel_ids.reshape(-1) if 0 <= int(v) < E)):
        rows, cols = np.nonzero(sel_ids == e)
        if not (block_valid(q[e][0]) and block_valid(q[e][1])):
            continue
        Wgu = fp16_bits_to_f64(_dequant_cached(planes[e][0], luts[e][0], int(q[e][0]), cache))
        Wd = fp16_bits_to_f64(_dequant_cached(planes[e][1], luts[e][1], int(q[e][1]), cache))
        xe = x[tok[rows]].astype(np.float64)
        o = expert_ffn(xe, Wgu, Wd, I)
        for r, (ti, j) in enumerate(zip(rows, cols)):
            y[ti] += float(w[tok[ti], j]) * o[r]
    return y


def moe_forward_layer(layer, tokens=None, cache=None, q=None, ids=None, w=None) -> np.ndarray:
    wl = layer.wl
    return moe_forward(layer.x, layer.ids if ids is None else ids, layer.w if w is None else w,
                       layer.planes, layer.luts, layer.q if q is None else q,
                       wl.H, wl.I, wl.E, tokens=tokens, cache=cache)
