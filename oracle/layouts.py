"""Accumulator-layout maps stated on the pages -- TEST INFRASTRUCTURE ONLY.

Each function maps an output element (i, j) of block b to the (lane, register)
that holds it after one matrix instruction, or back.  They are written from
the formulas on the pages and are pinned in the tests against the row-band
tables the same pages print:

* "CDNA dense MFMA builtins", section "Accumulator layout":
  - 32x32 layout (two blocks; one-block variants use block 0),
  - 16x16 layout (four blocks; one-block variants use block 0),
  - 4x4 layout (sixteen blocks).
* "CDNA3 sparse MFMA builtins", section "Accumulator layout": every sparse
  instruction has block count 1 and uses the one-block layout of the dense
  tile of the same M x N (16x16 and 32x32 subsections).

The GPU epilogue implements its own copy of the 32x32 one-block map; GEMM
parity on the GPU is what confirms that copy.
"""

WAVE = 64


def blocks_of(shape):
    """Block counts of the page's layouts: 32x32 -> 2, 16x16 -> 4, 4x4 -> 16."""
    return {32: 2, 16: 4, 4: 16}[shape]


def regs_per_lane(shape, blocks):
    """Registers per lane = blocks * M*N / wavefront size ("Accumulator layout")."""
    return blocks * shape * shape // WAVE


# ---- 32x32 ("CDNA dense MFMA builtins", 32x32 layout) -------------------------

def fwd_32x32(i, j, b=0):
    """(i, j, block) -> (lane, reg): lane = (32*floor(i/4)) mod 64 + j,
    reg = 16*b + 4*floor(i/8) + (i mod 4)."""
    lane = (32 * (i // 4)) % 64 + j
    reg = 16 * b + 4 * (i // 8) + (i % 4)
    return lane, reg


def inv_32x32(lane, reg):
    """(lane, reg) -> (i, j, block): i = (8*floor(G/4)) mod 32 + 4*floor(L/32) + (G mod 4),
    j = L mod 32, b = floor(G/16)."""
    i = (8 * (reg // 4)) % 32 + 4 * (lane // 32) + (reg % 4)
    j = lane % 32
    b = reg // 16
    return i, j, b


# ---- 16x16 ("CDNA dense MFMA builtins", 16x16 layout) -------------------------

def fwd_16x16(i, j, b=0):
    """lane = 16*floor(i/4) + j, reg = 4*b + (i mod 4)."""
    return 16 * (i // 4) + j, 4 * b + (i % 4)


def inv_16x16(lane, reg):
    """i = 4*floor(L/16) + (G mod 4), j = L mod 16, b = floor(G/4)."""
    return 4 * (lane // 16) + (reg % 4), lane % 16, reg // 4


# ---- 4x4 ("CDNA dense MFMA builtins", 4x4 layout) -----------------------------

def fwd_4x4(i, j, b=0):
    """lane = 4*b + j, reg = i."""
    return 4 * b + j, i


def inv_4x4(lane, reg):
    """i = G mod 4, j = L mod 4, b = floor(L/4)."""
    return reg % 4, lane % 4, lane // 4


# ---- sparse, one block ("CDNA3 sparse MFMA builtins", accumulator layout) ----

def fwd_sparse_32x32(i, j):
    """lane = (32*floor(i/4)) mod 64 + j, VGPR = 4*floor(i/8) + (i mod 4)."""
    return (32 * (i // 4)) % 64 + j, 4 * (i // 8) + (i % 4)


def inv_sparse_32x32(lane, reg):
    """i = (8*floor(G/4)) mod 32 + 4*floor(L/32) + (G mod 4), j = L mod 32."""
    return (8 * (reg // 4)) % 32 + 4 * (lane // 32) + (reg % 4), lane % 32


def fwd_sparse_16x16(i, j):
    """lane = 16*floor(i/4) + j, VGPR = i mod 4."""
    return 16 * (i // 4) + j, i % 4


def inv_sparse_16x16(lane, reg):
    """i = 4*floor(L/16) + (G mod 4), j = L mod 16."""
    return 4 * (lane // 16) + (reg % 4), lane % 16
