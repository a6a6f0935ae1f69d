"""The pages' analytic cost model of AttnRes: residual I/O per layer, extra
arithmetic, parameters, history memory and pipeline communication.

Pure arithmetic on sizes (no data), used by bench.py to put the measured
bytes per token and sublayer beside the pages' model.  Units: I/O in
elements per token (rows of d elements), arithmetic in FLOPs per token,
memory in bytes, pipeline communication in multiples of N_p d.

Sources, by function:
- "Attention Residuals" (structured notes on arXiv 2603.15031), section 10
  (inference system: the per-layer analytic I/O table) and section 9
  (training system: cached cross-stage blocks).
- "Attention Residuals 阅读补充", section "Full AttnRes" (arithmetic,
  static queries and two-phase computation, history memory, training) and
  section "Block AttnRes" (history memory, activation memory).
"""
from __future__ import annotations

# ---------------------------------------------------------------- I/O per layer
# Structured notes, section 10, analytic I/O table: elements read and written
# per token by the residual mechanism itself in one layer (the sublayer's own
# traffic excluded).


def io_standard_residual(d: int) -> float:
    """Plain residual: read the stream and the sublayer output, write the sum."""
    return 3.0 * d


def io_mhc(m: int, d: int) -> float:
    """mHC with expansion m: (8m + 2) rows of d plus 2m^2 + 4m scalars (the
    notes round the m = 4 value to 34d, dropping the scalars)."""
    return (8.0 * m + 2.0) * d + 2 * m * m + 4 * m


def io_full_two_phase(S: int, N: int, d: int) -> float:
    """Full AttnRes with the two-phase schedule over N groups of S layers:
    S + N rows per layer (the reading notes' static-query section writes it
    O((S + G) d) with G groups)."""
    return float(S + N) * d


def io_block_two_phase(N: int, S: float, d: int) -> float:
    """Block AttnRes with the two-phase schedule, N blocks of S sublayers:
    the completed blocks read once per block (N / S rows per sublayer) plus
    5 rows per sublayer for the merge (the notes give no breakdown of the 5)."""
    return (N / S + 5.0) * d


def batched_history_reads(S: int, R: int, d: int, b: int) -> tuple:
    """Reading notes, static queries: ideal K/V read bytes of R history rows
    for S queries, one read per query (2 S R d b) versus once per group
    (2 R d b)."""
    return 2 * S * R * d * b, 2 * R * d * b


# ---------------------------------------------------------------- arithmetic
# Reading notes, section "Full AttnRes", arithmetic.


def full_pairs(L: int) -> int:
    """Source-target pairs of Full AttnRes over L layers: layer l sees l
    earlier representations, 1 + 2 + ... + L."""
    return L * (L + 1) // 2


def full_forward_flops(L: int, d: int) -> int:
    """Extra forward FLOPs per token: 4d per pair (a dot product and a
    weighted accumulation, multiply and add counted separately)."""
    return 4 * d * full_pairs(L)


def full_train_flops(L: int, d: int) -> int:
    """Forward plus backward, about three times the forward."""
    return 3 * full_forward_flops(L, d)


def query_params(L: int, d: int) -> int:
    """Parameters added: one query vector and one RMSNorm gain per layer."""
    return 2 * L * d


# ---------------------------------------------------------------- memory (bytes)


def full_prefill_bytes(B: int, T: int, L: int, d: int, b: int = 2) -> int:
    """Reading notes, Full AttnRes history memory: all L + 1 representations
    of B x T tokens."""
    return b * B * T * (L + 1) * d


def depth_state_bytes(n_states: int, d: int, b: int = 2) -> int:
    """Decode: one token's depth states (its L + 1 representations for Full
    AttnRes), independent of the context length."""
    return n_states * d * b


def history_bytes(M: int, n_states: int, d: int, b: int = 2) -> int:
    """Training activation memory of the depth history for a microbatch of
    M tokens: Full keeps L + 1 states, Block keeps N block representations."""
    return M * n_states * d * b


def block_prefill_bytes(B: int, N: int, T: int, d: int, P: int = 1, b: int = 2) -> float:
    """Reading notes, Block AttnRes history memory: N block representations
    of B x T tokens, sharded over P devices along the sequence."""
    return b * B * N * T * d / P


# ---------------------------------------------------------------- pipeline (units of N_p d)
# Structured notes, section 9: interleaved pipeline with P physical stages of
# V virtual stages each (C = P V chunks), N_p block representations produced
# per physical stage on average.


def pp_comm_naive(P: int, V: int) -> float:
    """Every chunk boundary resends the whole history: C (C - 1) / 2."""
    C = P * V
    return C * (C - 1) / 2.0


def pp_comm_cached(P: int, V: int) -> float:
    """Each physical stage keeps the blocks it already received, so later
    virtual stages send only new ones: P (P - 1) / 2 + (V - 1) P^2 (the form
    whose worked example, P = 4 and V = 2, gives 22)."""
    return P * (P - 1) / 2.0 + (V - 1) * P * P


def model_for(L: int, N: int) -> dict:
    """The pages' per-layer I/O in rows of d at L sublayers in N blocks
    (Block: S = L / N sublayers per block; Full two-phase over the same N
    groups)."""
    S = L / N
    return {"standard_residual": io_standard_residual(1),
            "full_two_phase": io_full_two_phase(int(round(S)), N, 1),
            "block_two_phase": round(io_block_two_phase(N, S, 1), 3)}
