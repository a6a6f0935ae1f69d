"""The boundary's contract: each of the four calls the hot path is specified
with (phase 1, the phase-2 merge, the one-shot Full site, the block sum) keeps
its specified arguments, in order, in include/attnres.h; every argument the
header adds is named here with the reason, so a change of the contract shows
up as a failing test.  Parses the header only (no library, no GPU)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")

# The specified argument lists (names as in the problem statement of the
# two-phase scheme: phase 1 returns outputs + max + log-sum-exp, phase 2
# merges one more source for later sublayers, the one-shot site, the block sum).
SPECIFIED = {
    "attnres_phase1": ["dt", "src", "n_src", "src_stride", "T", "d", "w", "key_gain", "S", "eps", "out",
                       "m_out", "lse_out", "stream"],
    "attnres_phase2_merge": ["dt", "T", "d", "p1_out", "p1_lse", "partial_in", "sublayer_prev", "partial_out",
                             "w", "key_gain", "prenorm_gain", "eps", "h_out", "x_out", "stream"],
    "attnres_full": ["dt", "src", "n_src", "src_stride", "T", "d", "w", "key_gain", "prenorm_gain", "eps",
                     "h_out", "x_out", "lse_out", "stream"],
    "attnres_block_accumulate": ["dt", "T", "d", "partial_in", "v", "out", "stream"],
    "attnres_status_string": ["status"],
}

# Arguments the header adds to a specified call, and why.
EXTENSIONS = {
    "attnres_phase1": {
        # fp32 sources with bf16 outputs: a training forward keeps the block
        # sums exact (they are what the backward differentiates)
        "src_dt": "dtype of the source rows (dt, or F32 with bf16 outputs)",
        # caller-owned memory for the packed queries and the softmax weights
        # between the scoring and output kernels (the library allocates nothing)
        "workspace": "scratch of attnres_phase1_workspace_bytes()",
        "workspace_bytes": "its size, checked before any launch",
    },
    "attnres_phase2_merge": {
        # the running partial sum is never bf16: Q16, P24 or fp32 (precision)
        "partial_dt": "format of partial_in (F32, P24, Q16 or a sublayer output's dtype)",
        # storing the partial only every second sublayer saves bytes
        "sublayer_prev2": "the output before the previous one, added first",
        "partial_out_dt": "format of partial_out (F32, P24 or Q16)",
    },
    "attnres_full": {},
    "attnres_block_accumulate": {
        "partial_dt": "format of partial_in (F32, P24, Q16 or dt)",
        "out_dt": "dtype of the block sum (dt, or F32: a training forward keeps it exact)",
        "v2": "the block's one-before-last output (partial stored every second sublayer)",
    },
    "attnres_status_string": {},
}


def header_params(name):
    text = open(HEADER).read()
    m = re.search(r"\b%s\s*\(([^;{]*)\)\s*;" % re.escape(name), text, re.S)
    assert m, "%s is not declared" % name
    params = []
    for arg in m.group(1).split(","):
        arg = re.sub(r"/\*.*?\*/", "", arg, flags=re.S).strip()
        params.append(re.findall(r"(\w+)\s*$", arg)[0])
    return params


def test_specified_calls_keep_their_arguments_in_order():
    for name, spec in SPECIFIED.items():
        params = header_params(name)
        ext = EXTENSIONS[name]
        for extra in ext:
            assert extra in params, "%s: documented extension %s is gone" % (name, extra)
        kept = [p for p in params if p not in ext]
        assert kept == spec, "%s: %s differs from the specified %s" % (name, kept, spec)


def test_stream_is_an_opaque_pointer():
    # hipStream_t is passed as void* so the header needs no HIP include
    text = open(HEADER).read()
    assert "#include <hip" not in text
    for name in SPECIFIED:
        if name != "attnres_status_string":
            m = re.search(r"\b%s\s*\(([^;{]*)\)\s*;" % name, text, re.S)
            assert re.search(r"void\s*\*\s*stream\s*$", m.group(1).strip()), name


def test_phase1_accumulate_is_phase1_plus_the_block_sum():
    # the fused call takes the phase-1 call's specified arguments and the
    # block sum's pieces (its `v` is the block's last output, sublayer_prev)
    params = header_params("attnres_phase1_accumulate")
    for a in SPECIFIED["attnres_phase1"]:
        assert a in params, a
    for a in ("partial_in", "sublayer_prev"):
        assert a in params, a
    pos = [params.index(a) for a in SPECIFIED["attnres_phase1"]]
    assert pos == sorted(pos), "the phase-1 arguments keep their order"
